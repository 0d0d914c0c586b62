"""ctypes binding of liboscar.so: the C ABI of include/oscar.h with the same names.

Argument marshalling only: torch tensors supply device pointers and the current HIP stream;
every step of the computation runs in the library's kernels. There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
# OSCAR_LIB names another build of the same library (the host sanitizer build for CPU tests)
LIB_PATH = os.environ.get("OSCAR_LIB") or os.path.join(HERE, "liboscar.so")

OSCAR_OK = 0
STATUS = {0: "OSCAR_OK", -1: "OSCAR_ERR_INVALID_ARG", -2: "OSCAR_ERR_UNSUPPORTED", -3: "OSCAR_ERR_WORKSPACE",
          -4: "OSCAR_ERR_LAUNCH"}


class Layout(ctypes.Structure):
    """oscar_layout_t."""
    _fields_ = [("num_q_heads", c_int32), ("num_kv_heads", c_int32), ("head_dim", c_int32),
                ("group_size", c_int32), ("sink_len", c_int32), ("recent_len", c_int32),
                ("page_size", c_int32), ("mixed", c_int32), ("int4_page_offset", c_int64),
                ("pool_pages", c_int64), ("clip_k", c_float), ("clip_v", c_float),
                ("clip_k4", c_float), ("clip_v4", c_float), ("codebook", c_void_p)]


_P = c_void_p
_SIGS = {
    "oscar_status_string": (c_char_p, [c_int32]),
    "oscar_version": (c_char_p, []),
    "oscar_page_bytes": (c_size_t, [_P, c_int32]),
    "oscar_window_bytes": (c_size_t, [_P, c_int32]),
    "oscar_pool_bytes": (c_size_t, [_P]),
    "oscar_quantize_pack": (c_int32, [c_int64, c_int32, c_int32, c_int32, c_float, _P, _P, _P, _P]),
    "oscar_quantize_pack_codebook": (c_int32, [c_int64, c_int32, c_int32, c_float, _P, _P, _P, _P, _P]),
    "oscar_codebook_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "oscar_codebook_fit": (c_int32, [c_int32, c_int32, c_int32, _P, _P, c_float, c_int32, c_double, _P, c_size_t,
                                     _P, _P, _P, _P]),
    "oscar_kv_prefill": (c_int32, [_P, c_int32, c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_int32, _P, _P, _P]),
    "oscar_kv_demote": (c_int32, [_P, c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_int32, _P, _P, _P, _P]),
    "oscar_decode_workspace_bytes": (c_size_t, [_P, c_int32, c_int32]),
    "oscar_decode_attn": (c_int32, [_P, c_int32, c_int32, _P, _P, _P, _P, _P, _P, _P, c_int32, _P, _P, c_float,
                                    _P, c_size_t, _P, _P]),
    "oscar_decode_attn_profiled": (c_int32, [_P, c_int32, c_int32, _P, _P, _P, _P, _P, _P, _P, c_int32, _P, _P,
                                             c_float, _P, c_size_t, _P, _P, c_int32, _P]),
    "oscar_decode_step": (c_int32, [_P, c_int32, c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_int32, _P,
                                    _P, _P, c_float, _P, c_size_t, _P, _P]),
    "oscar_decode_step_profiled": (c_int32, [_P, c_int32, c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             c_int32, _P, _P, _P, c_float, _P, c_size_t, _P, _P, c_int32, _P]),
    "oscar_decode_step_noalloc": (c_int32, [_P, c_int32, c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            c_int32, _P, _P, _P, c_float, _P, _P]),
    "oscar_allocate_bits": (c_int32, [c_int32, _P, _P, _P, c_double, c_int32, _P, _P]),
    "oscar_route_tokens": (c_int32, [c_int32, c_int32, _P, _P, c_int32, _P, _P, _P]),
    "oscar_calib_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "oscar_calib_query_cov": (c_int32, [c_int32, c_int32, c_int32, c_int32, _P, _P, c_size_t, _P, _P]),
    "oscar_calib_value_cov": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, _P, _P, _P, c_float, _P,
                                        c_size_t, _P, _P]),
    "oscar_rotation_from_covariance": (c_int32, [c_int32, c_int32, _P, _P, _P, _P]),
    "oscar_bf16_fill": (c_int32, [_P, c_int32, c_int32, _P, _P, _P, _P, c_int64, _P, c_int32, _P]),
    "oscar_bf16_decode_workspace_bytes": (c_size_t, [_P, c_int32, c_int32]),
    "oscar_bf16_decode_attn": (c_int32, [_P, c_int32, c_int32, _P, _P, _P, c_int64, _P, c_int32, c_float, _P,
                                         c_size_t, _P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_rotated_kv_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_string(code: int) -> str:
    return lib().oscar_status_string(int(code)).decode()


def check(code: int, what: str):
    if code != OSCAR_OK:
        raise RuntimeError(f"{what} failed: {status_string(code)}")
