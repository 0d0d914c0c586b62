"""MI355X (gfx950) attention-aware INT2 KV caching: decode attention over a BF16 sink | rotated
INT2 history | BF16 recent cache, and the per-step demote, as hand-written HIP kernels behind
the C ABI of include/oscar.h. This package is the thin Python binding of that library.

Importing the package does not load the library; the first call does, and raises if it has
not been built (``python -m bit_rotated_kv_amd.build``). There is no fallback path.
"""
from ._lib import LIB_PATH, Layout, lib, status_string
from .ops import (make_layout, page_bytes, window_bytes, pool_bytes, decode_workspace_bytes,
                  bf16_decode_workspace_bytes, quantize_pack, quantize_pack_codebook, set_codebook, codebook_workspace_bytes,
                  codebook_fit, kv_prefill, kv_demote, decode_attn,
                  decode_step, decode_step_noalloc, bf16_fill, bf16_decode_attn, allocate_bits, route_tokens, calib_query_cov,
                  calib_value_cov, rotation_from_covariance)
from .cache import CacheBuffers, allocate_cache

__all__ = ["LIB_PATH", "Layout", "lib", "status_string", "make_layout", "page_bytes", "window_bytes",
           "pool_bytes", "decode_workspace_bytes", "bf16_decode_workspace_bytes", "quantize_pack",
           "quantize_pack_codebook", "set_codebook", "codebook_workspace_bytes", "codebook_fit", "kv_prefill", "kv_demote", "decode_attn", "decode_step", "decode_step_noalloc",
           "bf16_fill", "bf16_decode_attn", "allocate_bits", "route_tokens", "calib_query_cov", "calib_value_cov",
           "rotation_from_covariance", "CacheBuffers", "allocate_cache"]
