"""Torch-facing wrappers of the C ABI (include/oscar.h), one per entry point, same names.

Each wrapper checks dtypes/devices/shapes, passes device pointers and the current HIP stream,
and raises on a non-OK status. No arithmetic of the method happens here.
"""
from __future__ import annotations

from ctypes import c_void_p
from typing import Optional

import torch

from ._lib import Layout, check, lib

PAGE = 16


def make_layout(num_q_heads: int, num_kv_heads: int, head_dim: int, group_size: Optional[int] = None,
                sink_len: int = 64, recent_len: int = 256, mixed: bool = False, int4_page_offset: int = 0,
                pool_pages: int = 0, clip_k: float = 0.96, clip_v: float = 0.92, clip_k4: float = 1.0,
                clip_v4: float = 1.0, codebook: Optional[torch.Tensor] = None) -> Layout:
    """``codebook``: optional INT2 codebook table, a device int16 tensor [Hkv, 2, 4] of fp16 level
    patterns (K, then V); the layout keeps a reference to it."""
    lay = Layout(num_q_heads, num_kv_heads, head_dim, head_dim if group_size is None else group_size, sink_len,
                 recent_len, PAGE, 1 if mixed else 0, int4_page_offset, pool_pages, clip_k, clip_v, clip_k4,
                 clip_v4, None)
    set_codebook(lay, codebook)
    return lay


def set_codebook(layout: Layout, codebook: Optional[torch.Tensor]) -> None:
    """Point the layout at an INT2 codebook table [Hkv, 2, 4] int16 (fp16 patterns), or at none."""
    if codebook is not None:
        _need(codebook, torch.int16, "codebook")
        if tuple(codebook.shape) != (layout.num_kv_heads, 2, 4):
            raise ValueError(f"codebook must be [{layout.num_kv_heads}, 2, 4], got {tuple(codebook.shape)}")
    layout.codebook = None if codebook is None else codebook.data_ptr()
    layout._codebook_ref = codebook


def _p(t: Optional[torch.Tensor]):
    return None if t is None else c_void_p(t.data_ptr())


def _stream():
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: Optional[torch.Tensor], dtype, name: str, optional: bool = False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t: Optional[torch.Tensor], shape: tuple, name: str):
    """Exact shape check (the library cannot see buffer sizes: an undersized tensor would be an
    out-of-bounds device access)."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _bytes_at_least(t: Optional[torch.Tensor], n: int, name: str):
    if t is not None and t.numel() * t.element_size() < n:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, the layout needs {n}")


def _tables(batch: int, page_table: torch.Tensor, page_table4: Optional[torch.Tensor]) -> int:
    """[B, stride] page tables (INT2 and, for mixed caches, INT4 with the same stride)."""
    if page_table.dim() != 2 or page_table.shape[0] != batch:
        raise ValueError(f"page_table must be [{batch}, stride], got {tuple(page_table.shape)}")
    _shape(page_table4, tuple(page_table.shape), "page_table4")
    return page_table.shape[1]


def _rotations(layout: Layout, rot_k: torch.Tensor, rot_v: torch.Tensor):
    d = layout.head_dim
    _shape(rot_k, (layout.num_kv_heads, d, d), "rot_k")
    _shape(rot_v, (layout.num_kv_heads, d, d), "rot_v")


def _cache(layout: Layout, batch: int, pool: torch.Tensor, window: torch.Tensor):
    _bytes_at_least(pool, pool_bytes(layout), "pool")
    _bytes_at_least(window, window_bytes(layout, batch), "window")


def _ref(layout: Layout):
    import ctypes
    return ctypes.byref(layout)


# ---------------------------------------------------------------- sizes
def page_bytes(layout: Layout, bits: int) -> int:
    return int(lib().oscar_page_bytes(_ref(layout), bits))


def window_bytes(layout: Layout, batch: int) -> int:
    return int(lib().oscar_window_bytes(_ref(layout), batch))


def pool_bytes(layout: Layout) -> int:
    return int(lib().oscar_pool_bytes(_ref(layout)))


def decode_workspace_bytes(layout: Layout, batch: int, max_seq_len: int) -> int:
    return int(lib().oscar_decode_workspace_bytes(_ref(layout), batch, max_seq_len))


def bf16_decode_workspace_bytes(layout: Layout, batch: int, max_seq_len: int) -> int:
    return int(lib().oscar_bf16_decode_workspace_bytes(_ref(layout), batch, max_seq_len))


# ---------------------------------------------------------------- entry points
def quantize_pack(x: torch.Tensor, group: int, bits: int, clip: float, codes: Optional[torch.Tensor] = None,
                  scale_zero: Optional[torch.Tensor] = None):
    """x [rows, dim] fp32 -> (codes uint8 [rows, dim*bits/8], scale_zero int16 [rows, dim/group, 2] bf16 bits)."""
    _need(x, torch.float32, "x")
    rows, dim = x.shape
    if codes is None:
        codes = torch.empty((rows, dim * bits // 8), dtype=torch.uint8, device=x.device)
    if scale_zero is None:
        scale_zero = torch.empty((rows, dim // group, 2), dtype=torch.int16, device=x.device)
    _need(codes, torch.uint8, "codes")
    _need(scale_zero, torch.int16, "scale_zero")
    if group <= 0 or dim % group or bits not in (2, 4):
        raise ValueError("group must divide dim and bits must be 2 or 4")
    _shape(codes, (rows, dim * bits // 8), "codes")
    _shape(scale_zero, (rows, dim // group, 2), "scale_zero")
    check(lib().oscar_quantize_pack(rows, dim, group, bits, clip, _p(x), _p(codes), _p(scale_zero), _stream()),
          "oscar_quantize_pack")
    return codes, scale_zero


def quantize_pack_codebook(x: torch.Tensor, group: int, clip: float, levels, codes: Optional[torch.Tensor] = None,
                           scale_zero: Optional[torch.Tensor] = None):
    """INT2 codes under a codebook: x [rows, dim] fp32, levels four fp16 patterns (host ints)."""
    import ctypes
    _need(x, torch.float32, "x")
    rows, dim = x.shape
    lv = (ctypes.c_uint16 * 4)(*[int(v) & 0xFFFF for v in levels])
    if codes is None:
        codes = torch.empty((rows, dim // 4), dtype=torch.uint8, device=x.device)
    if scale_zero is None:
        scale_zero = torch.empty((rows, dim // group, 2), dtype=torch.int16, device=x.device)
    _need(codes, torch.uint8, "codes")
    _need(scale_zero, torch.int16, "scale_zero")
    if group <= 0 or dim % group:
        raise ValueError("group must divide dim")
    _shape(codes, (rows, dim // 4), "codes")
    _shape(scale_zero, (rows, dim // group, 2), "scale_zero")
    check(lib().oscar_quantize_pack_codebook(rows, dim, group, clip, _p(x), ctypes.cast(lv, c_void_p), _p(codes),
                                             _p(scale_zero), _stream()), "oscar_quantize_pack_codebook")
    return codes, scale_zero


def codebook_workspace_bytes(num_kv_heads: int, n_rows: int, head_dim: int) -> int:
    return int(lib().oscar_codebook_workspace_bytes(num_kv_heads, n_rows, head_dim))


def codebook_fit(x: torch.Tensor, rot: torch.Tensor, clip: float, max_iter: int = 100, tol: float = 1e-7,
                 workspace: Optional[torch.Tensor] = None):
    """Lloyd-Max INT2 codebooks of calibration rows x [Hkv, n, d] bf16 under rotations rot [Hkv, d, d]
    fp32. Returns (levels float64 [Hkv, 4], fp16 patterns int16 [Hkv, 4], iterations int32 [Hkv])."""
    import ctypes
    import numpy as np
    _need(x, torch.bfloat16, "x")
    _need(rot, torch.float32, "rot")
    hkv, n, d = x.shape
    _shape(rot, (hkv, d, d), "rot")
    if workspace is None:
        workspace = torch.empty(max(codebook_workspace_bytes(hkv, n, d), 1), dtype=torch.uint8, device=x.device)
    _need(workspace, torch.uint8, "workspace")
    levels = np.zeros((hkv, 4), np.float64)
    pats = np.zeros((hkv, 4), np.uint16)
    iters = np.zeros(hkv, np.int32)
    check(lib().oscar_codebook_fit(hkv, n, d, _p(x), _p(rot), clip, max_iter, tol, _p(workspace),
                                   workspace.numel(), levels.ctypes.data_as(c_void_p), pats.ctypes.data_as(c_void_p),
                                   iters.ctypes.data_as(c_void_p), _stream()), "oscar_codebook_fit")
    return levels, pats.view(np.int16), iters


def kv_prefill(layout: Layout, seq_len: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rot_k: torch.Tensor,
               rot_v: torch.Tensor, pool: torch.Tensor, page_table: torch.Tensor, window: torch.Tensor,
               token_bits: Optional[torch.Tensor] = None, page_table4: Optional[torch.Tensor] = None,
               n_int4_out: Optional[torch.Tensor] = None):
    """k, v [B, Hkv, max_seq_len, d] bf16; seq_len [B] int32; page tables [B, stride] int32."""
    _need(seq_len, torch.int32, "seq_len")
    _need(k, torch.bfloat16, "k")
    _need(v, torch.bfloat16, "v")
    _need(rot_k, torch.float32, "rot_k")
    _need(rot_v, torch.float32, "rot_v")
    _need(pool, torch.uint8, "pool")
    _need(page_table, torch.int32, "page_table")
    _need(window, torch.uint8, "window")
    _need(token_bits, torch.uint8, "token_bits", optional=True)
    _need(page_table4, torch.int32, "page_table4", optional=True)
    _need(n_int4_out, torch.int32, "n_int4_out", optional=True)
    if k.dim() != 4:
        raise ValueError("k must be [B, Hkv, max_seq_len, d]")
    B, hkv, tmax, d = k.shape
    _shape(k, (B, layout.num_kv_heads, tmax, layout.head_dim), "k")
    _shape(v, tuple(k.shape), "v")
    _shape(seq_len, (B,), "seq_len")
    _shape(token_bits, (B, tmax), "token_bits")
    _shape(n_int4_out, (B,), "n_int4_out")
    _rotations(layout, rot_k, rot_v)
    _cache(layout, B, pool, window)
    stride = _tables(B, page_table, page_table4)
    check(lib().oscar_kv_prefill(_ref(layout), B, tmax, _p(seq_len), _p(k), _p(v), _p(token_bits), _p(rot_k),
                                 _p(rot_v), _p(pool), _p(page_table), _p(page_table4), stride,
                                 _p(window), _p(n_int4_out), _stream()), "oscar_kv_prefill")


def kv_demote(layout: Layout, seq_len: torch.Tensor, new_k: torch.Tensor, new_v: torch.Tensor, rot_k: torch.Tensor,
              rot_v: torch.Tensor, pool: torch.Tensor, page_table: torch.Tensor, window: torch.Tensor,
              n_int4: Optional[torch.Tensor] = None, demote_bits: Optional[torch.Tensor] = None,
              page_table4: Optional[torch.Tensor] = None, seq_len_out: Optional[torch.Tensor] = None,
              n_int4_out: Optional[torch.Tensor] = None):
    """One step's cache update. new_k, new_v [B, Hkv, d] bf16."""
    _need(seq_len, torch.int32, "seq_len")
    _need(new_k, torch.bfloat16, "new_k")
    _need(new_v, torch.bfloat16, "new_v")
    _need(rot_k, torch.float32, "rot_k")
    _need(rot_v, torch.float32, "rot_v")
    _need(pool, torch.uint8, "pool")
    _need(page_table, torch.int32, "page_table")
    _need(window, torch.uint8, "window")
    for t, n in ((n_int4, "n_int4"), (page_table4, "page_table4"), (seq_len_out, "seq_len_out"),
                 (n_int4_out, "n_int4_out")):
        _need(t, torch.int32, n, optional=True)
    _need(demote_bits, torch.uint8, "demote_bits", optional=True)
    B = new_k.shape[0]
    _shape(new_k, (B, layout.num_kv_heads, layout.head_dim), "new_k")
    _shape(new_v, tuple(new_k.shape), "new_v")
    for t, n in ((seq_len, "seq_len"), (n_int4, "n_int4"), (seq_len_out, "seq_len_out"), (n_int4_out, "n_int4_out"),
                 (demote_bits, "demote_bits")):
        _shape(t, (B,), n)
    _rotations(layout, rot_k, rot_v)
    _cache(layout, B, pool, window)
    stride = _tables(B, page_table, page_table4)
    check(lib().oscar_kv_demote(_ref(layout), B, _p(seq_len), _p(n_int4), _p(new_k), _p(new_v), _p(demote_bits),
                                _p(rot_k), _p(rot_v), _p(pool), _p(page_table), _p(page_table4), stride,
                                _p(window), _p(seq_len_out), _p(n_int4_out), _stream()), "oscar_kv_demote")


def decode_attn(layout: Layout, q: torch.Tensor, seq_len: torch.Tensor, window: torch.Tensor, pool: torch.Tensor,
                page_table: torch.Tensor, rot_k: torch.Tensor, rot_v: torch.Tensor, workspace: torch.Tensor,
                max_seq_len: int, out: Optional[torch.Tensor] = None, n_int4: Optional[torch.Tensor] = None,
                page_table4: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                events: Optional[list] = None) -> torch.Tensor:
    """q [B, Hq, d] bf16 -> out [B, Hq, d] fp32. With ``events`` (4 torch.cuda.Event), calls the
    timing variant, which records them around the kernels of the call (split, merge)."""
    _need(q, torch.bfloat16, "q")
    _need(seq_len, torch.int32, "seq_len")
    _need(window, torch.uint8, "window")
    _need(pool, torch.uint8, "pool")
    _need(page_table, torch.int32, "page_table")
    _need(rot_k, torch.float32, "rot_k")
    _need(rot_v, torch.float32, "rot_v")
    _need(workspace, torch.uint8, "workspace")
    _need(n_int4, torch.int32, "n_int4", optional=True)
    _need(page_table4, torch.int32, "page_table4", optional=True)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    B = q.shape[0]
    _shape(q, (B, layout.num_q_heads, layout.head_dim), "q")
    _shape(out, tuple(q.shape), "out")
    _shape(seq_len, (B,), "seq_len")
    _shape(n_int4, (B,), "n_int4")
    _rotations(layout, rot_k, rot_v)
    _cache(layout, B, pool, window)
    stride = _tables(B, page_table, page_table4)
    if events is None:
        check(lib().oscar_decode_attn(_ref(layout), B, max_seq_len, _p(q), _p(seq_len), _p(n_int4), _p(window),
                                      _p(pool), _p(page_table), _p(page_table4), stride, _p(rot_k),
                                      _p(rot_v), softmax_scale, _p(workspace), workspace.numel(), _p(out), _stream()),
              "oscar_decode_attn")
        return out
    import ctypes
    arr = (c_void_p * len(events))(*[c_void_p(e.cuda_event) for e in events])
    check(lib().oscar_decode_attn_profiled(_ref(layout), B, max_seq_len, _p(q), _p(seq_len), _p(n_int4), _p(window),
                                           _p(pool), _p(page_table), _p(page_table4), stride,
                                           _p(rot_k), _p(rot_v), softmax_scale, _p(workspace), workspace.numel(),
                                           _p(out), ctypes.cast(arr, c_void_p), len(events), _stream()),
          "oscar_decode_attn_profiled")
    return out


def _step_args(layout, seq_len, new_k, new_v, q, rot_k, rot_v, pool, page_table, window, seq_len_out, max_seq_len,
               out, n_int4, n_int4_out, demote_bits, page_table4, softmax_scale):
    """Checks the arguments of a decode step and returns (out, the C arguments before the workspace)."""
    _need(seq_len, torch.int32, "seq_len")
    _need(new_k, torch.bfloat16, "new_k")
    _need(new_v, torch.bfloat16, "new_v")
    _need(q, torch.bfloat16, "q")
    _need(rot_k, torch.float32, "rot_k")
    _need(rot_v, torch.float32, "rot_v")
    _need(pool, torch.uint8, "pool")
    _need(page_table, torch.int32, "page_table")
    _need(window, torch.uint8, "window")
    _need(seq_len_out, torch.int32, "seq_len_out")
    for t, n in ((n_int4, "n_int4"), (n_int4_out, "n_int4_out"), (page_table4, "page_table4")):
        _need(t, torch.int32, n, optional=True)
    _need(demote_bits, torch.uint8, "demote_bits", optional=True)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    B = q.shape[0]
    _shape(q, (B, layout.num_q_heads, layout.head_dim), "q")
    _shape(out, tuple(q.shape), "out")
    _shape(new_k, (B, layout.num_kv_heads, layout.head_dim), "new_k")
    _shape(new_v, tuple(new_k.shape), "new_v")
    for t, n in ((seq_len, "seq_len"), (n_int4, "n_int4"), (seq_len_out, "seq_len_out"), (n_int4_out, "n_int4_out"),
                 (demote_bits, "demote_bits")):
        _shape(t, (B,), n)
    _rotations(layout, rot_k, rot_v)
    _cache(layout, B, pool, window)
    _tables(B, page_table, page_table4)
    args = (_ref(layout), q.shape[0], max_seq_len, _p(seq_len), _p(n_int4), _p(new_k), _p(new_v), _p(demote_bits),
            _p(q), _p(rot_k), _p(rot_v), _p(pool), _p(page_table), _p(page_table4), page_table.shape[1], _p(window),
            _p(seq_len_out), _p(n_int4_out), softmax_scale)
    return out, args


def decode_step(layout: Layout, seq_len: torch.Tensor, new_k: torch.Tensor, new_v: torch.Tensor, q: torch.Tensor,
                rot_k: torch.Tensor, rot_v: torch.Tensor, pool: torch.Tensor, page_table: torch.Tensor,
                window: torch.Tensor, seq_len_out: torch.Tensor, workspace: torch.Tensor, max_seq_len: int,
                out: Optional[torch.Tensor] = None, n_int4: Optional[torch.Tensor] = None,
                n_int4_out: Optional[torch.Tensor] = None, demote_bits: Optional[torch.Tensor] = None,
                page_table4: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                events: Optional[list] = None) -> torch.Tensor:
    """kv_demote's cache update and decode_attn over the updated cache, in one call (split and
    merge kernels). With ``events`` (4 torch.cuda.Event), calls the timing variant."""
    _need(workspace, torch.uint8, "workspace")
    out, args = _step_args(layout, seq_len, new_k, new_v, q, rot_k, rot_v, pool, page_table, window, seq_len_out,
                           max_seq_len, out, n_int4, n_int4_out, demote_bits, page_table4, softmax_scale)
    args = args + (_p(workspace), workspace.numel(), _p(out))
    if events is None:
        check(lib().oscar_decode_step(*args, _stream()), "oscar_decode_step")
        return out
    import ctypes
    arr = (c_void_p * len(events))(*[c_void_p(e.cuda_event) for e in events])
    check(lib().oscar_decode_step_profiled(*args, ctypes.cast(arr, c_void_p), len(events), _stream()),
          "oscar_decode_step_profiled")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_step_noalloc(layout: Layout, seq_len: torch.Tensor, new_k: torch.Tensor, new_v: torch.Tensor,
                        q: torch.Tensor, rot_k: torch.Tensor, rot_v: torch.Tensor, pool: torch.Tensor,
                        page_table: torch.Tensor, window: torch.Tensor, seq_len_out: torch.Tensor, max_seq_len: int,
                        out: torch.Tensor, n_int4: Optional[torch.Tensor] = None,
                        n_int4_out: Optional[torch.Tensor] = None, demote_bits: Optional[torch.Tensor] = None,
                        page_table4: Optional[torch.Tensor] = None, softmax_scale: float = 0.0) -> torch.Tensor:
    """decode_step without a workspace argument: the library's own per-device array of
    NOALLOC_SCRATCH_BYTES serves as the workspace, and the call allocates nothing (``out`` is
    required). Calls that overlap in time on one device race."""
    out, args = _step_args(layout, seq_len, new_k, new_v, q, rot_k, rot_v, pool, page_table, window, seq_len_out,
                           max_seq_len, out, n_int4, n_int4_out, demote_bits, page_table4, softmax_scale)
    check(lib().oscar_decode_step_noalloc(*args, _p(out), _stream()), "oscar_decode_step_noalloc")
    return out

def bf16_fill(layout: Layout, seq_len: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pages: torch.Tensor,
              num_pages: int, page_table: torch.Tensor):
    _need(seq_len, torch.int32, "seq_len")
    _need(k, torch.bfloat16, "k")
    _need(v, torch.bfloat16, "v")
    _need(pages, torch.uint8, "pages")
    _need(page_table, torch.int32, "page_table")
    if k.dim() != 4:
        raise ValueError("k must be [B, Hkv, max_seq_len, d]")
    B, hkv, tmax, d = k.shape
    _shape(k, (B, layout.num_kv_heads, tmax, layout.head_dim), "k")
    _shape(v, tuple(k.shape), "v")
    _shape(seq_len, (B,), "seq_len")
    _bytes_at_least(pages, num_pages * page_bytes(layout, 16), "pages")
    _tables(B, page_table, None)
    check(lib().oscar_bf16_fill(_ref(layout), B, tmax, _p(seq_len), _p(k), _p(v), _p(pages), num_pages,
                                _p(page_table), page_table.shape[1], _stream()), "oscar_bf16_fill")


def bf16_decode_attn(layout: Layout, q: torch.Tensor, seq_len: torch.Tensor, pages: torch.Tensor, num_pages: int,
                     page_table: torch.Tensor, workspace: torch.Tensor, max_seq_len: int,
                     out: Optional[torch.Tensor] = None, softmax_scale: float = 0.0) -> torch.Tensor:
    _need(q, torch.bfloat16, "q")
    _need(seq_len, torch.int32, "seq_len")
    _need(pages, torch.uint8, "pages")
    _need(page_table, torch.int32, "page_table")
    _need(workspace, torch.uint8, "workspace")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    B = q.shape[0]
    _shape(q, (B, layout.num_q_heads, layout.head_dim), "q")
    _shape(out, tuple(q.shape), "out")
    _shape(seq_len, (B,), "seq_len")
    _bytes_at_least(pages, num_pages * page_bytes(layout, 16), "pages")
    _tables(B, page_table, None)
    check(lib().oscar_bf16_decode_attn(_ref(layout), q.shape[0], max_seq_len, _p(q), _p(seq_len), _p(pages),
                                       num_pages, _p(page_table), page_table.shape[1], softmax_scale, _p(workspace),
                                       workspace.numel(), _p(out), _stream()), "oscar_bf16_decode_attn")
    return out


ALLOC_METHODS = {"greedy": 0, "exhaustive": 1}


def allocate_bits(d2, d4, counts, budget_bits: float, method: str = "greedy"):
    """INT2/INT4 width per tag class (host call): returns (bits uint8 [n], total distortion)."""
    import ctypes

    import numpy as np
    d2 = np.ascontiguousarray(d2, np.float64)
    d4 = np.ascontiguousarray(d4, np.float64)
    counts = np.ascontiguousarray(counts, np.int64)
    n = len(d2)
    if len(d4) != n or len(counts) != n:
        raise ValueError("d2, d4 and counts must have one entry per class")
    if method not in ALLOC_METHODS:
        raise ValueError(f"method must be one of {sorted(ALLOC_METHODS)}")
    bits = np.zeros(n, np.uint8)
    cost = ctypes.c_double(0.0)
    check(lib().oscar_allocate_bits(n, d2.ctypes.data, d4.ctypes.data, counts.ctypes.data, float(budget_bits),
                                    ALLOC_METHODS[method], bits.ctypes.data, ctypes.byref(cost)),
          "oscar_allocate_bits")
    return bits, cost.value


def route_tokens(seq_len: torch.Tensor, tags: torch.Tensor, class_bits, token_bits: Optional[torch.Tensor] = None
                 ) -> torch.Tensor:
    """tags [B, max_seq_len] int32 (device) -> token widths [B, max_seq_len] uint8 (positions below
    seq_len[b] written; a fresh output starts at 2 bits)."""
    import numpy as np
    _need(seq_len, torch.int32, "seq_len")
    _need(tags, torch.int32, "tags")
    cb = np.ascontiguousarray(class_bits, np.uint8)
    if token_bits is None:
        token_bits = torch.full(tags.shape, 2, dtype=torch.uint8, device=tags.device)
    _need(token_bits, torch.uint8, "token_bits")
    if token_bits.shape != tags.shape or tags.dim() != 2 or seq_len.shape[0] != tags.shape[0]:
        raise ValueError("tags and token_bits must be [B, max_seq_len] with B = len(seq_len)")
    check(lib().oscar_route_tokens(tags.shape[0], tags.shape[1], _p(seq_len), _p(tags), len(cb),
                                   c_void_p(cb.ctypes.data) if len(cb) else None, _p(token_bits), _stream()),
          "oscar_route_tokens")
    return token_bits


def calib_query_cov(q: torch.Tensor) -> torch.Tensor:
    """q [Hkv, gq, N, d] bf16 (calibration queries) -> C_Q [Hkv, d, d] fp32 on the GPU."""
    _need(q, torch.bfloat16, "q")
    if q.dim() != 4:
        raise ValueError("q must be [Hkv, gq, N, d]")
    hkv, gq, n, d = q.shape
    ws = torch.empty(lib().oscar_calib_workspace_bytes(hkv, gq, n, d), dtype=torch.uint8, device=q.device)
    cov = torch.empty((hkv, d, d), dtype=torch.float32, device=q.device)
    check(lib().oscar_calib_query_cov(hkv, gq, n, d, _p(q), _p(ws), ws.numel(), _p(cov), _stream()),
          "oscar_calib_query_cov")
    return cov


def calib_value_cov(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, softmax_scale: float = 0.0) -> torch.Tensor:
    """q [Hkv, gq, N, d], k, v [Hkv, n, d] bf16 -> C_S [Hkv, d, d] fp32 on the GPU."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, name)
    if q.dim() != 4 or k.dim() != 3 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[3]:
        raise ValueError("q must be [Hkv, gq, N, d] and k, v [Hkv, n, d]")
    hkv, gq, n, d = q.shape
    ws = torch.empty(lib().oscar_calib_workspace_bytes(hkv, gq, n, d), dtype=torch.uint8, device=q.device)
    cov = torch.empty((hkv, d, d), dtype=torch.float32, device=q.device)
    check(lib().oscar_calib_value_cov(hkv, gq, n, k.shape[1], d, _p(q), _p(k), _p(v), softmax_scale, _p(ws),
                                      ws.numel(), _p(cov), _stream()), "oscar_calib_value_cov")
    return cov


def rotation_from_covariance(cov, return_eig: bool = False):
    """R = U . H . P_br (fp32 numpy [n, d, d]) from symmetric covariances ``cov`` [n, d, d] or
    [d, d] (any array-like; passed to the host call as fp64). With ``return_eig`` also returns the
    descending eigenvalues [n, d] and eigenvectors U [n, d, d] (columns) the call formed."""
    import numpy as np
    c = np.ascontiguousarray(np.asarray(cov, dtype=np.float64))
    single = c.ndim == 2
    if single:
        c = c[None]
    if c.ndim != 3 or c.shape[1] != c.shape[2]:
        raise ValueError("cov must be [n, d, d] or [d, d]")
    n, d, _ = c.shape
    rot = np.zeros((n, d, d), np.float32)
    w = np.zeros((n, d), np.float64)
    u = np.zeros((n, d, d), np.float64)
    check(lib().oscar_rotation_from_covariance(n, d, c.ctypes.data, rot.ctypes.data, w.ctypes.data, u.ctypes.data),
          "oscar_rotation_from_covariance")
    if single:
        rot, w, u = rot[0], w[0], u[0]
    return (rot, w, u) if return_eig else rot
