"""The C-ABI library loads, exports every function include/oscar.h declares, and validates its
arguments on the host (no device work: every call here returns before any launch)."""
import ctypes
import os
import re

import pytest

import bit_rotated_kv_amd as brk
from bit_rotated_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from bit_rotated_kv_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("oscar_kv_demote", "oscar_decode_attn", "oscar_quantize_pack", "oscar_kv_prefill",
              "oscar_bf16_decode_attn", "oscar_decode_workspace_bytes", "oscar_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(raw, n), n
    assert set(declared_functions()) <= set(_lib._SIGS)


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert brk.status_string(code) == name
    assert brk.status_string(7) == "OSCAR_ERR_UNKNOWN"
    assert b"gfx950" in lib.oscar_version()


def test_layout_struct_size():
    assert ctypes.sizeof(_lib.Layout) == 72
    assert _lib.Layout.codebook.offset == 64


def layout(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, pool_pages=100)
    base.update(kw)
    return brk.make_layout(**base)


def test_sizes(lib):
    L = layout()
    assert brk.page_bytes(L, 2) == 8 * 1152
    assert brk.page_bytes(L, 4) == 8 * 2176
    assert brk.page_bytes(L, 16) == 8 * 8192
    assert brk.window_bytes(L, 3) == 3 * 8 * 20 * 8192
    assert brk.pool_bytes(L) == 100 * 8 * 1152
    M = layout(mixed=True, int4_page_offset=60)
    assert brk.pool_bytes(M) == 60 * 8 * 1152 + 40 * 8 * 2176
    assert brk.page_bytes(layout(head_dim=64, num_q_heads=2, num_kv_heads=1), 2) == 640
    # the workspace holds a partial per work unit (a bounded number per kv-head, at least one per
    # request) whatever the context; it is 0 for invalid layouts
    assert brk.decode_workspace_bytes(L, 1, 100_000) == brk.decode_workspace_bytes(L, 1, 1000) > 0
    assert brk.decode_workspace_bytes(L, 300, 1000) > brk.decode_workspace_bytes(L, 32, 1000)
    assert brk.decode_workspace_bytes(layout(head_dim=96), 1, 1000) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), -2), (dict(num_q_heads=24, num_kv_heads=8), -2), (dict(num_q_heads=30), -1),
    (dict(group_size=64), -2), (dict(group_size=48), -1), (dict(clip_k=0.0), -1), (dict(clip_v=1.5), -1),
    (dict(sink_len=72), -2), (dict(recent_len=0), -1), (dict(mixed=1, int4_page_offset=200), -1),
    (dict(num_q_heads=64, num_kv_heads=4), -2),
])
def test_invalid_layouts_rejected(lib, kw, code):
    L = layout(**kw)
    r = lib.oscar_decode_attn(ctypes.byref(L), 1, 1000, 1, 1, None, 1, 1, 1, None, 100, 1, 1, 0.0, 1, 1 << 30, 1,
                              None)
    assert r == code
    r = lib.oscar_kv_demote(ctypes.byref(L), 1, 1, None, 1, 1, None, 1, 1, 1, 1, None, 100, 1, None, None, None)
    assert r == code


def test_decode_argument_checks(lib):
    L = ctypes.byref(layout())
    ok_ptr = 1
    # null q
    assert lib.oscar_decode_attn(L, 1, 1000, None, ok_ptr, None, ok_ptr, ok_ptr, ok_ptr, None, 100, ok_ptr, ok_ptr,
                                 0.0, ok_ptr, 1 << 30, ok_ptr, None) == -1
    # empty page table although the length bound has a history
    assert lib.oscar_decode_attn(L, 1, 100_000, ok_ptr, ok_ptr, None, ok_ptr, ok_ptr, ok_ptr, None, 0, ok_ptr,
                                 ok_ptr, 0.0, ok_ptr, 1 << 30, ok_ptr, None) == -1
    # workspace too small
    assert lib.oscar_decode_attn(L, 1, 1000, ok_ptr, ok_ptr, None, ok_ptr, ok_ptr, ok_ptr, None, 100, ok_ptr, ok_ptr,
                                 0.0, ok_ptr, 16, ok_ptr, None) == -3
    # negative softmax scale
    assert lib.oscar_decode_attn(L, 1, 1000, ok_ptr, ok_ptr, None, ok_ptr, ok_ptr, ok_ptr, None, 100, ok_ptr, ok_ptr,
                                 -1.0, ok_ptr, 1 << 30, ok_ptr, None) == -1
    # batch 0 is a no-op
    assert lib.oscar_decode_attn(L, 0, 1000, None, None, None, None, None, None, None, 0, None, None, 0.0, None, 0,
                                 None, None) == 0
    # mixed cache without INT4 page table
    M = ctypes.byref(layout(mixed=True, int4_page_offset=50))
    assert lib.oscar_decode_attn(M, 1, 1000, ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, None, 100, ok_ptr,
                                 ok_ptr, 0.0, ok_ptr, 1 << 30, ok_ptr, None) == -1


def test_demote_argument_checks(lib):
    L = ctypes.byref(layout())
    p = 1
    # aliasing seq_len and seq_len_out
    assert lib.oscar_kv_demote(L, 2, 5, None, p, p, None, p, p, p, p, None, 10, p, 5, None, None) == -1
    assert lib.oscar_kv_demote(L, 2, None, None, p, p, None, p, p, p, p, None, 10, p, None, None, None) == -1


def test_step_argument_checks(lib):
    L = ctypes.byref(layout())
    p = 1
    st = lib.oscar_decode_step
    # (layout, batch, max_seq_len, seq_len, n_int4, new_k, new_v, demote_bits, q, rot_k, rot_v, pool,
    #  page_table, page_table4, pt_stride, window, seq_len_out, n_int4_out, scale, ws, ws_bytes, out, stream)
    assert st(L, 1, 1000, p, None, p, p, None, p, p, p, p, p, None, 100, p, None, None, 0.0, p, 1 << 30, p, None) == -1
    assert st(L, 1, 1000, 5, None, p, p, None, p, p, p, p, p, None, 100, p, 5, None, 0.0, p, 1 << 30, p, None) == -1
    assert st(L, 1, 1000, p, None, p, p, None, None, p, p, p, p, None, 100, p, 2, None, 0.0, p, 1 << 30, p, None) == -1
    assert st(L, 1, 1000, p, None, p, p, None, p, p, p, p, p, None, 100, p, 2, None, 0.0, p, 16, p, None) == -3
    M = ctypes.byref(layout(mixed=True, int4_page_offset=50))
    assert st(M, 1, 1000, p, p, p, p, None, p, p, p, p, p, p, 100, p, 2, None, 0.0, p, 1 << 30, p, None) == -1
    assert st(L, 0, 1000, None, None, None, None, None, None, None, None, None, None, None, 100, None, 2, None, 0.0,
              None, 0, None, None) == 0


def test_noalloc_step_limits(lib):
    """The no-allocation step accepts exactly the calls whose workspace bound fits its per-device
    array (checked before any device work) and follows the step's argument checks."""
    m = re.search(r"#define OSCAR_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == brk.ops.NOALLOC_SCRATCH_BYTES
    lay = layout()
    assert brk.decode_workspace_bytes(lay, 256, 1 << 20) <= brk.ops.NOALLOC_SCRATCH_BYTES
    big = next(b for b in range(256, 1 << 16, 64)
               if brk.decode_workspace_bytes(lay, b, 1000) > brk.ops.NOALLOC_SCRATCH_BYTES)
    L = ctypes.byref(lay)
    p = 1
    st = lib.oscar_decode_step_noalloc
    # (layout, batch, max_seq_len, seq_len, n_int4, new_k, new_v, demote_bits, q, rot_k, rot_v, pool,
    #  page_table, page_table4, pt_stride, window, seq_len_out, n_int4_out, scale, out, stream)
    assert st(L, big, 1000, p, None, p, p, None, p, p, p, p, p, None, 100, p, 2, None, 0.0, p, None) == -3
    assert st(L, -1, 1000, p, None, p, p, None, p, p, p, p, p, None, 100, p, 2, None, 0.0, p, None) == -1
    assert st(L, 0, 1000, None, None, None, None, None, None, None, None, None, None, None, 100, None, 2, None, 0.0,
              None, None) == 0


def test_profiled_argument_checks(lib):
    """The timing variants need 4 caller-created events; nothing is enqueued otherwise."""
    L = ctypes.byref(layout())
    p = 1
    ev3 = (ctypes.c_void_p * 3)(1, 1, 1)
    ev4null = (ctypes.c_void_p * 4)(1, 1, None, 1)
    da = lib.oscar_decode_attn_profiled
    for evs, n in ((None, 4), (ctypes.cast(ev3, ctypes.c_void_p), 3), (ctypes.cast(ev4null, ctypes.c_void_p), 4)):
        assert da(L, 1, 1000, p, p, None, p, p, p, None, 100, p, p, 0.0, p, 1 << 30, p, evs, n, None) == -1
        assert lib.oscar_decode_step_profiled(L, 1, 1000, p, None, p, p, None, p, p, p, p, p, None, 100, p, 2, None,
                                              0.0, p, 1 << 30, p, evs, n, None) == -1


def test_step_workspace_covers_plain_decode(lib):
    """One workspace size serves both the plain decode and the fused step (which adds a window
    workgroup and a history slot per (request, kv-head))."""
    for b, t in ((1, 100_000), (32, 32_768), (3, 321), (2, 64)):
        assert brk.decode_workspace_bytes(layout(), b, t) > 0


def test_quantize_pack_argument_checks(lib):
    q = lib.oscar_quantize_pack
    assert q(-1, 128, 128, 2, 0.96, 1, 1, 1, None) == -1
    assert q(4, 128, 48, 2, 0.96, 1, 1, 1, None) == -1      # group does not divide dim
    assert q(4, 128, 128, 3, 0.96, 1, 1, 1, None) == -1     # bits
    assert q(4, 6, 6, 2, 0.96, 1, 1, 1, None) == -1         # group not a multiple of codes per byte
    assert q(4, 128, 128, 2, 0.0, 1, 1, 1, None) == -1      # clip
    assert q(4, 2048, 128, 2, 0.96, 1, 1, 1, None) == -2    # dim beyond this build
    assert q(4, 128, 128, 2, 0.96, None, 1, 1, None) == -1  # null x
    assert q(0, 128, 128, 2, 0.96, None, None, None, None) == 0


def test_quantize_pack_codebook_argument_checks(lib):
    q = lib.oscar_quantize_pack_codebook

    def lv(*v):
        return ctypes.cast((ctypes.c_uint16 * 4)(*v), ctypes.c_void_p)

    good = lv(0x0000, 0x3C00, 0x4000, 0x4200)     # 0, 1, 2, 3
    assert q(0, 128, 128, 0.96, None, good, None, None, None) == 0
    assert q(4, 128, 128, 0.96, 1, None, 1, 1, None) == -1                        # no levels
    assert q(4, 128, 128, 0.96, 1, lv(0x0000, 0x4000, 0x3C00, 0x4200), 1, 1, None) == -1   # not increasing
    assert q(4, 128, 128, 0.96, 1, lv(0x0000, 0x3C00, 0x3C00, 0x4200), 1, 1, None) == -1   # repeated level
    assert q(4, 128, 128, 0.96, 1, lv(0x0000, 0x3C00, 0x4000, 0x7E00), 1, 1, None) == -1   # NaN
    assert q(4, 128, 128, 0.96, 1, lv(0x0000, 0x3C00, 0x4000, 0x7C00), 1, 1, None) == -1   # infinity
    assert q(4, 128, 48, 0.96, 1, good, 1, 1, None) == -1
    assert q(4, 6, 6, 0.96, 1, good, 1, 1, None) == -1
    assert q(4, 128, 128, 1.5, 1, good, 1, 1, None) == -1
    assert q(4, 2048, 128, 0.96, 1, good, 1, 1, None) == -2
    assert q(4, 128, 128, 0.96, None, good, 1, 1, None) == -1


def test_codebook_fit_argument_checks(lib):
    """Invalid arguments are rejected before any device work; with no rows the uniform levels come
    back after one iteration (no device call is made)."""
    f = lib.oscar_codebook_fit
    lv = (ctypes.c_double * 8)()
    pats = (ctypes.c_uint16 * 8)()
    its = (ctypes.c_int32 * 2)()
    P_ = ctypes.c_void_p
    out = (ctypes.cast(lv, P_), ctypes.cast(pats, P_), ctypes.cast(its, P_))
    assert f(2, 0, 128, None, None, 0.96, 100, 1e-7, None, 0, *out, None) == 0
    assert list(lv) == [0.0, 1.0, 2.0, 3.0] * 2 and list(pats) == [0x0000, 0x3C00, 0x4000, 0x4200] * 2
    assert list(its) == [1, 1]
    assert f(0, 10, 128, 1, 1, 0.96, 100, 1e-7, 1, 1 << 30, *out, None) == -1      # no heads
    assert f(2, 10, 96, 1, 1, 0.96, 100, 1e-7, 1, 1 << 30, *out, None) == -2       # head_dim
    assert f(2, 10, 128, 1, 1, 0.0, 100, 1e-7, 1, 1 << 30, *out, None) == -1       # clip
    assert f(2, 10, 128, 1, 1, 0.96, 0, 1e-7, 1, 1 << 30, *out, None) == -1        # max_iter
    assert f(2, 10, 128, 1, 1, 0.96, 100, -1.0, 1, 1 << 30, *out, None) == -1      # tol
    assert f(2, 10, 128, None, 1, 0.96, 100, 1e-7, 1, 1 << 30, *out, None) == -1   # null rows
    assert f(2, 10, 128, 1, 1, 0.96, 100, 1e-7, 1, 1 << 30, None, out[1], None, None) == -1
    assert f(2, 10, 128, 1, 1, 0.96, 100, 1e-7, 1, 16, *out, None) == -3           # workspace
    assert brk.codebook_workspace_bytes(2, 10, 128) >= 2 * 10 * 128 * 4
    assert brk.codebook_workspace_bytes(2, 10, 96) == 0


def test_misaligned_codebook_rejected(lib):
    L = layout()
    L.codebook = 0x1002
    assert brk.page_bytes(L, 2) == 0 and brk.decode_workspace_bytes(L, 1, 1000) == 0
    r = lib.oscar_decode_attn(ctypes.byref(L), 1, 1000, 1, 1, None, 1, 1, 1, None, 100, 1, 1, 0.0, 1, 1 << 30, 1,
                              None)
    assert r == -1
    L.codebook = 0x1000
    assert brk.page_bytes(L, 2) == 8 * 1152


def test_bf16_argument_checks(lib):
    L = ctypes.byref(layout())
    assert lib.oscar_bf16_decode_attn(L, 1, 1000, None, 1, 1, 10, 1, 100, 0.0, 1, 1 << 30, 1, None) == -1
    assert lib.oscar_bf16_decode_attn(L, 1, 1000, 1, 1, 1, 10, 1, 100, 0.0, 1, 8, 1, None) == -3
    assert lib.oscar_bf16_fill(L, 1, 1000, 1, 1, 1, 1, 10, 1, 0, None) == -1   # empty page table
