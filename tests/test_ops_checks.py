"""The Python wrappers reject tensors whose shapes or sizes do not match the layout before they call
the library (the C ABI sees pointers only, so a short buffer would become an out-of-bounds device
access). CPU only: the device check is stubbed out and the library's compute entry points are
replaced by a guard that fails the test if reached; size queries go to the real library."""
import os

import pytest
import torch

from bit_rotated_kv_amd import _lib, ops


class _Guard:
    """The real library for size queries; any other call is an error."""

    SIZE = ("oscar_page_bytes", "oscar_window_bytes", "oscar_pool_bytes", "oscar_decode_workspace_bytes",
            "oscar_bf16_decode_workspace_bytes", "oscar_status_string")

    def __init__(self, real):
        self.real = real

    def __getattr__(self, name):
        if name in self.SIZE:
            return getattr(self.real, name)
        raise AssertionError(f"{name} reached with invalid arguments")


@pytest.fixture(autouse=True)
def guarded(monkeypatch):
    if not os.path.exists(_lib.LIB_PATH):
        from bit_rotated_kv_amd import build
        build.build()
    real = _lib.lib()
    monkeypatch.setattr(ops, "_need", lambda *a, **k: None)
    monkeypatch.setattr(ops, "lib", lambda: _Guard(real))
    monkeypatch.setattr(ops, "_stream", lambda: None)


B, HQ, HKV, D, TMAX, STRIDE, POOL = 2, 8, 2, 64, 600, 24, 48


def layout():
    return ops.make_layout(HQ, HKV, D, pool_pages=POOL)


def bufs(lay):
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt)
    return dict(
        q=z(B, HQ, D, dt=torch.bfloat16), out=z(B, HQ, D), seq_len=z(B, dt=torch.int32),
        pool=z(ops.pool_bytes(lay), dt=torch.uint8), window=z(ops.window_bytes(lay, B), dt=torch.uint8),
        page_table=z(B, STRIDE, dt=torch.int32), rot_k=z(HKV, D, D), rot_v=z(HKV, D, D),
        new_k=z(B, HKV, D, dt=torch.bfloat16), new_v=z(B, HKV, D, dt=torch.bfloat16),
        seq_len_out=z(B, dt=torch.int32), workspace=z(1 << 20, dt=torch.uint8),
        k=z(B, HKV, TMAX, D, dt=torch.bfloat16), v=z(B, HKV, TMAX, D, dt=torch.bfloat16))


def call_decode(lay, b):
    ops.decode_attn(lay, b["q"], b["seq_len"], b["window"], b["pool"], b["page_table"], b["rot_k"], b["rot_v"],
                    b["workspace"], TMAX, out=b["out"])


def call_step(lay, b):
    ops.decode_step(lay, b["seq_len"], b["new_k"], b["new_v"], b["q"], b["rot_k"], b["rot_v"], b["pool"],
                    b["page_table"], b["window"], b["seq_len_out"], b["workspace"], TMAX, out=b["out"])


def call_demote(lay, b):
    ops.kv_demote(lay, b["seq_len"], b["new_k"], b["new_v"], b["rot_k"], b["rot_v"], b["pool"], b["page_table"],
                  b["window"], seq_len_out=b["seq_len_out"])


def call_prefill(lay, b):
    ops.kv_prefill(lay, b["seq_len"], b["k"], b["v"], b["rot_k"], b["rot_v"], b["pool"], b["page_table"],
                   b["window"])


BAD = [
    ("q", lambda b: b["q"][:, :-1]),
    ("out", lambda b: b["out"][:1]),
    ("seq_len", lambda b: b["seq_len"][:1]),
    ("page_table", lambda b: b["page_table"][:1]),
    ("rot_k", lambda b: b["rot_k"][:1]),
    ("rot_v", lambda b: b["rot_v"][:, :-1]),
    ("pool", lambda b: b["pool"][:-1]),
    ("window", lambda b: b["window"][:-16]),
]


@pytest.mark.parametrize("name,mutate", BAD, ids=[n for n, _ in BAD])
def test_decode_attn_rejects(name, mutate):
    lay = layout()
    b = bufs(lay)
    b[name] = mutate(b)
    with pytest.raises(ValueError):
        call_decode(lay, b)


STEP_BAD = BAD + [("new_k", lambda b: b["new_k"][:, :1]), ("new_v", lambda b: b["new_v"][:1]),
                  ("seq_len_out", lambda b: b["seq_len_out"][:1])]


@pytest.mark.parametrize("name,mutate", STEP_BAD, ids=[n for n, _ in STEP_BAD])
def test_decode_step_rejects(name, mutate):
    lay = layout()
    b = bufs(lay)
    b[name] = mutate(b)
    with pytest.raises(ValueError):
        call_step(lay, b)


@pytest.mark.parametrize("name,mutate", [x for x in STEP_BAD if x[0] not in ("q", "out")],
                         ids=[n for n, _ in STEP_BAD if n not in ("q", "out")])
def test_kv_demote_rejects(name, mutate):
    lay = layout()
    b = bufs(lay)
    b[name] = mutate(b)
    with pytest.raises(ValueError):
        call_demote(lay, b)


PREFILL_BAD = [x for x in BAD if x[0] not in ("q", "out")] + [
    ("k", lambda b: b["k"][:, :, :, :-1]), ("v", lambda b: b["v"][:, :, :-1])]


@pytest.mark.parametrize("name,mutate", PREFILL_BAD, ids=[n for n, _ in PREFILL_BAD])
def test_kv_prefill_rejects(name, mutate):
    lay = layout()
    b = bufs(lay)
    b[name] = mutate(b)
    with pytest.raises(ValueError):
        call_prefill(lay, b)


def test_mismatched_int4_table_rejected():
    lay = ops.make_layout(HQ, HKV, D, mixed=True, int4_page_offset=POOL // 2, pool_pages=POOL)
    b = bufs(lay)
    b["pool"] = torch.zeros(ops.pool_bytes(lay), dtype=torch.uint8)
    with pytest.raises(ValueError):
        ops.decode_attn(lay, b["q"], b["seq_len"], b["window"], b["pool"], b["page_table"], b["rot_k"], b["rot_v"],
                        b["workspace"], TMAX, out=b["out"], n_int4=b["seq_len"],
                        page_table4=torch.zeros(B, STRIDE + 1, dtype=torch.int32))


def test_bf16_baseline_rejects_short_pages():
    lay = layout()
    b = bufs(lay)
    pages = torch.zeros(10 * ops.page_bytes(lay, 16) - 1, dtype=torch.uint8)
    with pytest.raises(ValueError):
        ops.bf16_decode_attn(lay, b["q"], b["seq_len"], pages, 10, b["page_table"], b["workspace"], TMAX,
                             out=b["out"])
    with pytest.raises(ValueError):
        ops.bf16_fill(lay, b["seq_len"], b["k"], b["v"], pages, 10, b["page_table"])


def test_quantize_pack_rejects_short_outputs():
    x = torch.zeros(5, 128)
    with pytest.raises(ValueError):
        ops.quantize_pack(x, 128, 2, 0.96, codes=torch.zeros(5, 31, dtype=torch.uint8))
    with pytest.raises(ValueError):
        ops.quantize_pack(x, 128, 2, 0.96, scale_zero=torch.zeros(4, 1, 2, dtype=torch.int16))


def test_valid_shapes_reach_the_library():
    """The same buffers, unmodified, pass every check and reach the guarded compute entry point."""
    lay = layout()
    b = bufs(lay)
    with pytest.raises(AssertionError, match="oscar_decode_attn reached"):
        call_decode(lay, b)
    with pytest.raises(AssertionError, match="oscar_decode_step reached"):
        call_step(lay, b)
