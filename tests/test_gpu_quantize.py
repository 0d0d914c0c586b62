"""oscar_quantize_pack on the GPU is bit-exact with the oracle quantiser on the same fp32 inputs."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_amd as brk
import oracle
import synth

pytestmark = pytest.mark.gpu


def gpu_qp(x, group, bits, clip):
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    codes, sz = brk.quantize_pack(xt, group, bits, clip)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sz.cpu().numpy().view(np.uint16)


def oracle_qp(x, group, bits, clip):
    c, sz = oracle.quantize_rows(x, group, bits, clip)
    return oracle.pack_codes(c, bits), sz


def rows_with_outliers(seed, n, dim, scale):
    x = synth.standard_rows(seed, n, dim, scale)
    r = np.random.default_rng(seed)
    cols = r.choice(dim, size=max(1, dim // 32), replace=False)
    x[:, cols] *= np.float32(r.uniform(10, 30))
    return x


@pytest.mark.parametrize("dim,group,bits,clip", [
    (128, 128, 2, 0.96), (128, 128, 2, 0.92), (64, 64, 2, 0.96), (128, 64, 2, 0.96), (128, 32, 2, 1.0),
    (128, 128, 4, 1.0), (256, 128, 4, 0.9), (1024, 1024, 2, 0.96), (8, 4, 2, 0.5), (100, 20, 2, 0.96),
])
def test_quantize_pack_bit_exact(dim, group, bits, clip):
    print(f"case dim={dim} group={group} bits={bits} clip={clip}", flush=True)
    x = rows_with_outliers(dim + bits, 777, dim, 3.0)
    gc, gs = gpu_qp(x, group, bits, clip)
    oc, os_ = oracle_qp(x, group, bits, clip)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


def test_quantize_pack_edge_groups():
    rows = [
        np.zeros(64), np.full(64, 3.7), np.full(64, -1e-3),
        np.tile([0.0, 1.0, 2.0, 3.0, 0.5, 1.5, 2.5, 3.0], 8),                     # exact ties on the grid
        np.linspace(-1e30, 1e30, 64), np.linspace(-1e-30, 2e-30, 64),           # huge / tiny ranges
        -np.abs(np.linspace(1, 9, 64)), np.abs(np.linspace(1, 9, 64)),          # one-signed groups
        np.where(np.arange(64) == 7, 100.0, 0.0), np.where(np.arange(64) == 7, -100.0, 1.0),
    ]
    x = np.stack(rows).astype(np.float32)
    for bits, clip in ((2, 0.96), (2, 1.0), (4, 1.0), (2, 0.5)):
        gc, gs = gpu_qp(x, 64, bits, clip)
        oc, os_ = oracle_qp(x, 64, bits, clip)
        assert np.array_equal(gs, os_), (bits, clip)
        assert np.array_equal(gc, oc), (bits, clip)


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("bits,clip", [(2, 0.96), (2, 0.92), (4, 1.0), (2, 1.0)])
def test_quantize_pack_near_rounding_midpoints(bits, clip):
    """Values a few ulps either side of every code midpoint z + (k + 1/2) s of their group, where the
    kernel's reciprocal estimate hands the decision to the exact division (and exact midpoints,
    which round to even): codes equal the oracle's. Sentinels at channels 0 and 1 fix each group's
    range, so the grid is known before the row is filled."""
    rng = np.random.default_rng(17 + bits)
    n, dim = 96, 128
    base = np.zeros((n, dim), np.float32)
    base[:, 0] = -rng.uniform(0.05, 40.0, n).astype(np.float32)
    base[:, 1] = rng.uniform(0.05, 40.0, n).astype(np.float32)
    _, sz = oracle.quantize_rows(base, dim, bits, clip)
    sz = np.asarray(sz).reshape(n, 2)
    s, z = _bf16_to_f32(sz[:, 0]), _bf16_to_f32(sz[:, 1])
    levels = (1 << bits) - 1
    x = base.copy()
    for r in range(n):
        vals = []
        for k in range(levels):
            m = np.float32(z[r] + np.float32(np.float32(k + 0.5) * s[r]))
            v = m
            for _ in range(3):
                v = np.nextafter(v, np.float32(-np.inf))
            for _ in range(7):
                vals.append(v)
                v = np.nextafter(v, np.float32(np.inf))
        vals = np.array(vals, np.float32)[: dim - 2]
        x[r, 2:2 + len(vals)] = vals
    _, sz2 = oracle.quantize_rows(x, dim, bits, clip)
    assert np.array_equal(np.asarray(sz2).reshape(n, 2), sz)      # the sentinels still set the grid
    gc, gs = gpu_qp(x, dim, bits, clip)
    oc, os_ = oracle_qp(x, dim, bits, clip)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


def test_quantize_pack_many_rows_ragged_tail():
    x = rows_with_outliers(5, 100_003, 128, 1.0)
    gc, gs = gpu_qp(x, 128, 2, 0.96)
    oc, os_ = oracle_qp(x, 128, 2, 0.96)
    assert np.array_equal(gs, os_) and np.array_equal(gc, oc)


def test_quantize_pack_empty():
    codes, sz = brk.quantize_pack(torch.zeros((0, 128), dtype=torch.float32, device="cuda"), 128, 2, 0.96)
    assert codes.shape == (0, 32) and sz.shape == (0, 1, 2)
