"""Pins of the oracle's Lloyd-Max codebook (no GPU): textbook Lloyd-Max values, closed forms,
the fixed-point conditions, brute force on the encoder, and the reduction to the uniform codec."""
import numpy as np
import pytest
from scipy.special import ndtri

import oracle
import synth


def test_lloyd_max_gaussian_matches_max_table():
    # Max (1960), optimum 4-level quantiser of the unit normal density: output levels +-0.4528,
    # +-1.510, decision thresholds 0, +-0.9816, mean squared error 0.1175. The samples are the
    # normal quantiles at (i + 1/2) / n, a deterministic stand-in for the density.
    n = 400_000
    x = ndtri((np.arange(n) + 0.5) / n)
    lv, it, mse = oracle.lloyd_max(x, init=(-1.5, -0.5, 0.5, 1.5), max_iter=2000, tol=1e-10)
    assert it < 2000
    assert np.allclose(lv, [-1.510, -0.4528, 0.4528, 1.510], atol=2e-3)
    assert np.allclose(0.5 * (lv[:-1] + lv[1:]), [-0.9816, 0.0, 0.9816], atol=2e-3)
    assert abs(mse[-1] - 0.1175) < 1e-3


def test_lloyd_max_uniform_density_closed_form():
    # for the uniform density on [0, 3] the optimum 4-level quantiser is uniform: levels at the
    # cell centres 3/8, 9/8, 15/8, 21/8, and the squared error (3/4)^2 / 12
    n = 300_000
    x = 3.0 * (np.arange(n) + 0.5) / n
    lv, it, mse = oracle.lloyd_max(x, max_iter=2000, tol=1e-12)
    assert np.allclose(lv, [3 / 8, 9 / 8, 15 / 8, 21 / 8], atol=1e-5)
    assert abs(mse[-1] - 0.75 ** 2 / 12) < 1e-6


def test_lloyd_max_fixed_point_and_monotone_error():
    r = np.random.default_rng(5)
    x = np.concatenate([r.normal(0.3, 0.2, 3000), r.normal(1.4, 0.5, 5000), r.uniform(0, 3, 2000),
                        np.zeros(300), np.full(300, 3.0)])
    lv, it, mse = oracle.lloyd_max(x, max_iter=5000, tol=1e-13)
    assert np.all(np.diff(mse) <= 1e-15)            # Lloyd never raises the error
    assert mse[-1] < mse[0]
    t = 0.5 * (lv[:-1] + lv[1:])
    cell = np.searchsorted(t, x, side="left")       # brute-force nearest level (no sample on a threshold)
    near = np.argmin(np.abs(x[:, None] - lv[None, :]), axis=1)
    assert np.array_equal(cell, near)
    for j in range(4):                              # centroid condition
        assert abs(lv[j] - x[cell == j].mean()) < 1e-9


def test_lloyd_max_four_clusters_and_empty_cells():
    x = np.repeat([0.2, 1.1, 1.7, 2.9], [10, 3, 7, 5])
    lv, it, mse = oracle.lloyd_max(x, max_iter=100, tol=0.0)
    assert np.allclose(lv, [0.2, 1.1, 1.7, 2.9]) and mse[-1] < 1e-30
    # every sample in cell 2: the other levels do not move
    lv, it, _ = oracle.lloyd_max(np.full(50, 2.125), max_iter=10)
    assert lv.tolist() == [0.0, 1.0, 2.125, 3.0]
    with pytest.raises(ValueError):
        oracle.lloyd_max(x, init=(0.0, 2.0, 1.0, 3.0))


def _uniform_u(x, group, clip):
    """The quantiser's coordinate, recomputed here in fp32 from its definition."""
    n, d = x.shape
    out = np.zeros_like(x)
    ok = np.zeros(x.shape, bool)
    for i in range(n):
        for gi in range(d // group):
            v = x[i, gi * group:(gi + 1) * group]
            lo = np.float32(np.float32(clip) * v.min())
            hi = np.float32(np.float32(clip) * v.max())
            s = oracle.bf16_round(np.float32((hi - lo) / np.float32(3.0)))[()]
            z = oracle.bf16_round(lo)[()]
            if s == 0:
                continue
            xc = np.minimum(np.maximum(v, lo), hi)
            out[i, gi * group:(gi + 1) * group] = (xc - z) / s
            ok[i, gi * group:(gi + 1) * group] = True
    return out, ok


def test_codebook_encoder_is_nearest_level():
    r = np.random.default_rng(8)
    x = synth.standard_rows(4, 48, 64, scale=3.0)
    u_ref, ok = _uniform_u(x, 32, 0.96)
    for trial in range(6):
        lv = oracle.fp16_levels(np.sort(r.uniform(0, 3, 4)) + np.arange(4) * 0.01)
        codes, sz = oracle.quantize_rows_codebook(x, 32, 0.96, lv)
        dist = np.abs(u_ref.astype(np.float64)[..., None] - lv.astype(np.float64))
        best = np.argmin(dist, axis=-1)
        srt = np.sort(dist, axis=-1)
        clear = ok & (srt[..., 1] - srt[..., 0] > 1e-6)
        assert np.array_equal(codes[clear], best[clear])
        assert np.all(codes[~ok] == 0)
        assert np.array_equal(sz, oracle.quantize_rows(x, 32, 2, 0.96)[1])


def test_codebook_ties_go_even_and_uniform_levels_reduce_to_uniform_codec():
    # s = 1, z = 0: u equals x, and 0.5, 1.5, 2.5 lie exactly on the thresholds
    g = np.array([[0.0, 3.0, 0.5, 1.5, 2.5, 1.0, 2.0, 0.25]], np.float32)
    c, _ = oracle.quantize_rows_codebook(g, 8, 1.0, oracle.fp16_levels(oracle.UNIFORM_LEVELS))
    assert c[0].tolist() == [0, 3, 0, 2, 2, 1, 2, 0]
    # a threshold of an irregular codebook: u = t_1 goes up to code 2 (even), u = t_0 stays at 0
    lv = np.array([0.0, 1.0, 2.0, 2.5], np.float32)     # t = 0.5, 1.5, 2.25
    g = np.array([[0.0, 3.0, 0.5, 1.5, 2.25, 2.3]], np.float32)
    c, _ = oracle.quantize_rows_codebook(g, 6, 1.0, lv)
    assert c[0].tolist() == [0, 3, 0, 2, 2, 3]
    for seed in range(4):
        x = synth.standard_rows(seed, 30, 128, scale=5.0)
        for group in (32, 128):
            a = oracle.quantize_rows_codebook(x, group, 0.96, oracle.fp16_levels(oracle.UNIFORM_LEVELS))
            b = oracle.quantize_rows(x, group, 2, 0.96)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
            assert np.array_equal(oracle.dequantize_rows_codebook(a[0], a[1], group, oracle.UNIFORM_LEVELS),
                                  oracle.dequantize_rows(b[0], b[1], group))


def test_codebook_dequantisation_elementwise():
    x = synth.standard_rows(9, 5, 64, scale=2.0)
    lv = oracle.fp16_levels([0.21, 0.97, 2.03, 2.81])
    codes, sz = oracle.quantize_rows_codebook(x, 16, 0.92, lv)
    xh = oracle.dequantize_rows_codebook(codes, sz, 16, lv)
    for i in range(5):
        for j in range(64):
            s = float(oracle.bf16_from_bits(sz[i, j // 16, 0]))
            z = float(oracle.bf16_from_bits(sz[i, j // 16, 1]))
            assert xh[i, j] == z + s * float(lv[codes[i, j]])


def test_thresholds_and_fp16_rounding():
    lv = oracle.fp16_levels([0.1, 1.0000001, 2.3, 2.9999])
    assert lv.dtype == np.float32 and lv[1] == 1.0 and lv[3] == np.float32(np.float16(2.9999))
    t = oracle.thresholds_fp32(lv)
    assert np.array_equal(t.astype(np.float64), 0.5 * (lv[:-1].astype(np.float64) + lv[1:]))
    assert oracle.fp16_patterns([1.0, 2.0])[0] == 0x3C00 and oracle.fp16_patterns([1.0, 2.0])[1] == 0x4000


def test_fit_codebook_lowers_the_quantisation_error():
    d, n = 64, 256
    r = np.random.default_rng(2)
    x = (r.standard_normal((n, d)) * np.linspace(0.2, 3.0, d)).astype(np.float32)
    x = oracle.rotate_rows_fp32(x, synth.random_orthogonal(r, d).astype(np.float32))
    lv64, lv, it = oracle.fit_codebook(x, 64, 0.96)
    assert np.all(np.diff(lv64) > 0) and lv64[0] >= 0.0 and lv64[3] <= 3.0
    u, ok = oracle.group_coordinates(x, 64, 0.96)
    uu = u[ok].astype(np.float64)

    def err(levels):
        c = oracle.code_of_coordinate(u[ok], levels)
        return np.mean((uu - np.asarray(levels, np.float64)[c]) ** 2)

    assert err(lv) < err(oracle.fp16_levels(oracle.UNIFORM_LEVELS))
    assert np.allclose(lv64, lv, atol=2e-3)


def test_cache_with_codebook():
    w = synth.workload(1)
    kv = 0
    T = 600
    ks, vs = synth.kv_slice(w, 0, kv, T)
    rk = np.eye(w.head_dim, dtype=np.float32)[None]
    uni = oracle.fp16_levels(oracle.UNIFORM_LEVELS)[None]
    a = oracle.OracleCache.from_prefix(ks[None], vs[None], rk, rk, w.group_size)
    b = oracle.OracleCache.from_prefix(ks[None], vs[None], rk, rk, w.group_size, codebook_k=uni, codebook_v=uni)
    assert np.array_equal(a.k_codes, b.k_codes) and np.array_equal(a.v_sz, b.v_sz)
    q = synth.decode_query(w, 0)[:w.gqa]
    assert np.array_equal(oracle.decode_attention(a, q), oracle.decode_attention(b, q))
    lk = oracle.fp16_levels([0.3, 1.1, 1.9, 2.7])[None]
    lvv = oracle.fp16_levels([0.2, 1.05, 1.95, 2.8])[None]
    c = oracle.OracleCache.from_prefix(ks[None], vs[None], rk, rk, w.group_size, codebook_k=lk, codebook_v=lvv)
    xk, xv = c.history_rows(0)
    assert np.array_equal(xk, oracle.dequantize_rows_codebook(c.k_codes[0], c.k_sz[0], w.group_size, lk[0]))
    assert np.array_equal(xv, oracle.dequantize_rows_codebook(c.v_codes[0], c.v_sz[0], w.group_size, lvv[0]))
    # with R = I the history logits are plain dot products with the dequantised rows
    o = oracle.decode_attention(c, q)
    kb, vb, _ = c.bf16_rows(0)
    qq = oracle.bf16_round(q).astype(np.float64)
    for h in range(w.gqa):
        lg = np.concatenate([kb @ qq[h], xk @ qq[h]]) / np.sqrt(w.head_dim)
        p = np.exp(lg - lg.max())
        p /= p.sum()
        assert np.allclose(o[h], p[:len(kb)] @ vb + p[len(kb):] @ xv, rtol=1e-12, atol=1e-12)
