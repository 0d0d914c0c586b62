"""Pins of the oracle's cache segments, bits-per-element figures and step semantics
against numbers printed on the pages (tests/golden/page_figures.txt) (no GPU)."""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")


def golden():
    out = {}
    for line in open(GOLDEN):
        line = line.split("|")[0].strip()
        if not line or line.startswith("#"):
            continue
        k, v, prec = line.split()
        out[k] = (float(v), int(prec))
    return out


def test_page_constants():
    g = golden()
    assert oracle.SINK == g["sink_tokens"][0] and oracle.RECENT == g["recent_tokens"][0]
    assert 8 // 2 == g["codes_per_byte_int2"][0]
    assert oracle.pack_codes(np.zeros((1, 8), np.uint8), 2).shape[1] * g["codes_per_byte_int2"][0] == 8


def test_bf16_share_at_128k():
    g = golden()
    T = 131072
    (s0, s1), (h0, h1), (r0, r1) = oracle.segments(T)
    share = 100.0 * (T - (h1 - h0)) / T
    v, prec = g["bf16_share_128k_pct"]
    assert round(share, prec) == v


def test_effective_bits_match_pages():
    g = golden()
    for key, T in (("bpe_oscar_128k", 131072), ("bpe_oscar_32k", 32768)):
        v, prec = g[key]
        assert round(oracle.effective_bits(T, 128), prec) == v, key
    v, prec = g["bpe_plain_int2"]
    assert round(oracle.effective_bits(10 ** 6, 128, sink=0, recent=0), prec) == v
    v, prec = g["history_memory_ratio"]
    assert 16 / 2 == v


def test_segments_sum_and_bounds():
    for T in range(0, 2001):
        (s0, s1), (h0, h1), (r0, r1) = oracle.segments(T)
        assert (s1 - s0) + (h1 - h0) + (r1 - r0) == T
        assert s0 == 0 and s1 <= 64 and h0 <= h1 and r0 <= r1 == T
        assert s1 <= h0 or h1 == h0
        assert h1 <= r0 or h1 == h0
        if T > 320:
            assert (s1, h0, h1, r0) == (64, 64, T - 256, T - 256)
        assert r1 - r0 <= 256


def _tiny_cache_inputs(T, hkv=2, d=16, seed=20):
    r = np.random.default_rng(seed)
    K = r.standard_normal((hkv, T, d)).astype(np.float32) * 3
    V = r.standard_normal((hkv, T, d)).astype(np.float32)
    rk = np.stack([synth.random_orthogonal(r, d) for _ in range(hkv)]).astype(np.float32)
    rv = np.stack([synth.random_orthogonal(r, d) for _ in range(hkv)]).astype(np.float32)
    return K, V, rk, rv


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 319, 320, 321, 400])
def test_prefix_equals_step_by_step(T):
    K, V, rk, rv = _tiny_cache_inputs(T)
    bits = np.where(np.arange(T) % 3 == 0, 4, 2)
    a = oracle.OracleCache.from_prefix(K, V, rk, rv, 8, bits=bits)
    b = oracle.OracleCache(rk, rv, 8)
    for t in range(T):
        b.append(K[:, t], V[:, t], int(bits[t]))
    assert a.T == b.T == T
    assert a.bf16_positions() == b.bf16_positions()
    oa, ob = np.argsort(a.hist_pos), np.argsort(b.hist_pos)
    assert np.array_equal(a.hist_pos[oa], b.hist_pos[ob])
    for name in ("k_codes", "v_codes", "k_sz", "v_sz"):
        assert np.array_equal(getattr(a, name)[:, oa], getattr(b, name)[:, ob]), name
    (s0, s1), (h0, h1), (r0, r1) = oracle.segments(T)
    assert sorted(a.hist_pos.tolist()) == list(range(h0, h1))
    assert a.bf16_positions() == list(range(s0, s1)) + list(range(r0, r1))


def test_demote_moves_oldest_recent_token():
    K, V, rk, rv = _tiny_cache_inputs(330)
    c = oracle.OracleCache.from_prefix(K[:, :325], V[:, :325], rk, rv, 16)
    assert 325 - 256 in c.bf16_positions()
    c.append(K[:, 325], V[:, 325])
    assert 325 - 256 not in c.bf16_positions() and c.hist_pos[-1] == 69
    # the history entry is the quantised rotated bf16 key
    kc, ks = oracle.quantize_rows(oracle.rotate_rows_fp32(oracle.bf16_round(K[0, 69])[None], rk[0]), 16, 2, 0.96)
    assert np.array_equal(c.k_codes[0, -1], kc[0]) and np.array_equal(c.k_sz[0, -1], ks[0])
