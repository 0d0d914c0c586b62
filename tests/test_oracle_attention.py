"""Pins of the oracle's decode attention: brute force on tiny inputs, rotation
convention, split-and-merge equivalence, permutation invariance, closed forms (no GPU)."""
import numpy as np
import pytest

import oracle
import synth


def _cache(T, hkv=2, d=16, group=8, seed=30, bits=2, scale_k=3.0):
    r = np.random.default_rng(seed)
    K = r.standard_normal((hkv, T, d)).astype(np.float32) * scale_k
    V = r.standard_normal((hkv, T, d)).astype(np.float32)
    rk = np.stack([synth.random_orthogonal(r, d) for _ in range(hkv)]).astype(np.float32)
    rv = np.stack([synth.random_orthogonal(r, d) for _ in range(hkv)]).astype(np.float32)
    bits_arr = np.full(T, bits) if np.isscalar(bits) else bits
    c = oracle.OracleCache.from_prefix(K, V, rk, rv, group, bits=bits_arr)
    return c, K, V, r


def test_softmax_attention_brute_force():
    r = np.random.default_rng(31)
    lg = r.standard_normal(9) * 4
    v = r.standard_normal((9, 3))
    o, lse = oracle.softmax_attention(lg, v)
    e = [np.exp(x) for x in lg]
    ref = [sum(e[t] * v[t, j] for t in range(9)) / sum(e) for j in range(3)]
    assert np.allclose(o, ref, rtol=1e-13) and np.isclose(lse, np.log(sum(e)), rtol=1e-14)


def test_decode_brute_force_loops():
    """Scalar loops over tokens and channels (dequantise element by element, rotate with
    explicit sums) against the vectorised oracle."""
    c, K, V, r = _cache(400)
    q = r.standard_normal((4, 16)).astype(np.float32)
    out = oracle.decode_attention(c, q)
    qb = oracle.bf16_round(q).astype(np.float64)
    d, scale = 16, 1 / 4.0
    for h in range(4):
        kv = h // 2
        logits, vals = [], []
        for p in c.bf16_positions():
            logits.append(scale * sum(qb[h, j] * float(c.bf16_k[p][kv, j]) for j in range(d)))
            vals.append([float(c.bf16_v[p][kv, j]) for j in range(d)])
        qr = [sum(qb[h, i] * float(c.rot_k[kv][i, j]) for i in range(d)) for j in range(d)]
        for n in range(len(c.hist_pos)):
            xk, xv = [], []
            for j in range(d):
                g = j // c.group
                s = float(oracle.bf16_from_bits(c.k_sz[kv, n, g, 0])); z = float(oracle.bf16_from_bits(c.k_sz[kv, n, g, 1]))
                xk.append(s * c.k_codes[kv, n, j] + z)
                s = float(oracle.bf16_from_bits(c.v_sz[kv, n, g, 0])); z = float(oracle.bf16_from_bits(c.v_sz[kv, n, g, 1]))
                xv.append(s * c.v_codes[kv, n, j] + z)
            logits.append(scale * sum(qr[j] * xk[j] for j in range(d)))
            vals.append([sum(xv[i] * float(c.rot_v[kv][j, i]) for i in range(d)) for j in range(d)])
        m = max(logits)
        e = [np.exp(x - m) for x in logits]
        ref = [sum(e[t] * vals[t][j] for t in range(len(e))) / sum(e) for j in range(d)]
        assert np.allclose(out[h], ref, rtol=1e-11, atol=1e-12)


def test_rotation_convention_equals_unrotated_keys():
    """(q R_K) . x_hat = q . (x_hat R_K^T) and (p x_hat_V) R_V^T = p (x_hat_V R_V^T): the
    oracle equals plain attention over keys/values mapped back to the original basis."""
    c, K, V, r = _cache(500)
    q = r.standard_normal((4, 16)).astype(np.float32)
    out = oracle.decode_attention(c, q)
    qb = oracle.bf16_round(q).astype(np.float64)
    for h in range(4):
        kv = h // 2
        kb, vb, _ = c.bf16_rows(kv)
        kh = oracle.dequantize_rows(c.k_codes[kv], c.k_sz[kv], 8) @ c.rot_k[kv].astype(np.float64).T
        vh = oracle.dequantize_rows(c.v_codes[kv], c.v_sz[kv], 8) @ c.rot_v[kv].astype(np.float64).T
        o, _ = oracle.softmax_attention(0.25 * np.concatenate([kb, kh]) @ qb[h], np.concatenate([vb, vh]))
        assert np.allclose(out[h], o, rtol=1e-12, atol=1e-13)


def test_fine_quantiser_approaches_plain_attention():
    """With an 8-bit quantiser and no clip the history is nearly exact, so the mixed cache
    must reproduce plain BF16 attention (a wrong rotation or transpose would not)."""
    c, K, V, r = _cache(700, bits=8, scale_k=1.0)
    q = r.standard_normal((4, 16)).astype(np.float32)
    got = oracle.decode_attention(c, q)
    ref = oracle.plain_decode_attention(q, K, V)
    assert np.abs(got - ref).max() < 2e-2 * np.abs(ref).max()
    c2, *_ = _cache(700, bits=2, scale_k=1.0)
    coarse = np.abs(oracle.decode_attention(c2, q) - ref).max()
    assert coarse > np.abs(got - ref).max()


def test_split_and_merge_equals_single_softmax():
    r = np.random.default_rng(32)
    q = r.standard_normal(8)
    keys = r.standard_normal((300, 8)) * 2
    vals = r.standard_normal((300, 8))
    full = oracle.partial_attention(q, keys, vals, 0.35)
    for trial in range(5):
        cuts = np.sort(r.choice(np.arange(1, 300), size=r.integers(1, 10), replace=False))
        bounds = [0, *cuts.tolist(), 300]
        parts = [oracle.partial_attention(q, keys[a:b], vals[a:b], 0.35) for a, b in zip(bounds[:-1], bounds[1:])]
        parts.append(oracle.partial_attention(q, keys[:0], vals[:0], 0.35))   # empty part is neutral
        o, lse = oracle.lse_merge(parts)
        assert np.allclose(o, full[0], rtol=1e-13, atol=1e-14) and np.isclose(lse, full[1], rtol=1e-14)


def test_history_order_invariance():
    c, K, V, r = _cache(600, bits=np.where(np.arange(600) % 5 == 0, 4, 2))
    q = r.standard_normal((4, 16)).astype(np.float32)
    out = oracle.decode_attention(c, q)
    perm = r.permutation(len(c.hist_pos))
    for name in ("hist_pos", "hist_bits"):
        setattr(c, name, getattr(c, name)[perm])
    for name in ("k_codes", "v_codes", "k_sz", "v_sz"):
        setattr(c, name, getattr(c, name)[:, perm])
    assert np.allclose(oracle.decode_attention(c, q), out, rtol=1e-12, atol=1e-14)


def test_zero_query_gives_mean_of_values():
    c, K, V, r = _cache(450)
    out = oracle.decode_attention(c, np.zeros((4, 16), np.float32))
    for h in range(4):
        kv = h // 2
        kb, vb, _ = c.bf16_rows(kv)
        vh = oracle.dequantize_rows(c.v_codes[kv], c.v_sz[kv], 8) @ c.rot_v[kv].astype(np.float64).T
        assert np.allclose(out[h], np.concatenate([vb, vh]).mean(0), rtol=1e-12, atol=1e-13)


def test_plain_attention_dominant_key():
    K = np.zeros((1, 5, 4), np.float32)
    V = np.arange(20, dtype=np.float32).reshape(1, 5, 4)
    K[0, 3] = [100, 0, 0, 0]
    out = oracle.plain_decode_attention(np.array([[1, 0, 0, 0]], np.float32), K, V)
    assert np.allclose(out[0], V[0, 3], atol=1e-12)
