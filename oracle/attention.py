"""Decode attention over the mixed-precision cache (oracle, fp64).

Follows the OSCAR overview page (method paragraph: the INT2 kernel restores values from
scale and zero point and accumulates in floating point, the BF16 kernel handles sink and
recent, and an online-softmax merge combines them) and the OSCAR news article (keys are
stored as x . R_K, so logits of history keys use the rotated query q . R_K; values are
stored as v . R_V, so their weighted sum is taken back with R_V^T).

This is the definition written out: one softmax over all T logits of a query head, no
splitting. ``partial_attention`` and ``lse_merge`` state the split-and-merge form used by
the kernels; the tests pin that the two agree.

Readings: softmax scale 1/sqrt(d); the query is bf16; query head h reads kv-head
h // (Hq/Hkv) (contiguous GQA groups); the output is fp64 (compared as fp32).
"""
from __future__ import annotations

import numpy as np

from .quant import bf16_round


def softmax_attention(logits, values):
    """o = softmax(logits) @ values and lse = log sum exp(logits) (fp64, max-subtracted)."""
    logits = np.asarray(logits, np.float64)
    values = np.asarray(values, np.float64)
    if logits.size == 0:
        return np.zeros(values.shape[1] if values.ndim == 2 else 0), -np.inf
    m = logits.max()
    p = np.exp(logits - m)
    s = p.sum()
    return (p @ values) / s, m + np.log(s)


def partial_attention(q, keys, values, scale):
    """(o, lse) of one query over a subset of keys; an empty subset gives (0, -inf)."""
    keys = np.asarray(keys, np.float64)
    return softmax_attention(scale * (keys @ np.asarray(q, np.float64)), values)


def lse_merge(parts):
    """Merge partial results [(o_i, lse_i)] into the softmax over the union of their keys:
    o = sum_i exp(lse_i - LSE) o_i with LSE = log sum_i exp(lse_i)."""
    lses = np.array([p[1] for p in parts], np.float64)
    if np.all(np.isneginf(lses)):
        return np.zeros_like(np.asarray(parts[0][0], np.float64)), -np.inf
    m = lses.max()
    w = np.exp(lses - m)
    tot = w.sum()
    o = sum(wi * np.asarray(p[0], np.float64) for wi, p in zip(w, parts)) / tot
    return o, m + np.log(tot)


def decode_attention(cache, q, scale=None):
    """Attention output of decode queries q [Hq, d] over an ``OracleCache``; fp64 [Hq, d].

    Sink/recent logits: scale * q . k in the original basis. History logits:
    scale * (q . R_K) . x_hat_K with x_hat = s * code + z in the rotated basis (s * l[code] + z
    under a codebook). One softmax
    over all logits; o = sum_BF16 p v + (sum_hist p x_hat_V) . R_V^T."""
    q = bf16_round(np.asarray(q, np.float32)).astype(np.float64)
    hq, d = q.shape
    g = hq // cache.hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((hq, d))
    for h in range(hq):
        kv = h // g
        kb, vb, _ = cache.bf16_rows(kv)
        xk, xv = cache.history_rows(kv)
        q_rot = q[h] @ cache.rot_k[kv].astype(np.float64)
        logits = np.concatenate([scale * (kb @ q[h]), scale * (xk @ q_rot)])
        if logits.size == 0:
            continue
        m = logits.max()
        p = np.exp(logits - m)
        p /= p.sum()
        nb = kb.shape[0]
        out[h] = p[:nb] @ vb + (p[nb:] @ xv) @ cache.rot_v[kv].astype(np.float64).T
    return out


def plain_decode_attention(q, K, V, scale=None):
    """softmax(scale * q K^T) V per query head over full BF16 keys/values.

    q [Hq, d]; K, V [Hkv, T, d]; every input rounded to bf16 first. fp64 [Hq, d]."""
    q = bf16_round(np.asarray(q, np.float32)).astype(np.float64)
    K = bf16_round(np.asarray(K, np.float32)).astype(np.float64)
    V = bf16_round(np.asarray(V, np.float32)).astype(np.float64)
    hq, d = q.shape
    g = hq // K.shape[0]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((hq, d))
    for h in range(hq):
        o, _ = softmax_attention(scale * (K[h // g] @ q[h]), V[h // g])
        out[h] = o
    return out
