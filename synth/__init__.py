"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module only draws random numbers and lays out shapes. It holds none of the
method's arithmetic: no rotation, Hadamard, permutation, clipping, quantisation,
packing or attention. Every draw is keyed by (seed, role, indices) through
``numpy.random.SeedSequence`` so that one (request, kv-head) slice can be drawn
on its own, with the same values, whatever the batch it sits in.

The workload shapes follow the decode configurations of the OSCAR pages: a
Qwen3-8B-shaped layer (32 query heads, 8 KV heads, head_dim 128), a paged batch
of 32 requests, a Qwen3-32B-shaped layer (64 query heads, GQA 8) with ragged
lengths, and a TriAxialKV-style mixed INT2/INT4 history.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# role tags for SeedSequence keys
_ROLE = {
    "chan_k": 1, "chan_v": 2, "chan_q": 3, "mix_q": 4, "kv": 5, "q": 6,
    "u": 7, "cal_q": 8, "cal_ctx": 9, "pages": 10, "lens": 11, "tags": 12,
    "tagprob": 13, "int4cls": 14, "rows": 15, "tagsens": 16,
}


def rng_for(seed: int, role: str, *idx: int) -> np.random.Generator:
    """A generator keyed by (seed, role, idx...)."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), _ROLE[role], *[int(i) for i in idx]]))


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic decode workload."""
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    group_size: int
    seq_lens: tuple            # per-request context length T (tokens in cache incl. current)
    n_outliers: int            # heavy channels per head
    outlier_scale: tuple       # (lo, hi) of the uniform outlier multiplier; lo == hi -> fixed
    low_var_half: bool         # a seeded half of the other channels scaled by 0.5
    u_kind: str                # "qr" (random Gaussian QR) or "eig" (eigenbasis of covariances)
    paged_shuffle: bool        # page table = seeded permutation of a shared pool
    mixed: bool = False        # INT2/INT4 history (tag classes)
    n_tag_classes: int = 0
    bit_budget: float = 0.0    # average bits per history element the allocation may spend
    fp32_inputs: bool = False  # tiny reference config draws fp32 activations
    cal_tokens: int = 8878     # calibration query count for C_Q
    cal_ctx: int = 4096        # calibration context for C_S

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _ragged_lens(seed: int, batch: int, lo: int, hi: int) -> tuple:
    r = rng_for(seed, "lens")
    return tuple(int(x) for x in r.integers(lo, hi + 1, size=batch))


def workload(n: int, **over) -> Workload:
    """The five decode workloads (1-based index), optionally with fields overridden."""
    if n == 1:
        w = Workload("tiny-ref", 0, 1, 2, 1, 64, 64, (1024,), 4, (20.0, 20.0), False, "qr", False,
                     fp32_inputs=True, cal_tokens=1024, cal_ctx=256)
    elif n == 2:
        w = Workload("qwen3-8b-layer-100k-bs1", 1, 1, 32, 8, 128, 128, (100_000,), 8, (10.0, 30.0), True,
                     "eig", False)
    elif n == 3:
        w = Workload("qwen3-8b-layer-paged-bs32-32k", 2, 32, 32, 8, 128, 128, (32_768,) * 32, 8, (10.0, 30.0),
                     True, "eig", True)
    elif n == 4:
        w = Workload("qwen3-32b-layer-ragged-bs8", 3, 8, 64, 8, 128, 128, _ragged_lens(3, 8, 8192, 131_072), 8,
                     (10.0, 30.0), True, "eig", True)
    elif n == 5:
        w = Workload("mixed-int2-int4-bs16-64k", 4, 16, 32, 8, 128, 128, (65_536,) * 16, 8, (10.0, 30.0), True,
                     "eig", True, mixed=True, n_tag_classes=22, bit_budget=2.6)
    else:
        raise ValueError(f"no workload {n}")
    return dataclasses.replace(w, **over) if over else w


# ---------------------------------------------------------------- channel profiles
def channel_scales(w: Workload, role: str, kv: int) -> np.ndarray:
    """Per-channel standard deviations for one (layer, kv-head): a few heavy outlier
    channels, and (optionally) a low-variance half of the remaining channels."""
    r = rng_for(w.seed, role, kv)
    d = w.head_dim
    s = np.ones(d, dtype=np.float64)
    heavy = r.choice(d, size=w.n_outliers, replace=False)
    lo, hi = w.outlier_scale
    s[heavy] = lo if lo == hi else r.uniform(lo, hi, size=w.n_outliers)
    if w.low_var_half:
        rest = np.setdiff1d(np.arange(d), heavy)
        half = r.choice(rest, size=len(rest) // 2, replace=False)
        s[half] *= 0.5
    return s


def query_mixing(w: Workload, kv: int) -> np.ndarray:
    """A seeded orthogonal channel mixing for the query law of one kv-head (makes the
    query covariance dense). Identity for the tiny reference config."""
    if w.u_kind != "eig":
        return np.eye(w.head_dim)
    return random_orthogonal(rng_for(w.seed, "mix_q", kv), w.head_dim)


def random_orthogonal(r: np.random.Generator, d: int) -> np.ndarray:
    """Haar-distributed orthogonal matrix: QR of a Gaussian with the signs of R's
    diagonal folded into Q."""
    a = r.standard_normal((d, d))
    qm, rm = np.linalg.qr(a)
    return qm * np.sign(np.diag(rm))[None, :]


# ---------------------------------------------------------------- activations
def kv_slice(w: Workload, b: int, kv: int, T: Optional[int] = None, start: int = 0) -> tuple:
    """K, V of request ``b`` and kv-head ``kv`` for positions [start, start+T) as
    float32 arrays [T, d] (values not yet rounded to bf16). Positions are drawn in
    blocks of 4096 tokens so that any window reproduces the same values."""
    if T is None:
        T = w.seq_lens[b] - start
    d = w.head_dim
    sk = channel_scales(w, "chan_k", kv).astype(np.float32)
    sv = channel_scales(w, "chan_v", kv).astype(np.float32)
    K = np.empty((T, d), np.float32)
    V = np.empty((T, d), np.float32)
    blk = 4096
    p = start
    while p < start + T:
        bi = p // blk
        r = rng_for(w.seed, "kv", b, kv, bi)
        zk = r.standard_normal((blk, d), dtype=np.float32)
        zv = r.standard_normal((blk, d), dtype=np.float32)
        lo = p - bi * blk
        n = min(blk - lo, start + T - p)
        K[p - start:p - start + n] = zk[lo:lo + n] * sk
        V[p - start:p - start + n] = zv[lo:lo + n] * sv
        p += n
    return K, V


def query_law(w: Workload, kv: int, z: np.ndarray) -> np.ndarray:
    """Map standard normal draws z [..., d] to the query law of kv-head ``kv``."""
    sq = channel_scales(w, "chan_q", kv)
    return (z * sq) @ query_mixing(w, kv)


def decode_query(w: Workload, b: int) -> np.ndarray:
    """Decode query of request ``b``: float32 [Hq, d]."""
    out = np.empty((w.num_q_heads, w.head_dim), np.float64)
    for h in range(w.num_q_heads):
        kv = h // w.gqa
        z = rng_for(w.seed, "q", b, h).standard_normal(w.head_dim)
        out[h] = query_law(w, kv, z)
    return out.astype(np.float32)


def calibration_queries(w: Workload, kv: int) -> np.ndarray:
    """Calibration queries of the g query heads of kv-head ``kv``: float64 [g, N, d]."""
    r = rng_for(w.seed, "cal_q", kv)
    z = r.standard_normal((w.gqa, w.cal_tokens, w.head_dim))
    return query_law(w, kv, z)


def calibration_context(w: Workload, kv: int) -> tuple:
    """A calibration context (keys, values) of ``cal_ctx`` tokens for kv-head ``kv``,
    drawn from the same per-channel law as the cache: float64 [n, d] each."""
    r = rng_for(w.seed, "cal_ctx", kv)
    sk = channel_scales(w, "chan_k", kv)
    sv = channel_scales(w, "chan_v", kv)
    n = w.cal_ctx
    return r.standard_normal((n, w.head_dim)) * sk, r.standard_normal((n, w.head_dim)) * sv


def random_basis(w: Workload, kv: int, which: str) -> np.ndarray:
    """Seeded random orthogonal basis U (the tiny reference config's recipe)."""
    return random_orthogonal(rng_for(w.seed, "u", kv, 0 if which == "k" else 1), w.head_dim)


# ---------------------------------------------------------------- paging and tags
def page_permutation(seed: int, n_pages: int) -> np.ndarray:
    """A seeded permutation of a shared pool of ``n_pages`` page ids."""
    return rng_for(seed, "pages").permutation(n_pages).astype(np.int32)


def tag_classes(w: Workload, b: int, n_tokens: int) -> np.ndarray:
    """Per-token tag class ids in [0, n_tag_classes) for request ``b`` (categorical with
    seeded Dirichlet(1) class probabilities shared by all requests)."""
    probs = rng_for(w.seed, "tagprob").dirichlet(np.ones(w.n_tag_classes))
    return rng_for(w.seed, "tags", b).choice(w.n_tag_classes, size=n_tokens, p=probs).astype(np.int32)


def tag_class_probs(w: Workload) -> np.ndarray:
    return rng_for(w.seed, "tagprob").dirichlet(np.ones(w.n_tag_classes))


def tag_sensitivity(w: Workload) -> tuple:
    """A seeded synthetic sensitivity table (d2, d4) [n_tag_classes]: the attention-output
    distortion of each tag class stored at 2 and at 4 bits (d2 > d4 > 0, spread over decades,
    standing in for a calibration measurement)."""
    r = rng_for(w.seed, "tagsens")
    d4 = 10.0 ** r.uniform(-4.0, -2.0, w.n_tag_classes)
    d2 = d4 + 10.0 ** r.uniform(-3.0, -0.5, w.n_tag_classes)
    return d2, d4


def tag_nominal_counts(w: Workload, tokens: int = 1_000_000) -> np.ndarray:
    """Expected tokens per tag class in a cache of ``tokens`` tokens (int64)."""
    return np.rint(tag_class_probs(w) * tokens).astype(np.int64)


def standard_rows(seed: int, n: int, d: int, scale: float = 1.0) -> np.ndarray:
    """Plain float32 normal rows [n, d] (quantiser tests)."""
    return (rng_for(seed, "rows", n, d).standard_normal((n, d)) * scale).astype(np.float32)
