"""Seeded decode problems for the GPU parity tests (test infrastructure).

Inputs come from ``synth``; rotations, caches and expected outputs from ``oracle``; device
buffers are filled either by the library (GPU-written cache) or from the oracle's codes through
``layout_ref`` (oracle-written cache). Nothing here reads a value produced by the HIP path
into an expected value.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import layout_ref
import oracle
import synth


@dataclasses.dataclass
class Problem:
    w: synth.Workload
    K: list            # per request [Hkv, T, d] float32 (raw draws)
    V: list
    q: np.ndarray      # [B, Hq, d] float32
    rot_k: np.ndarray  # [Hkv, d, d] float32
    rot_v: np.ndarray
    bits: list         # per request [T] int (2/4)
    caches: list       # per request oracle.OracleCache
    mixed: bool
    pages2: int
    pages4: int
    order2: np.ndarray
    order4: np.ndarray
    codebook: np.ndarray = None   # [Hkv, 2, 4] fp16-valued INT2 levels (K, V), or None (uniform)


def rotations(w: synth.Workload):
    rk, rv = [], []
    for kv in range(w.num_kv_heads):
        if w.u_kind == "qr":
            uk, uv = synth.random_basis(w, kv, "k"), synth.random_basis(w, kv, "v")
        else:
            qc = synth.calibration_queries(w, kv)
            uk = oracle.eigenbasis(oracle.query_covariance(qc))
            kc, vc = synth.calibration_context(w, kv)
            uv = oracle.eigenbasis(oracle.score_weighted_value_covariance(qc[:, :1024], kc, vc,
                                                                          1.0 / np.sqrt(w.head_dim)))
        rk.append(oracle.rotation_fp32(oracle.compose_rotation(uk)))
        rv.append(oracle.rotation_fp32(oracle.compose_rotation(uv)))
    return np.stack(rk), np.stack(rv)


def fit_codebooks(w: synth.Workload, rk: np.ndarray, rv: np.ndarray) -> np.ndarray:
    """INT2 codebooks [Hkv, 2, 4] (fp16 values): the oracle's Lloyd-Max fit on the workload's
    calibration context, rotated per kv-head, with the INT2 clip ratios."""
    out = np.zeros((w.num_kv_heads, 2, 4), np.float32)
    for kv in range(w.num_kv_heads):
        kc, vc = synth.calibration_context(w, kv)
        for j, (x, r, clip) in enumerate(((kc, rk[kv], 0.96), (vc, rv[kv], 0.92))):
            xr = oracle.rotate_rows_fp32(oracle.bf16_round(x.astype(np.float32)), r)
            out[kv, j] = oracle.fit_codebook(xr, w.group_size, clip)[1]
    return out


def codebook_patterns(cb: np.ndarray) -> np.ndarray:
    """fp16 bit patterns [Hkv, 2, 4] as int16 (the library's codebook table)."""
    return oracle.fp16_patterns(cb).view(np.int16)


def class_bits(w: synth.Workload) -> np.ndarray:
    """Bits of each tag class: the oracle's TriAxialKV greedy over the workload's sensitivity table,
    nominal class counts and bit budget."""
    d2, d4 = synth.tag_sensitivity(w)
    return oracle.greedy_bit_allocation(d2, d4, synth.tag_nominal_counts(w), w.bit_budget)


def token_bits(w: synth.Workload, b: int, T: int) -> np.ndarray:
    if not w.mixed:
        return np.full(T, 2, np.int64)
    return class_bits(w)[synth.tag_classes(w, b, T)].astype(np.int64)


def make_problem(w: synth.Workload, shuffle: bool = True, with_oracle: bool = True, codebook=None) -> Problem:
    """``codebook``: None (uniform INT2 levels), "fit" (``fit_codebooks``) or a [Hkv, 2, 4] array."""
    B = w.batch
    K, V, bits = [], [], []
    for b in range(B):
        T = w.seq_lens[b]
        ks, vs = [], []
        for kv in range(w.num_kv_heads):
            k_, v_ = synth.kv_slice(w, b, kv, T)
            ks.append(k_); vs.append(v_)
        K.append(np.stack(ks) if T else np.zeros((w.num_kv_heads, 0, w.head_dim), np.float32))
        V.append(np.stack(vs) if T else np.zeros((w.num_kv_heads, 0, w.head_dim), np.float32))
        bits.append(token_bits(w, b, T))
    q = np.stack([synth.decode_query(w, b) for b in range(B)])
    rk, rv = rotations(w)
    if isinstance(codebook, str):
        codebook = fit_codebooks(w, rk, rv)
    cbk = None if codebook is None else codebook[:, 0]
    cbv = None if codebook is None else codebook[:, 1]
    caches = []
    if with_oracle:
        for b in range(B):
            caches.append(oracle.OracleCache.from_prefix(K[b], V[b], rk, rv, w.group_size, bits=bits[b],
                                                         codebook_k=cbk, codebook_v=cbv))
    n2 = [max(0, T - 320) - int((bits[b][64:max(64, T - 256)] == 4).sum()) for b, T in enumerate(w.seq_lens)]
    n4 = [int((bits[b][64:max(64, T - 256)] == 4).sum()) for b, T in enumerate(w.seq_lens)]
    pages2 = max([(n + 15) // 16 for n in n2] + [1])
    pages4 = max([(n + 15) // 16 for n in n4] + [1]) if w.mixed else 0
    r = np.random.default_rng(w.seed + 1000)
    order2 = r.permutation(B * pages2) if shuffle else np.arange(B * pages2)
    order4 = r.permutation(max(B * pages4, 0)) if shuffle else np.arange(B * pages4)
    return Problem(w, K, V, q, rk, rv, bits, caches, w.mixed, pages2, pages4, order2, order4, codebook)


def max_len(p: Problem) -> int:
    return max(p.w.seq_lens) if p.w.seq_lens else 0


def kv_bits_tensor(p: Problem, which: str) -> np.ndarray:
    """[B, Hkv, Tmax, d] uint16 bf16 bit patterns of K or V (zero padded)."""
    w = p.w
    tm = max(max_len(p), 1)
    out = np.zeros((w.batch, w.num_kv_heads, tm, w.head_dim), np.uint16)
    src = p.K if which == "k" else p.V
    for b in range(w.batch):
        T = w.seq_lens[b]
        if T:
            out[b, :, :T] = oracle.bf16_bits(src[b])
    return out


def bits_tensor(p: Problem) -> np.ndarray:
    tm = max(max_len(p), 1)
    out = np.full((p.w.batch, tm), 2, np.uint8)
    for b in range(p.w.batch):
        out[b, :p.w.seq_lens[b]] = p.bits[b]
    return out


def oracle_history(cache: oracle.OracleCache, kv: int, bits: int):
    """Oracle history entries of one width in slot order (= position order)."""
    sel = np.where(cache.hist_bits == bits)[0]
    sel = sel[np.argsort(cache.hist_pos[sel], kind="stable")]
    return cache.k_codes[kv, sel], cache.v_codes[kv, sel], cache.k_sz[kv, sel, 0], cache.v_sz[kv, sel, 0]


def oracle_pool_and_window(p: Problem, layout, pt2: np.ndarray, pt4, pool_nbytes: int, window_nbytes: int):
    """Pool and window bytes holding exactly the oracle caches (packed by layout_ref)."""
    w = p.w
    d, hkv = w.head_dim, w.num_kv_heads
    off4 = layout.int4_page_offset if p.mixed else layout.pool_pages
    pool = np.zeros(pool_nbytes, np.uint8)
    W = (64 + 256) // 16
    win = np.zeros((w.batch, hkv, W, 32 * d), np.uint16)
    kb, vb = kv_bits_tensor(p, "k"), kv_bits_tensor(p, "v")
    for b in range(w.batch):
        T = w.seq_lens[b]
        c = p.caches[b]
        for kv in range(hkv):
            layout_ref.write_window(win[b, kv], d, 64, 256, T, kb[b, kv], vb[b, kv])
            for bits, pt in ((2, pt2), (4, pt4)):
                if bits == 4 and not p.mixed:
                    continue
                ck, cv, sk, sv = oracle_history(c, kv, bits)
                if len(ck):
                    layout_ref.write_history(pool, d, hkv, off4, kv, bits, pt[b], ck, cv, sk, sv)
    return pool, win.view(np.uint8).reshape(-1)[:window_nbytes]


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)
