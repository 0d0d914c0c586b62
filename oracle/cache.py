"""Three-region KV cache and decode-step semantics (oracle).

Follows the OSCAR news article (section "serving system: mixed-precision cache layout"):
per request the first 64 tokens (sink) and the last 256 tokens (recent) stay in BF16 and
every token in between (history) is stored in INT2 after the OSCAR rotation and clipping.
The OSCAR overview page (method paragraph) and the study note (SGLang case) give the step:
a new token is written into the BF16 recent window, and as decoding advances the oldest
recent token is rotated, clipped, quantised, packed and demoted into the INT2 history.

Readings where the pages are silent:
* The recent window includes the current token: for T tokens in cache the segments are
  sink [0, min(T, 64)), recent [max(64, T-256), T), history [64, T-256) when T > 320.
* K and V enter the cache as bf16 (round to nearest even), since every history token
  passes through the BF16 recent window first.
* One decode step with T tokens in cache and T >= 320: demote position T-256 into the
  history, then append the new token at position T (it takes the freed recent slot).
* Mixed INT2/INT4 history (TriAxialKV reading note, section 4): each token carries a bit
  width chosen when it is created; it is quantised at that width when demoted, with the
  INT4 clip ratio (1.0 unless given, since TriAxialKV names no clipping).
* Optional Lloyd-Max codebooks (``codebook.py``): per kv-head four fp16 levels for K and for
  V replace the uniform INT2 levels; INT4 tokens keep the uniform levels.
"""
from __future__ import annotations

import numpy as np

from .quant import bf16_round, rotate_rows_fp32, quantize_rows, dequantize_rows
from .codebook import quantize_rows_codebook, dequantize_rows_codebook

SINK = 64
RECENT = 256


def segments(T: int, sink: int = SINK, recent: int = RECENT):
    """Position ranges (start, end) of the sink, history and recent segments for T
    tokens in cache. The three lengths sum to T."""
    s_end = min(T, sink)
    r_start = min(max(sink, T - recent), T)
    h_start, h_end = sink, max(sink, r_start)
    if h_end == h_start:
        h_start = h_end = min(T, sink)
    return (0, s_end), (h_start, h_end), (r_start, T)


def effective_bits(T: int, group: int, bits: int = 2, meta_bits: int = 32,
                   sink: int = SINK, recent: int = RECENT) -> float:
    """Average stored bits per KV element for a cache of T tokens: history elements cost
    ``bits`` plus ``meta_bits`` per group of ``group`` elements (scale + zero), sink and
    recent elements cost 16 bits."""
    (s0, s1), (h0, h1), (r0, r1) = segments(T, sink, recent)
    n_hist = h1 - h0
    n_bf16 = T - n_hist
    return (n_hist * (bits + meta_bits / group) + n_bf16 * 16.0) / T


class OracleCache:
    """The cache of one request: BF16 rows for sink/recent positions and quantised rows
    (rotated space) for history positions, for every kv-head."""

    def __init__(self, rot_k32, rot_v32, group: int, clip_k: float = 0.96, clip_v: float = 0.92,
                 clip_k4: float = 1.0, clip_v4: float = 1.0, sink: int = SINK, recent: int = RECENT,
                 codebook_k=None, codebook_v=None):
        self.rot_k = np.asarray(rot_k32, dtype=np.float32)   # [Hkv, d, d]
        self.rot_v = np.asarray(rot_v32, dtype=np.float32)
        self.hkv, self.d = self.rot_k.shape[0], self.rot_k.shape[1]
        self.group = group
        self.clip = {2: (clip_k, clip_v), 4: (clip_k4, clip_v4)}
        self.sink, self.recent = sink, recent
        # INT2 codebooks [Hkv, 4] (fp16-valued levels), or None for the uniform levels
        self.codebook = {"k": None if codebook_k is None else np.asarray(codebook_k, np.float32),
                         "v": None if codebook_v is None else np.asarray(codebook_v, np.float32)}
        self.T = 0
        self.bf16_k = {}    # pos -> [Hkv, d] float32 (bf16 values)
        self.bf16_v = {}
        self.bits = {}      # pos -> bit width used when the position is demoted
        ng = self.d // group
        self.hist_pos = np.zeros(0, np.int64)
        self.hist_bits = np.zeros(0, np.int64)
        self.k_codes = np.zeros((self.hkv, 0, self.d), np.uint8)
        self.v_codes = np.zeros((self.hkv, 0, self.d), np.uint8)
        self.k_sz = np.zeros((self.hkv, 0, ng, 2), np.uint16)
        self.v_sz = np.zeros((self.hkv, 0, ng, 2), np.uint16)

    # ------------------------------------------------------------ quantisation of rows
    def quantize_tokens(self, k_rows, v_rows, bits: int):
        """k_rows, v_rows [Hkv, n, d] bf16-valued -> codes/sz for K and V (rotated space)."""
        ck, cv = self.clip.get(bits, (1.0, 1.0))
        kc, ks, vc, vs = [], [], [], []
        for h in range(self.hkv):
            c, s = self._quantize(rotate_rows_fp32(k_rows[h], self.rot_k[h]), bits, ck, "k", h)
            kc.append(c); ks.append(s)
            c, s = self._quantize(rotate_rows_fp32(v_rows[h], self.rot_v[h]), bits, cv, "v", h)
            vc.append(c); vs.append(s)
        return np.stack(kc), np.stack(ks), np.stack(vc), np.stack(vs)

    def _quantize(self, x, bits, clip, which, h):
        cb = self.codebook[which]
        if bits == 2 and cb is not None:
            return quantize_rows_codebook(x, self.group, clip, cb[h])
        return quantize_rows(x, self.group, bits, clip)

    def history_rows(self, kv: int):
        """Dequantised history rows (rotated basis) of a kv-head: (K_hat, V_hat) fp64 [n, d]."""
        out = []
        for which, codes, sz in (("k", self.k_codes, self.k_sz), ("v", self.v_codes, self.v_sz)):
            x = dequantize_rows(codes[kv], sz[kv], self.group)
            cb = self.codebook[which]
            sel = self.hist_bits == 2
            if cb is not None and sel.any():
                x[sel] = dequantize_rows_codebook(codes[kv][sel], sz[kv][sel], self.group, cb[kv])
            out.append(x)
        return out[0], out[1]

    def _push_history(self, pos, bits, kc, ks, vc, vs):
        self.hist_pos = np.concatenate([self.hist_pos, np.asarray(pos, np.int64)])
        self.hist_bits = np.concatenate([self.hist_bits, np.asarray(bits, np.int64)])
        self.k_codes = np.concatenate([self.k_codes, kc], axis=1)
        self.k_sz = np.concatenate([self.k_sz, ks], axis=1)
        self.v_codes = np.concatenate([self.v_codes, vc], axis=1)
        self.v_sz = np.concatenate([self.v_sz, vs], axis=1)

    # ------------------------------------------------------------ step semantics
    def append(self, k, v, bits: int = 2):
        """One decode step's cache update: demote the oldest recent token if the window is
        full, then store the new token (k, v: [Hkv, d]) in BF16 at position T."""
        T = self.T
        if T >= self.sink + self.recent:
            self.demote(T - self.recent)
        self.bf16_k[T] = bf16_round(np.asarray(k, np.float32))
        self.bf16_v[T] = bf16_round(np.asarray(v, np.float32))
        self.bits[T] = bits
        self.T = T + 1

    def demote(self, pos: int):
        """Rotate, clip, quantise and move BF16 position ``pos`` into the history."""
        b = self.bits[pos]
        k = self.bf16_k.pop(pos)[:, None, :]
        v = self.bf16_v.pop(pos)[:, None, :]
        kc, ks, vc, vs = self.quantize_tokens(k, v, b)
        self._push_history([pos], [b], kc, ks, vc, vs)

    @classmethod
    def from_prefix(cls, K, V, rot_k32, rot_v32, group, bits=None, **kw):
        """The cache after T tokens (K, V [Hkv, T, d]), built segment by segment; it equals
        appending the T tokens one at a time. ``bits`` [T] gives each token's width."""
        c = cls(rot_k32, rot_v32, group, **kw)
        K = np.asarray(K, np.float32)
        V = np.asarray(V, np.float32)
        T = K.shape[1]
        bits = np.full(T, 2, np.int64) if bits is None else np.asarray(bits, np.int64)
        (s0, s1), (h0, h1), (r0, r1) = segments(T, c.sink, c.recent)
        for p in list(range(s0, s1)) + list(range(r0, r1)):
            c.bf16_k[p] = bf16_round(K[:, p])
            c.bf16_v[p] = bf16_round(V[:, p])
        for p in range(T):
            c.bits[p] = int(bits[p])
        for b in sorted(set(int(x) for x in bits[h0:h1])):
            pos = np.arange(h0, h1)[bits[h0:h1] == b]
            if len(pos):
                kc, ks, vc, vs = c.quantize_tokens(bf16_round(K[:, pos]), bf16_round(V[:, pos]), b)
                c._push_history(pos, np.full(len(pos), b), kc, ks, vc, vs)
        c.T = T
        return c

    # ------------------------------------------------------------ views
    def bf16_positions(self):
        return sorted(self.bf16_k.keys())

    def bf16_rows(self, kv: int):
        pos = self.bf16_positions()
        if not pos:
            return np.zeros((0, self.d)), np.zeros((0, self.d)), pos
        return (np.stack([self.bf16_k[p][kv] for p in pos]).astype(np.float64),
                np.stack([self.bf16_v[p][kv] for p in pos]).astype(np.float64), pos)
