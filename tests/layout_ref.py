"""numpy statement of the byte layouts documented in include/oscar.h (test infrastructure).

Written from the header's text, independently of the HIP sources: it packs oracle codes into
pool pages (so the GPU decode can be checked on exactly the oracle's codes) and reads pages
written by the GPU back into canonical per-token codes.
"""
from __future__ import annotations

import numpy as np

PAGE = 16


def qpage_head_bytes(d: int, bits: int) -> int:
    return 4 * d * bits + 128


def bf16_page_head_bytes(d: int) -> int:
    return 64 * d


def key_offsets(d: int, bits: int):
    """(byte offset, bit-in-byte) of the key code of every (slot t, channel ch): arrays [16, d]."""
    t = np.arange(PAGE)[:, None]
    ch = np.arange(d)[None, :]
    kk, g, m, hf = ch // 32, (ch % 32) // 8, (ch % 8) // 2, ch % 2
    lane = 16 * g + t
    cb = d * bits // 32
    if bits == 2:
        word, bit = kk // 2, 8 * (kk % 2) + 2 * m + 16 * hf
    else:
        word, bit = kk, 4 * m + 16 * hf
    part = lane * 2 * cb if bits == 2 else lane * cb     # INT4: all key parts come first
    byte = part + 4 * word + bit // 8
    return np.broadcast_to(byte, (PAGE, d)), np.broadcast_to(bit % 8, (PAGE, d))


def value_offsets(d: int, bits: int):
    t = np.arange(PAGE)[:, None]
    ch = np.arange(d)[None, :]
    nb, c, g, m, hf = ch // 16, ch % 16, t // 4, (t % 4) // 2, t % 2
    lane = 16 * g + c
    cb = d * bits // 32
    if bits == 2:
        word, bit = nb // 4, 2 * (nb % 4) + 8 * m + 16 * hf
    else:
        word, bit = nb // 2, 4 * (nb % 2) + 8 * m + 16 * hf
    part = lane * 2 * cb + cb if bits == 2 else (64 + lane) * cb
    byte = part + 4 * word + bit // 8
    return np.broadcast_to(byte, (PAGE, d)), np.broadcast_to(bit % 8, (PAGE, d))


def pack_page_head(d, bits, codes_k, codes_v, sz_k, sz_v) -> np.ndarray:
    """Page-head bytes from codes [n<=16, d] and (s, z) uint16 [n, 2] of the first n slots."""
    out = np.zeros(qpage_head_bytes(d, bits), np.uint8)
    n = codes_k.shape[0]
    for codes, (byte, bit) in ((codes_k, key_offsets(d, bits)), (codes_v, value_offsets(d, bits))):
        vals = (codes.astype(np.uint16) << bit[:n].astype(np.uint16)).astype(np.uint16)
        lo = (vals & 0xFF).astype(np.uint8)
        np.bitwise_or.at(out, byte[:n].ravel(), lo.ravel())
        hi = (vals >> 8).astype(np.uint8)
        sel = hi.ravel() != 0
        np.bitwise_or.at(out, byte[:n].ravel()[sel] + 1, hi.ravel()[sel])
    meta = np.zeros((PAGE, 4), np.uint16)
    meta[:n, 0:2] = sz_k[:n]
    meta[:n, 2:4] = sz_v[:n]
    out[4 * d * bits:] = meta.view(np.uint8).ravel()
    return out


def unpack_page_head(d, bits, raw):
    """codes_k, codes_v [16, d] and sz_k, sz_v [16, 2] from page-head bytes."""
    raw = np.asarray(raw, np.uint8)
    mask = (1 << bits) - 1
    res = []
    for byte, bit in (key_offsets(d, bits), value_offsets(d, bits)):
        w = raw[byte].astype(np.uint16) | (raw[np.minimum(byte + 1, len(raw) - 1)].astype(np.uint16) << 8)
        res.append(((w >> bit.astype(np.uint16)) & mask).astype(np.uint8))
    meta = raw[4 * d * bits:4 * d * bits + 128].copy().view(np.uint16).reshape(PAGE, 4)
    return res[0], res[1], meta[:, 0:2].copy(), meta[:, 2:4].copy()


def page_addr(page, kv, hkv, d, off4):
    p2 = qpage_head_bytes(d, 2) * hkv
    if page < off4:
        return page * p2 + kv * qpage_head_bytes(d, 2)
    p4 = qpage_head_bytes(d, 4) * hkv
    return off4 * p2 + (page - off4) * p4 + kv * qpage_head_bytes(d, 4)


def write_history(pool, d, hkv, off4, kv, bits, pt_row, codes_k, codes_v, sz_k, sz_v):
    """Write n history slots (slot order) of one (request, kv-head) into pool bytes."""
    n = codes_k.shape[0]
    for j in range((n + PAGE - 1) // PAGE):
        sl = slice(PAGE * j, min(n, PAGE * j + PAGE))
        raw = pack_page_head(d, bits, codes_k[sl], codes_v[sl], sz_k[sl], sz_v[sl])
        a = page_addr(int(pt_row[j]), kv, hkv, d, off4)
        pool[a:a + len(raw)] = raw


def read_history(pool, d, hkv, off4, kv, bits, pt_row, n):
    """Inverse of write_history: codes_k, codes_v [n, d], sz_k, sz_v [n, 2]."""
    ck, cv, sk, sv = [], [], [], []
    for j in range((n + PAGE - 1) // PAGE):
        a = page_addr(int(pt_row[j]), kv, hkv, d, off4)
        k_, v_, s1, s2 = unpack_page_head(d, bits, pool[a:a + qpage_head_bytes(d, bits)])
        m = min(PAGE, n - PAGE * j)
        ck.append(k_[:m]); cv.append(v_[:m]); sk.append(s1[:m]); sv.append(s2[:m])
    if not ck:
        return (np.zeros((0, d), np.uint8),) * 2 + (np.zeros((0, 2), np.uint16),) * 2
    return np.concatenate(ck), np.concatenate(cv), np.concatenate(sk), np.concatenate(sv)


def bf16_key_index(d):
    t = np.arange(PAGE)[:, None]
    ch = np.arange(d)[None, :]
    kk, g, i = ch // 32, (ch % 32) // 8, ch % 8
    return ((g * 16 + t) * (d // 32) + kk) * 8 + i


def bf16_value_index(d):
    t = np.arange(PAGE)[:, None]
    ch = np.arange(d)[None, :]
    nb, c, g, r = ch // 16, ch % 16, t // 4, t % 4
    return 16 * d + ((g * 16 + c) * (d // 16) + nb) * 4 + r


def window_position(j, t, T, sink, recent):
    """Position held by window page j, slot t (or -1), per the header's ring rule."""
    if j < sink // PAGE:
        p = PAGE * j + t
        return p if p < T else -1
    if T <= sink:
        return -1
    s = PAGE * (j - sink // PAGE) + t
    p = T - 1 - ((T - 1 - s) % recent)
    return p if p >= sink else -1


def write_window(win_u16, d, sink, recent, T, K_bits, V_bits):
    """Fill one (request, kv-head) window (uint16 view [W, 32*d]) from bf16 bit patterns
    K_bits, V_bits [T, d]."""
    W = (sink + recent) // PAGE
    ki, vi = bf16_key_index(d), bf16_value_index(d)
    win_u16[:] = 0
    for j in range(W):
        for t in range(PAGE):
            p = window_position(j, t, T, sink, recent)
            if p >= 0:
                win_u16[j, ki[t]] = K_bits[p]
                win_u16[j, vi[t]] = V_bits[p]


def read_window(win_u16, d, sink, recent, T):
    """{position: (k_bits, v_bits)} held by one (request, kv-head) window."""
    W = (sink + recent) // PAGE
    ki, vi = bf16_key_index(d), bf16_value_index(d)
    out = {}
    for j in range(W):
        for t in range(PAGE):
            p = window_position(j, t, T, sink, recent)
            if p >= 0:
                out[p] = (win_u16[j, ki[t]].copy(), win_u16[j, vi[t]].copy())
    return out
