"""Clip, group quantisation, packing (oracle).

Follows the OSCAR overview page (method paragraph): the oldest recent token is rotated,
clipped, quantised and packed into the INT2 history, four 2-bit values per byte, and the
INT2 kernel restores values from the scale and zero point. Clip constants come from the
OSCAR study note, case 2 (c_K ~ 0.96, c_V ~ 0.92).

Readings where the pages are silent (each one is listed with its reason in the design
notes of the repository):
* Clip: per group, lo = c * min(x), hi = c * max(x) (the clip ratio scales both ends).
* Asymmetric quantiser with a float zero point: s = (hi - lo) / (2^b - 1), z = lo, both
  stored as bf16 (round to nearest even); codes use the stored (bf16) s and z.
* code = clamp(round_half_even((clamp(x, lo, hi) - z) / s), 0, 2^b - 1); if the stored s
  is 0 every code is 0.
* Dequantisation x_hat = s * code + z.
* Packing is LSB first: 2-bit code i of a byte sits at bits 2i..2i+1; 4-bit code i at
  bits 4i..4i+3.

The integer decisions are taken in fp32 op by op (numpy float32 arithmetic is IEEE
single with round-to-nearest-even and never fuses a multiply-add).
"""
from __future__ import annotations

import numpy as np


def bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even) and return the 16-bit
    patterns. Finite inputs only."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    """fp32 values of 16-bit bf16 patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """fp32 -> nearest bf16 value (as fp32)."""
    return bf16_from_bits(bf16_bits(x))


def rotate_rows_fp32(x, r32) -> np.ndarray:
    """x_rot = fp32(x . R): the product taken in fp64 from the given values and rounded
    once to fp32. ``x`` [n, d] (e.g. bf16-valued keys), ``r32`` the fp32 rotation."""
    return (np.asarray(x, dtype=np.float64) @ np.asarray(r32, dtype=np.float64)).astype(np.float32)


def quantize_group(x, bits: int, clip: float):
    """Quantise one group (1-D fp32 array). Returns (codes uint8, s_bits, z_bits)."""
    x = np.asarray(x, dtype=np.float32)
    c = np.float32(clip)
    levels = np.float32((1 << bits) - 1)
    mn = x.min()
    mx = x.max()
    lo = np.float32(c * mn)
    hi = np.float32(c * mx)
    s32 = np.float32(np.float32(hi - lo) / levels)
    s_b = bf16_bits(s32)[()]
    z_b = bf16_bits(lo)[()]
    s = bf16_from_bits(s_b)[()]
    z = bf16_from_bits(z_b)[()]
    if s == np.float32(0.0):
        return np.zeros(x.shape, np.uint8), s_b, z_b
    xc = np.minimum(np.maximum(x, lo), hi)
    t = np.float32(np.float32(xc - z) / s)
    code = np.clip(np.rint(t), 0, levels).astype(np.uint8)
    return code, s_b, z_b


def quantize_rows(x, group: int, bits: int, clip: float):
    """Quantise rows [n, d] group by group along the last axis (vectorised form of
    ``quantize_group``; same fp32 operations in the same order).

    Returns codes uint8 [n, d] and sz uint16 [n, d/group, 2] holding (s, z) bf16 patterns."""
    x = np.asarray(x, dtype=np.float32)
    n, d = x.shape
    if d % group:
        raise ValueError("group must divide the row length")
    g = x.reshape(n, d // group, group)
    c = np.float32(clip)
    levels = np.float32((1 << bits) - 1)
    mn = g.min(axis=2, keepdims=True)
    mx = g.max(axis=2, keepdims=True)
    lo = (c * mn).astype(np.float32)
    hi = (c * mx).astype(np.float32)
    s32 = ((hi - lo).astype(np.float32) / levels).astype(np.float32)
    s_b = bf16_bits(s32)
    z_b = bf16_bits(lo)
    s = bf16_from_bits(s_b)
    z = bf16_from_bits(z_b)
    xc = np.minimum(np.maximum(g, lo), hi)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = ((xc - z).astype(np.float32) / s).astype(np.float32)
    code = np.clip(np.rint(t), 0, levels)
    code = np.where(s == np.float32(0.0), 0.0, code).astype(np.uint8)
    sz = np.stack([s_b[..., 0], z_b[..., 0]], axis=-1)
    return code.reshape(n, d), sz


def pack_codes(codes, bits: int) -> np.ndarray:
    """Pack codes [n, d] LSB first: 4 two-bit codes or 2 four-bit codes per byte."""
    codes = np.asarray(codes, dtype=np.uint8)
    per = 8 // bits
    n, d = codes.shape
    if d % per:
        raise ValueError("row length must be a multiple of codes per byte")
    c = codes.reshape(n, d // per, per).astype(np.uint16)
    out = np.zeros((n, d // per), np.uint16)
    for i in range(per):
        out |= c[:, :, i] << (bits * i)
    return out.astype(np.uint8)


def unpack_codes(packed, bits: int, d: int) -> np.ndarray:
    """Inverse of ``pack_codes``."""
    packed = np.asarray(packed, dtype=np.uint8)
    per = 8 // bits
    mask = (1 << bits) - 1
    out = np.zeros((packed.shape[0], d), np.uint8)
    for i in range(per):
        out[:, i::per] = (packed >> (bits * i)) & mask
    return out


def dequantize_rows(codes, sz, group: int) -> np.ndarray:
    """x_hat = s * code + z (fp64), rows [n, d] with (s, z) per group."""
    codes = np.asarray(codes, dtype=np.float64)
    n, d = codes.shape
    s = bf16_from_bits(sz[..., 0]).astype(np.float64)
    z = bf16_from_bits(sz[..., 1]).astype(np.float64)
    g = codes.reshape(n, d // group, group)
    return (g * s[..., None] + z[..., None]).reshape(n, d)
