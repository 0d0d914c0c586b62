"""Lloyd-Max 4-level codebook for the INT2 history (oracle).

The OSCAR overview page (the paragraph that sets OSCAR beside TurboQuant) says only that the
latest OSCAR code pairs the attention-aware rotation with a Lloyd-Max codebook. Everything
else below is a reading, each listed with its reason in the design notes of the repository:

* The codebook replaces the four uniform INT2 levels 0, 1, 2, 3 of the normalised group
  coordinate u = (clip(x) - z) / s by four increasing levels l_0 < l_1 < l_2 < l_3, one
  codebook per (kv-head, K or V). Scale, zero point, clipping and 2-bit packing stay as in the
  uniform codec, and dequantisation is x_hat = z + s * l[code].
* The levels are stored as fp16 values (round to nearest even of the fitted levels).
* Encoding picks the nearest level: code = [u > t_0] + [u >= t_1] + [u > t_2] with the
  decision thresholds t_j = (l_j + l_{j+1}) / 2, exact in fp32 for fp16 levels. A u exactly on
  a threshold goes to the even code, so the levels (0, 1, 2, 3) reproduce the uniform codec's
  round-half-to-even code for code. u is the uniform quantiser's fp32 quotient, taken op by
  op; a group whose stored scale is 0 gets code 0 everywhere.
* Fit: Lloyd-Max (Lloyd's method I; Max, "Quantizing for minimum distortion", 1960), i.e.
  alternate nearest-level cells (thresholds at midpoints) and cell means, on the empirical
  distribution of u over all calibration rows, groups and channels of a kv-head (rotated with
  that head's rotation, clipped with the codec's clip ratio); groups with a zero scale carry
  no u and are left out. Start from the uniform levels (0, 1, 2, 3); an empty cell keeps its
  level; stop when no level moves by more than ``tol`` or after ``max_iter`` iterations. The
  squared error is measured in u (the unit the codebook lives in).

Precision: the fit in fp64; u and the code decisions in fp32 op by op, as the uniform
quantiser takes them.
"""
from __future__ import annotations

import numpy as np

from .quant import bf16_bits, bf16_from_bits

UNIFORM_LEVELS = (0.0, 1.0, 2.0, 3.0)


def fp16_levels(levels) -> np.ndarray:
    """Levels rounded to fp16 (nearest even), returned as fp32 values."""
    return np.asarray(levels, np.float64).astype(np.float16).astype(np.float32)


def fp16_patterns(levels) -> np.ndarray:
    """16-bit fp16 patterns of the levels (nearest even)."""
    return np.asarray(levels, np.float64).astype(np.float16).view(np.uint16)


def thresholds_fp32(levels_fp16) -> np.ndarray:
    """Decision thresholds t_j = (l_j + l_{j+1}) / 2 of fp16-valued levels, in fp32 (both the
    sum and the halving are exact for fp16 inputs)."""
    lv = np.asarray(levels_fp16, np.float32)
    return ((lv[:-1] + lv[1:]) * np.float32(0.5)).astype(np.float32)


def code_of_coordinate(u, levels_fp16) -> np.ndarray:
    """Nearest-level code of fp32 coordinates u, ties to the even code."""
    u = np.asarray(u, np.float32)
    t = thresholds_fp32(levels_fp16)
    c = (u > t[0]).astype(np.uint8) + (u >= t[1]).astype(np.uint8) + (u > t[2]).astype(np.uint8)
    return c


def _grids(x, group: int, clip: float):
    """Per-group grid of the uniform INT2 quantiser, fp32 op by op: (groups view, lo, hi, s, z,
    s_bits, z_bits)."""
    x = np.asarray(x, dtype=np.float32)
    n, d = x.shape
    if d % group:
        raise ValueError("group must divide the row length")
    g = x.reshape(n, d // group, group)
    c = np.float32(clip)
    lo = (c * g.min(axis=2, keepdims=True)).astype(np.float32)
    hi = (c * g.max(axis=2, keepdims=True)).astype(np.float32)
    s32 = ((hi - lo).astype(np.float32) / np.float32(3.0)).astype(np.float32)
    s_b = bf16_bits(s32)
    z_b = bf16_bits(lo)
    return g, lo, hi, bf16_from_bits(s_b), bf16_from_bits(z_b), s_b, z_b


def group_coordinates(x, group: int, clip: float):
    """u = fl(fl(clip(x) - z) / s) of rotated fp32 rows [n, d], the quantiser's own quotient.
    Returns (u [n, d] fp32, valid [n, d] bool: False where the group's stored scale is 0)."""
    g, lo, hi, s, z, _, _ = _grids(x, group, clip)
    xc = np.minimum(np.maximum(g, lo), hi)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = ((xc - z).astype(np.float32) / s).astype(np.float32)
    valid = np.broadcast_to(s != np.float32(0.0), g.shape)
    n, d = np.asarray(x).shape
    return u.reshape(n, d), valid.reshape(n, d).copy()


def quantize_rows_codebook(x, group: int, clip: float, levels_fp16):
    """INT2 codes of rotated fp32 rows [n, d] under the codebook. Returns codes uint8 [n, d]
    and sz uint16 [n, d/group, 2] with (s, z) bf16 patterns, as ``quantize_rows``."""
    g, lo, hi, s, z, s_b, z_b = _grids(x, group, clip)
    u, valid = group_coordinates(x, group, clip)
    code = np.where(valid, code_of_coordinate(np.where(valid, u, 0.0), levels_fp16), 0).astype(np.uint8)
    sz = np.stack([s_b[..., 0], z_b[..., 0]], axis=-1)
    return code, sz


def dequantize_rows_codebook(codes, sz, group: int, levels_fp16) -> np.ndarray:
    """x_hat = z + s * l[code] (fp64), rows [n, d] with (s, z) per group."""
    lv = np.asarray(levels_fp16, np.float64)
    codes = np.asarray(codes, np.int64)
    n, d = codes.shape
    s = bf16_from_bits(sz[..., 0]).astype(np.float64)
    z = bf16_from_bits(sz[..., 1]).astype(np.float64)
    g = lv[codes].reshape(n, d // group, group)
    return (g * s[..., None] + z[..., None]).reshape(n, d)


def lloyd_max(samples, init=UNIFORM_LEVELS, max_iter: int = 100, tol: float = 1e-7):
    """Lloyd-Max iteration on 1-D samples (fp64). Each iteration puts the thresholds at the
    midpoints of the current levels, assigns every sample to its cell (a sample on a threshold
    goes to the even level, as the encoder decides) and moves each level to its cell's mean
    (an empty cell keeps its level). Stops when no level moved by more than ``tol``.

    Returns (levels fp64 [4], iterations run, list of the mean squared error before each
    iteration's update and after the last)."""
    x = np.asarray(samples, np.float64).ravel()
    lv = np.asarray(init, np.float64).copy()
    if lv.shape != (4,) or not np.all(np.diff(lv) > 0):
        raise ValueError("four increasing initial levels are required")
    mse = []
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (lv[:-1] + lv[1:])
        cell = (x > t[0]).astype(np.int64) + (x >= t[1]) + (x > t[2])
        mse.append(float(np.mean((x - lv[cell]) ** 2)) if x.size else 0.0)
        new = lv.copy()
        for j in range(4):
            m = cell == j
            if m.any():
                new[j] = x[m].sum() / m.sum()
        moved = np.max(np.abs(new - lv))
        lv = new
        if moved <= tol:
            break
    t = 0.5 * (lv[:-1] + lv[1:])
    cell = (x > t[0]).astype(np.int64) + (x >= t[1]) + (x > t[2])
    mse.append(float(np.mean((x - lv[cell]) ** 2)) if x.size else 0.0)
    return lv, it, mse


def fit_codebook(x_rot, group: int, clip: float, init=UNIFORM_LEVELS, max_iter: int = 100, tol: float = 1e-7):
    """Codebook of one kv-head from its rotated fp32 calibration rows [n, d]: Lloyd-Max on the
    group coordinates. Returns (levels fp64 [4], fp16-valued levels fp32 [4], iterations)."""
    u, valid = group_coordinates(x_rot, group, clip)
    lv, it, _ = lloyd_max(u[valid], init, max_iter, tol)
    return lv, fp16_levels(lv), it
