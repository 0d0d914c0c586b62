"""Offline calibration for the library's inputs (not on the decode path): rotations and codebooks.

Every step runs in the library: the covariances C_Q and C_S on the GPU matrix cores, their
eigenvectors and R = U . H . P_br in the host call oscar_rotation_from_covariance ("Together AI
open-sources OSCAR", section on what makes OSCAR different), the Lloyd-Max codebook fit on the GPU.
This module only moves the buffers between those calls.
"""
from __future__ import annotations

import torch


def rotations_on_gpu(q_cal: torch.Tensor, k_ctx: torch.Tensor, v_ctx: torch.Tensor, n_value_queries: int,
                     scale: float) -> tuple:
    """R_K, R_V [Hkv, d, d] fp32 (device) from calibration activations on the GPU: q_cal
    [Hkv, gq, N, d] bf16 queries, k_ctx, v_ctx [Hkv, n, d] bf16 context. C_Q is accumulated over
    all N queries, C_S over the first n_value_queries; R comes from the library's host call."""
    from .ops import calib_query_cov, calib_value_cov, rotation_from_covariance
    cq = calib_query_cov(q_cal)
    cs = calib_value_cov(q_cal[:, :, :n_value_queries].contiguous(), k_ctx, v_ctx, scale)
    rk = rotation_from_covariance(cq.cpu().numpy())
    rv = rotation_from_covariance(cs.cpu().numpy())
    return torch.from_numpy(rk).to(q_cal.device), torch.from_numpy(rv).to(q_cal.device)


def codebooks_on_gpu(k_ctx: torch.Tensor, v_ctx: torch.Tensor, rot_k: torch.Tensor, rot_v: torch.Tensor,
                     clip_k: float = 0.96, clip_v: float = 0.92, max_iter: int = 100, tol: float = 1e-7):
    """INT2 codebook table [Hkv, 2, 4] int16 (device; fp16 level patterns, K then V) from the
    library's Lloyd-Max fit over a calibration context k_ctx, v_ctx [Hkv, n, d] bf16 rotated by
    R_K, R_V. Also returns the fitted levels [Hkv, 2, 4] float64 and iterations [Hkv, 2]."""
    import numpy as np
    from .ops import codebook_fit
    lk, pk, ik = codebook_fit(k_ctx, rot_k, clip_k, max_iter, tol)
    lv, pv, iv = codebook_fit(v_ctx, rot_v, clip_v, max_iter, tol)
    table = torch.from_numpy(np.ascontiguousarray(np.stack([pk, pv], axis=1))).to(k_ctx.device)
    return table, np.stack([lk, lv], axis=1), np.stack([ik, iv], axis=1)
