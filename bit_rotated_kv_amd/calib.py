"""Offline rotation construction for the library's inputs (not on the decode path).

R = U . H . P_br, with U the eigenvectors (descending eigenvalue) of an attention covariance:
the query covariance C_Q = (1/N) sum q^T q for keys, the score-weighted value covariance
C_S = (1/N) (S V)^T (S V) for values ("Together AI open-sources OSCAR", section on what makes
OSCAR different). H is the orthonormal Sylvester Hadamard matrix and P_br the bit-reversal
permutation (P[i, rev(i)] = 1). Computed once, in float64 on the host, shipped as fp32.
"""
from __future__ import annotations

import torch


def sylvester_hadamard(d: int) -> torch.Tensor:
    if d < 1 or d & (d - 1):
        raise ValueError("head_dim must be a power of two")
    h = torch.ones(1, 1, dtype=torch.float64)
    base = torch.tensor([[1.0, 1.0], [1.0, -1.0]], dtype=torch.float64)
    while h.shape[0] < d:
        h = torch.kron(base, h)
    return h / d ** 0.5


def bit_reversal(d: int) -> torch.Tensor:
    bits = d.bit_length() - 1
    idx = torch.arange(d)
    rev = torch.zeros(d, dtype=torch.long)
    for b in range(bits):
        rev |= ((idx >> b) & 1) << (bits - 1 - b)
    return rev


def bit_reversal_matrix(d: int) -> torch.Tensor:
    p = torch.zeros(d, d, dtype=torch.float64)
    p[torch.arange(d), bit_reversal(d)] = 1.0
    return p


def eigvecs_descending(cov: torch.Tensor) -> torch.Tensor:
    w, u = torch.linalg.eigh(cov.to(torch.float64))
    u = u.flip(1)
    sign = torch.sign(u.gather(0, u.abs().argmax(0, keepdim=True)))
    sign[sign == 0] = 1.0
    return u * sign


def rotation(u: torch.Tensor) -> torch.Tensor:
    """fp32 R = U . H . P_br."""
    d = u.shape[0]
    return (u.to(torch.float64) @ sylvester_hadamard(d) @ bit_reversal_matrix(d)).to(torch.float32)


def query_covariance(q: torch.Tensor) -> torch.Tensor:
    """q [g, N, d] (the g query heads of a kv-head) -> sum over heads of q_h^T q_h / N."""
    q = q.to(torch.float64)
    if q.dim() == 2:
        q = q[None]
    return torch.einsum("hni,hnj->ij", q, q) / q.shape[1]


def value_covariance(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float) -> torch.Tensor:
    """C_S for calibration queries q [g, N, d] over a context (k, v [n, d])."""
    q = q.to(torch.float64)
    if q.dim() == 2:
        q = q[None]
    s = torch.softmax(scale * q @ k.to(torch.float64).T, dim=-1)
    sv = s @ v.to(torch.float64)
    return torch.einsum("hni,hnj->ij", sv, sv) / q.shape[1]


def rotations_on_gpu(q_cal: torch.Tensor, k_ctx: torch.Tensor, v_ctx: torch.Tensor, n_value_queries: int,
                     scale: float) -> tuple:
    """R_K, R_V [Hkv, d, d] fp32 (device) from calibration activations on the GPU: q_cal
    [Hkv, gq, N, d] bf16 queries, k_ctx, v_ctx [Hkv, n, d] bf16 context. The covariances are
    accumulated on the matrix cores (C_Q over all N queries, C_S over the first n_value_queries);
    their eigenvectors and R = U . H . P_br are formed on the host in float64."""
    from .ops import calib_query_cov, calib_value_cov
    cq = calib_query_cov(q_cal).double().cpu()
    cs = calib_value_cov(q_cal[:, :, :n_value_queries].contiguous(), k_ctx, v_ctx, scale).double().cpu()
    rk = torch.stack([rotation(eigvecs_descending(c)) for c in cq])
    rv = torch.stack([rotation(eigvecs_descending(c)) for c in cs])
    return rk.to(q_cal.device), rv.to(q_cal.device)


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
