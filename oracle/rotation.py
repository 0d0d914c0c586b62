"""Offline rotation construction (oracle, fp64).

Follows the OSCAR news article ("Together AI open-sources OSCAR", section on what makes
OSCAR different): keys are rotated by the eigenbasis U_Q of the query covariance
C_Q = (1/N) sum_n q_n^T q_n, values by the eigenbasis U_S of the score-weighted value
covariance C_S = (1/N) V^T S^T S V, and the composed rotations are
R_K = U_Q . H_Had . P_br and R_V = U_S . H_Had . P_br.

Readings where the pages are silent:
* H_Had is the Sylvester Hadamard matrix of full head_dim size, scaled by 1/sqrt(d) so it
  is orthogonal.
* P_br is the bit-reversal permutation matrix, P[i, rev(i)] = 1.
* Under GQA the key covariance sums the covariances of the query heads sharing the
  kv-head (summing the logit-error identity over those heads gives that weight).
* Eigenvectors are sorted by descending eigenvalue and each column's sign is fixed so its
  largest-magnitude entry is positive (the order and signs do not change the method).
* Row-vector convention: a key row x is rotated as x . R.
"""
from __future__ import annotations

import numpy as np


def hadamard(d: int) -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix H_d / sqrt(d) (H_1 = [1], H_2n = [[H, H], [H, -H]])."""
    if d < 1 or d & (d - 1):
        raise ValueError("Hadamard size must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def bitrev_indices(d: int) -> np.ndarray:
    """rev(i): the log2(d)-bit reversal of each index i in [0, d)."""
    m = d.bit_length() - 1
    if 1 << m != d:
        raise ValueError("bit reversal needs a power of two")
    out = np.zeros(d, dtype=np.int64)
    for i in range(d):
        r = 0
        for b in range(m):
            if i >> b & 1:
                r |= 1 << (m - 1 - b)
        out[i] = r
    return out


def bitrev_matrix(d: int) -> np.ndarray:
    """Permutation matrix P_br with P[i, rev(i)] = 1."""
    p = np.zeros((d, d))
    p[np.arange(d), bitrev_indices(d)] = 1.0
    return p


def query_covariance(q_cal: np.ndarray) -> np.ndarray:
    """C_Q = (1/N) sum_n q_n^T q_n over calibration queries.

    ``q_cal`` is [N, d] for one query head, or [g, N, d] for the g query heads that share a
    kv-head, in which case the per-head covariances are summed."""
    q = np.asarray(q_cal, dtype=np.float64)
    if q.ndim == 2:
        q = q[None]
    n = q.shape[1]
    c = np.zeros((q.shape[2], q.shape[2]))
    for h in range(q.shape[0]):
        c += q[h].T @ q[h]
    return c / n


def score_weighted_value_covariance(q_cal: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray,
                                    scale: float) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V with S = softmax(scale * Q K^T) (rows over the context).

    ``q_cal`` is [N, d] or [g, N, d] (summed over heads as for C_Q)."""
    q = np.asarray(q_cal, dtype=np.float64)
    if q.ndim == 2:
        q = q[None]
    k = np.asarray(k_ctx, dtype=np.float64)
    v = np.asarray(v_ctx, dtype=np.float64)
    n = q.shape[1]
    c = np.zeros((v.shape[1], v.shape[1]))
    for h in range(q.shape[0]):
        logits = scale * (q[h] @ k.T)
        logits -= logits.max(axis=1, keepdims=True)
        s = np.exp(logits)
        s /= s.sum(axis=1, keepdims=True)
        sv = s @ v
        c += sv.T @ sv
    return c / n


def eigenbasis(c: np.ndarray) -> np.ndarray:
    """Eigenvectors of a symmetric matrix as columns, by descending eigenvalue, with the
    largest-magnitude entry of each column made positive."""
    w, u = np.linalg.eigh(np.asarray(c, dtype=np.float64))
    order = np.argsort(w)[::-1]
    u = u[:, order]
    idx = np.argmax(np.abs(u), axis=0)
    signs = np.sign(u[idx, np.arange(u.shape[1])])
    signs[signs == 0] = 1.0
    return u * signs[None, :]


def compose_rotation(u: np.ndarray) -> np.ndarray:
    """R = U . H_Had . P_br (fp64)."""
    d = u.shape[0]
    return np.asarray(u, dtype=np.float64) @ hadamard(d) @ bitrev_matrix(d)


def rotation_fp32(r: np.ndarray) -> np.ndarray:
    """The shipped rotation: R rounded once to fp32."""
    return np.asarray(r, dtype=np.float64).astype(np.float32)
