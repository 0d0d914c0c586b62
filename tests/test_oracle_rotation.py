"""Pins of the oracle's rotation construction against textbook/library facts and exact
identities (no GPU)."""
import numpy as np
import pytest
import scipy.linalg

import oracle
import synth


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 128, 256])
def test_hadamard_matches_library(d):
    h = oracle.hadamard(d)
    assert np.array_equal(h * np.sqrt(d), scipy.linalg.hadamard(d).astype(np.float64))
    assert np.allclose(h @ h.T, np.eye(d), atol=1e-14)


def test_bitrev_textbook_values():
    # the 3-bit reversal permutation
    assert list(oracle.bitrev_indices(8)) == [0, 4, 2, 6, 1, 5, 3, 7]
    assert list(oracle.bitrev_indices(4)) == [0, 2, 1, 3]


@pytest.mark.parametrize("d", [8, 64, 128])
def test_bitrev_involution_and_matrix(d):
    r = oracle.bitrev_indices(d)
    assert np.array_equal(r[r], np.arange(d))
    assert r[1] == d // 2
    p = oracle.bitrev_matrix(d)
    assert np.array_equal(p, p.T)
    assert np.array_equal(p @ p, np.eye(d))
    # row i of P has its one at column rev(i): (x P)[rev(i)] = x[i]
    x = np.arange(d, dtype=np.float64)
    assert np.array_equal((x @ p)[r], x)


@pytest.mark.parametrize("d", [8, 64, 128])
def test_hadamard_commutes_with_bitrev(d):
    h, p = oracle.hadamard(d), oracle.bitrev_matrix(d)
    assert np.allclose(h @ p, p @ h, atol=1e-15)


def test_query_covariance_brute_force():
    r = np.random.default_rng(5)
    q = r.standard_normal((3, 7, 5))
    c = oracle.query_covariance(q)
    ref = np.zeros((5, 5))
    for h in range(3):
        for n in range(7):
            for i in range(5):
                for j in range(5):
                    ref[i, j] += q[h, n, i] * q[h, n, j]
    assert np.allclose(c, ref / 7, rtol=1e-13, atol=1e-13)


def test_query_covariance_weights_logit_error():
    """||Q K^T - Q Khat^T||_F^2 = tr((K - Khat) Q^T Q (K - Khat)^T) = N tr(dK C_Q dK^T)."""
    r = np.random.default_rng(6)
    q = r.standard_normal((50, 16)) * np.linspace(0.1, 5, 16)
    k = r.standard_normal((30, 16))
    khat = k + 0.05 * r.standard_normal((30, 16))
    lhs = np.linalg.norm(q @ k.T - q @ khat.T) ** 2
    dk = k - khat
    rhs = 50 * np.trace(dk @ oracle.query_covariance(q) @ dk.T)
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs)


def test_value_covariance_brute_force():
    r = np.random.default_rng(7)
    q = r.standard_normal((4, 6))
    k = r.standard_normal((9, 6))
    v = r.standard_normal((9, 6))
    scale = 0.4
    c = oracle.score_weighted_value_covariance(q, k, v, scale)
    ref = np.zeros((6, 6))
    for n in range(4):
        lg = [scale * sum(q[n, j] * k[t, j] for j in range(6)) for t in range(9)]
        e = [np.exp(x) for x in lg]
        s = [x / sum(e) for x in e]
        sv = [sum(s[t] * v[t, j] for t in range(9)) for j in range(6)]
        for i in range(6):
            for j in range(6):
                ref[i, j] += sv[i] * sv[j]
    assert np.allclose(c, ref / 4, rtol=1e-12, atol=1e-14)


def test_value_covariance_weights_output_error():
    """For a channel-space error V_hat = V (I + E): ||S V - S V_hat||_F^2 = N tr(E^T C_S E)."""
    r = np.random.default_rng(8)
    q = r.standard_normal((20, 8))
    k = r.standard_normal((15, 8))
    v = r.standard_normal((15, 8))
    e = 0.01 * r.standard_normal((8, 8))
    logits = 0.3 * q @ k.T
    s = np.exp(logits - logits.max(1, keepdims=True))
    s /= s.sum(1, keepdims=True)
    lhs = np.linalg.norm(s @ v - s @ (v @ (np.eye(8) + e))) ** 2
    rhs = 20 * np.trace(e.T @ oracle.score_weighted_value_covariance(q, k, v, 0.3) @ e)
    assert abs(lhs - rhs) <= 1e-10 * abs(lhs)


def test_eigenbasis_properties():
    r = np.random.default_rng(9)
    a = r.standard_normal((40, 12))
    c = a.T @ a
    u = oracle.eigenbasis(c)
    lam = np.diag(u.T @ c @ u)
    assert np.all(np.diff(lam) <= 1e-9)                          # descending
    assert np.allclose(c @ u, u * lam[None, :], atol=1e-10 * np.abs(c).max())
    assert np.allclose(u.T @ u, np.eye(12), atol=1e-12)
    idx = np.argmax(np.abs(u), axis=0)
    assert np.all(u[idx, np.arange(12)] > 0)


def test_composed_rotation_order():
    """x . R with R = U H P: the i-th eigen-direction u_i (as a row) maps to row i of H P,
    i.e. U acts first, then the Hadamard mix, then the bit-reversal reorder."""
    d = 16
    u = synth.random_orthogonal(np.random.default_rng(10), d)
    rm = oracle.compose_rotation(u)
    assert np.allclose(rm.T @ rm, np.eye(d), atol=1e-13)
    hp = oracle.hadamard(d) @ oracle.bitrev_matrix(d)
    for i in range(d):
        assert np.allclose(u[:, i] @ rm, hp[i], atol=1e-13)
    r32 = oracle.rotation_fp32(rm)
    assert r32.dtype == np.float32
    assert np.allclose(r32.astype(np.float64).T @ r32.astype(np.float64), np.eye(d), atol=1e-6)


def test_workload_rotation_from_covariance():
    """Key basis of a synthetic workload comes from C_Q: its leading direction carries the
    largest query energy."""
    w = synth.workload(2, cal_tokens=2000, num_q_heads=8, num_kv_heads=2)
    q = synth.calibration_queries(w, 0)
    c = oracle.query_covariance(q)
    u = oracle.eigenbasis(c)
    e = [np.mean((q.reshape(-1, w.head_dim) @ u[:, i]) ** 2) for i in (0, w.head_dim - 1)]
    assert e[0] > e[1]
