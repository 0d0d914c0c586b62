"""oscar_rotation_from_covariance (host call): R = U . H . P_br from a covariance, against the
oracle's eigenbasis and composition ("Together AI open-sources OSCAR", section on what makes OSCAR
different), and against closed forms that need no eigensolver."""
import os

import numpy as np
import pytest

import bit_rotated_kv_amd as brk
import oracle
import synth
from bit_rotated_kv_amd import _lib


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(_lib.LIB_PATH):
        from bit_rotated_kv_amd import build
        build.build()


def _spd(d, seed, spread=1.0):
    """A symmetric positive definite matrix with well separated eigenvalues."""
    rng = np.random.default_rng(seed)
    q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.exp(spread * np.linspace(3.0, -3.0, d)) * (1.0 + 0.1 * rng.random(d))
    return (q * lam) @ q.T


@pytest.mark.parametrize("d,seed", [(8, 0), (64, 1), (128, 2)])
def test_matches_the_oracle_rotation(d, seed):
    c = _spd(d, seed)
    ref = oracle.rotation_fp32(oracle.compose_rotation(oracle.eigenbasis(c)))
    got, w, u = brk.rotation_from_covariance(c, return_eig=True)
    assert got.dtype == np.float32 and got.shape == (d, d)
    assert np.abs(got.astype(np.float64) - ref).max() <= 1e-6
    assert np.allclose(w, np.sort(np.linalg.eigvalsh(c))[::-1], rtol=1e-11, atol=1e-13 * np.abs(w).max())
    assert np.abs(u - oracle.eigenbasis(c)).max() <= 1e-9


def test_calibration_covariance_of_a_workload():
    """The query covariance of a Qwen3-8B-shaped kv-head (8 heavy channels, a low-variance half)."""
    w = synth.workload(2)
    qc = synth.calibration_queries(w, 3)[:, :2048]
    c = oracle.query_covariance(qc)
    ref = oracle.rotation_fp32(oracle.compose_rotation(oracle.eigenbasis(c)))
    got = brk.rotation_from_covariance(c)
    assert np.abs(got.astype(np.float64) - ref).max() <= 1e-6


def test_batch_of_matrices_is_per_matrix():
    cs = np.stack([_spd(64, s) for s in range(3)])
    got = brk.rotation_from_covariance(cs)
    for i in range(3):
        assert np.array_equal(got[i], brk.rotation_from_covariance(cs[i]))


def test_diagonal_covariance_closed_form():
    """A diagonal C with distinct entries has the eigenvectors +e_i (the entry 1 is the largest),
    sorted by descending entry, so R[i][j] = H[pos(i)][rev(j)] with pos(i) the rank of C_ii."""
    d = 16
    rng = np.random.default_rng(5)
    diag = rng.permutation(np.arange(1, d + 1, dtype=np.float64))
    got = brk.rotation_from_covariance(np.diag(diag))
    rank = np.argsort(-diag).argsort()
    h = np.array([[(-1.0) ** bin(k & m).count("1") for m in range(d)] for k in range(d)]) / 4.0
    rev = [int(format(j, "04b")[::-1], 2) for j in range(d)]
    ref = np.array([[h[rank[i]][rev[j]] for j in range(d)] for i in range(d)])
    assert np.array_equal(got.astype(np.float64), ref)


def test_rotation_is_orthogonal_and_symmetrised():
    c = _spd(128, 7)
    asym = c + 1e-9 * np.triu(np.ones_like(c), 1)
    r = brk.rotation_from_covariance(asym).astype(np.float64)
    assert np.abs(r.T @ r - np.eye(128)).max() <= 1e-6
    sym = brk.rotation_from_covariance(0.5 * (asym + asym.T))
    assert np.array_equal(brk.rotation_from_covariance(asym), sym)


def test_rejections():
    lib = _lib.lib()
    c = np.eye(4)
    r = np.zeros((4, 4), np.float32)
    bad = c.copy()
    bad[1, 2] = np.nan
    assert lib.oscar_rotation_from_covariance(1, 6, c.ctypes.data, r.ctypes.data, None, None) == -1
    assert lib.oscar_rotation_from_covariance(1, 4, bad.ctypes.data, r.ctypes.data, None, None) == -1
    assert lib.oscar_rotation_from_covariance(1, 4, None, r.ctypes.data, None, None) == -1
    assert lib.oscar_rotation_from_covariance(-1, 4, c.ctypes.data, r.ctypes.data, None, None) == -1
    assert lib.oscar_rotation_from_covariance(1, 512, c.ctypes.data, r.ctypes.data, None, None) == -2
    assert lib.oscar_rotation_from_covariance(0, 4, None, None, None, None) == 0
