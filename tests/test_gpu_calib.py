"""Calibration statistics on the GPU (oscar_calib_query_cov, oscar_calib_value_cov) against the
oracle's float64 covariances of the same bf16 activations, and the eigenbases they give."""
import math

import numpy as np
import pytest
import torch

import bit_rotated_kv_amd as brk
import gpu_util as G
import oracle
import synth
from bit_rotated_kv_amd import calib

pytestmark = pytest.mark.gpu


def _bf16(x):
    """(device bf16 tensor, float64 values) of x rounded to bf16."""
    bits = oracle.bf16_bits(x)
    return G.bf16_tensor(bits), oracle.bf16_from_bits(bits).astype(np.float64)


def _max_rel(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


@pytest.mark.parametrize("base,kvs,n", [(2, (0, 5), 8878), (1, (0,), 1024), (2, (3,), 777)])
def test_query_covariance(base, kvs, n):
    """C_Q = (1/N) sum over heads of Q^T Q: bf16 products exact, fp32 sums in a fixed order."""
    w = synth.workload(base)
    print(f"case query covariance {w.name} n={n}", flush=True)
    qs = [synth.calibration_queries(w, kv)[:, :n] for kv in kvs]
    qt, qv = _bf16(np.stack(qs))
    got = brk.calib_query_cov(qt).cpu().numpy().astype(np.float64)
    for i, kv in enumerate(kvs):
        ref = oracle.query_covariance(qv[i])
        print(f"kv {kv}: max |C_gpu - C_oracle| / max |C| = {_max_rel(got[i], ref):.2e}")
        assert _max_rel(got[i], ref) <= 2e-5, (kv, _max_rel(got[i], ref))
        assert np.array_equal(got[i], got[i].T) or _max_rel(got[i], got[i].T) <= 1e-6


@pytest.mark.parametrize("base,kv,nq,nctx", [(2, 0, 1024, 4096), (1, 0, 300, 1000), (2, 6, 129, 33)])
def test_value_covariance(base, kv, nq, nctx):
    """C_S = (1/N) sum over heads of (S V)^T (S V), S = softmax(Q K^T / sqrt(d)): flash-attention S V
    in fp32 and a Gram of its bf16 high + low parts."""
    w = synth.workload(base)
    print(f"case value covariance {w.name} nq={nq} nctx={nctx}", flush=True)
    qc = synth.calibration_queries(w, kv)[:, :nq]
    kc, vc = synth.calibration_context(w, kv)
    qt, qv = _bf16(qc[None])
    kt, kvv = _bf16(kc[None, :nctx])
    vt, vv = _bf16(vc[None, :nctx])
    scale = 1.0 / math.sqrt(w.head_dim)
    got = brk.calib_value_cov(qt, kt, vt, scale).cpu().numpy().astype(np.float64)[0]
    ref = oracle.score_weighted_value_covariance(qv[0], kvv[0], vv[0], scale)
    print(f"max |C_gpu - C_oracle| / max |C| = {_max_rel(got, ref):.2e}")
    assert _max_rel(got, ref) <= 1e-4, _max_rel(got, ref)


def test_gpu_eigenbases_fit_the_oracle_covariances():
    """The eigenvectors of the GPU covariances leave residuals on the oracle's covariances no larger
    than the covariance difference, and the rotations built from them are orthogonal."""
    w = synth.workload(2)
    kvs = (0, 1)
    qc = np.stack([synth.calibration_queries(w, kv) for kv in kvs])
    ctx = [synth.calibration_context(w, kv) for kv in kvs]
    qt, qv = _bf16(qc)
    kt, kvv = _bf16(np.stack([c[0] for c in ctx]))
    vt, vv = _bf16(np.stack([c[1] for c in ctx]))
    scale = 1.0 / math.sqrt(w.head_dim)
    rk, rv = calib.rotations_on_gpu(qt, kt, vt, 1024, scale)
    cq = brk.calib_query_cov(qt).cpu().double()
    cs = brk.calib_value_cov(qt[:, :, :1024].contiguous(), kt, vt, scale).cpu().double()
    for i in range(len(kvs)):
        for gpu_c, ref_c in ((cq[i], oracle.query_covariance(qv[i])),
                             (cs[i], oracle.score_weighted_value_covariance(qv[i, :, :1024], kvv[i], vv[i], scale))):
            _, _, u = brk.rotation_from_covariance(gpu_c.numpy(), return_eig=True)
            lam = np.einsum("ij,ik,kj->j", u, ref_c, u)
            resid = np.linalg.norm(ref_c @ u - u * lam[None, :], axis=0).max()
            gap = np.linalg.norm(gpu_c.numpy() - ref_c, 2)
            assert resid <= 2.0 * gap + 1e-12 * np.linalg.norm(ref_c, 2), (resid, gap)
        for r in (rk[i], rv[i]):
            r64 = r.cpu().double().numpy()
            assert np.abs(r64.T @ r64 - np.eye(w.head_dim)).max() <= 1e-6
