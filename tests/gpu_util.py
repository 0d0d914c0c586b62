"""GPU-side helpers of the parity tests: build the library's buffers for a ``problem.Problem``
and run its entry points (test infrastructure)."""
from __future__ import annotations

import numpy as np
import torch

import bit_rotated_kv_amd as brk
import problem as P


def bf16_tensor(bits_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).cuda().view(torch.bfloat16)


def n_int4_counts(p: P.Problem):
    return [int((p.bits[b][64:max(64, T - 256)] == 4).sum()) for b, T in enumerate(p.w.seq_lens)]


def codebook_tensor(p: P.Problem):
    """The problem's INT2 codebook table on the device (None for the uniform levels)."""
    if p.codebook is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(P.codebook_patterns(p.codebook))).cuda()


def allocate(p: P.Problem, tmax: int):
    w = p.w
    return brk.allocate_cache(w.num_q_heads, w.num_kv_heads, w.head_dim, w.batch, tmax, mixed=p.mixed,
                              pages2_per_request=p.pages2, pages4_per_request=p.pages4, page_order2=p.order2,
                              page_order4=p.order4, codebook=codebook_tensor(p))


def build_cache(p: P.Problem, oracle_written: bool, max_seq_len: int = None):
    """Allocate buffers for p and fill them (GPU prefill, or the oracle's codes via layout_ref)."""
    w = p.w
    tmax = max(P.max_len(p), 1) if max_seq_len is None else max_seq_len
    cb = allocate(p, tmax)
    cb.seq_len.copy_(torch.tensor(list(w.seq_lens), dtype=torch.int32))
    rk = torch.from_numpy(p.rot_k).cuda()
    rv = torch.from_numpy(p.rot_v).cuda()
    if oracle_written:
        pt4 = None if cb.page_table4 is None else cb.page_table4.cpu().numpy()
        pool, win = P.oracle_pool_and_window(p, cb.layout, cb.page_table.cpu().numpy(), pt4, cb.pool.numel(),
                                             cb.window.numel())
        cb.pool.copy_(torch.from_numpy(pool))
        cb.window.copy_(torch.from_numpy(np.ascontiguousarray(win)))
        if p.mixed:
            cb.n_int4.copy_(torch.tensor(n_int4_counts(p), dtype=torch.int32))
    else:
        k = bf16_tensor(P.kv_bits_tensor(p, "k"))
        v = bf16_tensor(P.kv_bits_tensor(p, "v"))
        tb = torch.from_numpy(P.bits_tensor(p)).cuda() if p.mixed else None
        if k.shape[2] < tmax:
            pad = tmax - k.shape[2]
            k = torch.nn.functional.pad(k, (0, 0, 0, pad))
            v = torch.nn.functional.pad(v, (0, 0, 0, pad))
            if tb is not None:
                tb = torch.nn.functional.pad(tb, (0, pad), value=2)
        brk.kv_prefill(cb.layout, cb.seq_len, k.contiguous(), v.contiguous(), rk, rv, cb.pool, cb.page_table,
                       cb.window, token_bits=tb, page_table4=cb.page_table4, n_int4_out=cb.n_int4)
    torch.cuda.synchronize()
    return cb, rk, rv


def decode(p: P.Problem, cb, rk, rv, q: np.ndarray = None):
    qq = P.oracle.bf16_bits(p.q if q is None else q)
    qt = bf16_tensor(qq)
    ws = torch.zeros(brk.decode_workspace_bytes(cb.layout, p.w.batch, cb.max_seq_len), dtype=torch.uint8,
                     device="cuda")
    out = brk.decode_attn(cb.layout, qt, cb.seq_len, cb.window, cb.pool, cb.page_table, rk, rv, ws, cb.max_seq_len,
                          n_int4=cb.n_int4, page_table4=cb.page_table4)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), ws


def check_close(got, ref, rel=5e-3, abs_=1e-2, tag=""):
    """Per (request, head) relative L2 and global max-abs bars."""
    worst = 0.0
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            if np.linalg.norm(ref[b, h]) == 0:
                assert np.abs(got[b, h]).max() <= abs_, (tag, b, h)
                continue
            worst = max(worst, P.rel_l2(got[b, h], ref[b, h]))
    mab = np.abs(got - ref).max()
    assert worst <= rel and mab <= abs_, f"{tag}: worst rel-L2 {worst:.3e}, max-abs {mab:.3e}"
    return worst, mab
