"""Parity at the full sizes of the benchmark workloads, in the launch configuration bench.py
times: the whole batch is prefilled to T-1 tokens on the GPU and one fused decode step
(demote + append + attention) runs over it with the bench's length bound (T + 14). The oracle then
recomputes sampled (request, kv-head) groups one by one at full context. Sampled groups hold the
numpy draws of the workload; the other groups hold GPU draws of the same channel law (they are
computed but not compared)."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_amd as brk
import gpu_util as G
import oracle
import problem as P
import synth

pytestmark = pytest.mark.gpu

EXTRA = 14   # bench.py's length bound: context + steps // copies + 2


def _kv_device(w, T_max, sampled):
    """K, V [B, Hkv, T_max, d] bf16: numpy draws for the sampled groups, GPU draws otherwise."""
    B, hkv, d = w.batch, w.num_kv_heads, w.head_dim
    K = torch.empty((B, hkv, T_max, d), dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    gen = torch.Generator(device="cuda")
    for b in range(B):
        for kv in range(hkv):
            T = w.seq_lens[b]
            if (b, kv) in sampled:
                ks, vs = synth.kv_slice(w, b, kv, T)
                K[b, kv, :T] = torch.from_numpy(ks).cuda().bfloat16()
                V[b, kv, :T] = torch.from_numpy(vs).cuda().bfloat16()
            else:
                gen.manual_seed(1_000_003 * w.seed + 1009 * b + kv)
                sk = torch.from_numpy(synth.channel_scales(w, "chan_k", kv)).float().cuda()
                sv = torch.from_numpy(synth.channel_scales(w, "chan_v", kv)).float().cuda()
                K[b, kv, :T] = (torch.randn((T, d), generator=gen, device="cuda") * sk).bfloat16()
                V[b, kv, :T] = (torch.randn((T, d), generator=gen, device="cuda") * sv).bfloat16()
            if T < T_max:
                K[b, kv, T:] = 0
                V[b, kv, T:] = 0
    return K, V


def _run(w, sampled, codebook=False):
    B, hq, hkv, d, g = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.gqa
    lens = list(w.seq_lens)
    tmax = max(lens) + EXTRA
    rk, rv = P.rotations(w)
    cbk = P.fit_codebooks(w, rk, rv) if codebook else None
    table = torch.from_numpy(np.ascontiguousarray(P.codebook_patterns(cbk))).cuda() if codebook else None
    bits = [P.token_bits(w, b, lens[b]) for b in range(B)]
    hist = [max(0, T - 320) for T in lens]
    n4 = [int((bits[b][64:64 + hist[b]] == 4).sum()) for b in range(B)]
    n2 = [hist[b] - n4[b] for b in range(B)]
    tmax_hist = max(0, tmax - 320)
    pages2 = (tmax_hist + 15) // 16 if not w.mixed else max((n + 15) // 16 for n in n2) + 1
    pages4 = (max((n + 15) // 16 for n in n4) + 1) if w.mixed else 0
    order2 = synth.page_permutation(w.seed, B * pages2)
    order4 = synth.page_permutation(w.seed + 1, B * pages4) if w.mixed else None
    cb = brk.allocate_cache(hq, hkv, d, B, tmax, mixed=w.mixed, pages2_per_request=pages2,
                            pages4_per_request=pages4, page_order2=order2, page_order4=order4, codebook=table)
    K, V = _kv_device(w, tmax, sampled)
    rkt, rvt = torch.from_numpy(rk).cuda(), torch.from_numpy(rv).cuda()
    tb = None
    if w.mixed:
        tbn = np.full((B, tmax), 2, np.uint8)
        for b in range(B):
            tbn[b, :lens[b]] = bits[b]
        tb = torch.from_numpy(tbn).cuda()
    cb.seq_len.copy_(torch.tensor([T - 1 for T in lens], dtype=torch.int32))
    brk.kv_prefill(cb.layout, cb.seq_len, K, V, rkt, rvt, cb.pool, cb.page_table, cb.window, token_bits=tb,
                   page_table4=cb.page_table4, n_int4_out=cb.n_int4)
    nk = torch.stack([K[b, :, lens[b] - 1] for b in range(B)]).contiguous()
    nv = torch.stack([V[b, :, lens[b] - 1] for b in range(B)]).contiguous()
    db = None
    if w.mixed:
        db = torch.tensor([int(bits[b][lens[b] - 1 - 256]) if lens[b] - 1 >= 320 else 2 for b in range(B)],
                          dtype=torch.uint8, device="cuda")
    q = np.stack([synth.decode_query(w, b) for b in range(B)])
    qt = G.bf16_tensor(oracle.bf16_bits(q))
    ws = torch.zeros(brk.decode_workspace_bytes(cb.layout, B, tmax), dtype=torch.uint8, device="cuda")
    seq_out = torch.zeros_like(cb.seq_len)
    n4_out = torch.zeros_like(cb.n_int4) if w.mixed else None
    out = brk.decode_step(cb.layout, cb.seq_len, nk, nv, qt, rkt, rvt, cb.pool, cb.page_table, cb.window, seq_out,
                          ws, tmax, n_int4=cb.n_int4, n_int4_out=n4_out, demote_bits=db, page_table4=cb.page_table4)
    torch.cuda.synchronize()
    assert seq_out.cpu().tolist() == lens
    if w.mixed:
        assert n4_out.cpu().tolist() == n4
    assert int(ws[:4].view(torch.int32).item()) == 0
    got = out.cpu().numpy().astype(np.float64)
    del K, V, cb, ws
    torch.cuda.empty_cache()
    results = []
    for b, kv in sampled:
        ks, vs = synth.kv_slice(w, b, kv, lens[b])
        kw = {} if cbk is None else dict(codebook_k=cbk[kv:kv + 1, 0], codebook_v=cbk[kv:kv + 1, 1])
        cache = oracle.OracleCache.from_prefix(ks[None], vs[None], rk[kv:kv + 1], rv[kv:kv + 1], w.group_size,
                                               bits=bits[b], **kw)
        ref = oracle.decode_attention(cache, q[b, kv * g:(kv + 1) * g])
        worst, mab = G.check_close(got[b:b + 1, kv * g:(kv + 1) * g], ref[None], tag=f"{w.name} b{b} kv{kv}")
        results.append((b, kv, worst, mab))
        print(f"{w.name} request {b} kv-head {kv} (T={lens[b]}): worst rel-L2 {worst:.2e}, max-abs {mab:.2e}",
              flush=True)
    return results


def test_fullsize_qwen3_8b_bs1_100k():
    """The bench workload itself: one request, 100,000 tokens, 32 query / 8 kv heads."""
    print("case qwen3-8b bs1 100k", flush=True)
    _run(synth.workload(2), sampled=[(0, 0), (0, 5)])


def test_fullsize_paged_bs32_32k():
    print("case paged bs32 32k", flush=True)
    _run(synth.workload(3), sampled=[(0, 2), (17, 7), (31, 0)])


def test_fullsize_paged_bs32_100k():
    """The metric's literal batch-32 point: workload 3's paged batch at 100,000 tokens per request."""
    print("case paged bs32 100k", flush=True)
    w = synth.workload(3, seq_lens=(100_000,) * 32)
    _run(w, sampled=[(0, 3), (31, 6)])


def test_fullsize_ragged_bs8_gqa8():
    print("case ragged bs8 up to 131k, GQA 8", flush=True)
    w = synth.workload(4)
    longest = int(np.argmax(w.seq_lens))
    shortest = int(np.argmin(w.seq_lens))
    _run(w, sampled=[(longest, 3), (shortest, 6)])


def test_fullsize_mixed_int2_int4_bs16_64k():
    print("case mixed INT2/INT4 bs16 64k", flush=True)
    _run(synth.workload(5), sampled=[(0, 1), (9, 4)])


def test_fullsize_codebook_qwen3_8b_bs1_100k():
    """The bench workload with Lloyd-Max INT2 codebooks (fitted on the calibration context)."""
    print("case codebook qwen3-8b bs1 100k", flush=True)
    _run(synth.workload(2), sampled=[(0, 3), (0, 6)], codebook=True)


def test_fullsize_codebook_paged_bs32_32k():
    print("case codebook paged bs32 32k", flush=True)
    _run(synth.workload(3), sampled=[(5, 1), (30, 4)], codebook=True)
