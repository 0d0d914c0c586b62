"""Token routing on the GPU (oscar_route_tokens): tag classes to INT2/INT4 widths, and a mixed
cache prefilled from routed widths equals the one prefilled from the oracle's widths."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_amd as brk
import gpu_util as G
import problem as P
import synth

pytestmark = pytest.mark.gpu


def test_route_tokens_matches_a_table_lookup():
    r = np.random.default_rng(60)
    B, T = 5, 3000
    lens = np.array([0, 1, 1023, 1024, 3000], np.int32)
    tags = r.integers(-2, 25, (B, T)).astype(np.int32)      # includes out-of-range tags
    cb = r.choice([2, 4], 22).astype(np.uint8)
    got = brk.route_tokens(torch.from_numpy(lens).cuda(), torch.from_numpy(tags).cuda(), cb)
    torch.cuda.synchronize()
    ref = np.full((B, T), 2, np.uint8)
    for b in range(B):
        t = tags[b, :lens[b]]
        ref[b, :lens[b]] = np.where((t >= 0) & (t < 22), cb[np.clip(t, 0, 21)], 2)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_prefill_from_routed_widths_equals_oracle_widths():
    """Library greedy + GPU routing + prefill == prefill from the oracle-derived widths (pool,
    window and INT4 counts byte for byte)."""
    print("case mixed routing", flush=True)
    w = synth.workload(5, batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(1500, 900), cal_tokens=1500,
                       cal_ctx=512)
    pf = P.make_problem(w, with_oracle=False)
    d2, d4 = synth.tag_sensitivity(w)
    cb, _ = brk.allocate_bits(d2, d4, synth.tag_nominal_counts(w), w.bit_budget)
    tmax = max(w.seq_lens)
    tags = np.zeros((w.batch, tmax), np.int32)
    for b in range(w.batch):
        tags[b, :w.seq_lens[b]] = synth.tag_classes(w, b, w.seq_lens[b])
    lens = torch.tensor(list(w.seq_lens), dtype=torch.int32, device="cuda")
    routed = brk.route_tokens(lens, torch.from_numpy(tags).cuda(), cb)
    oracle_bits = torch.from_numpy(P.bits_tensor(pf)).cuda()
    assert torch.equal(routed, oracle_bits)
    caches = []
    for tb in (routed, oracle_bits):
        cbuf = brk.allocate_cache(w.num_q_heads, w.num_kv_heads, w.head_dim, w.batch, tmax, mixed=True,
                                  pages2_per_request=pf.pages2, pages4_per_request=pf.pages4,
                                  page_order2=pf.order2, page_order4=pf.order4)
        k = G.bf16_tensor(P.kv_bits_tensor(pf, "k"))
        v = G.bf16_tensor(P.kv_bits_tensor(pf, "v"))
        cbuf.seq_len.copy_(lens)
        brk.kv_prefill(cbuf.layout, cbuf.seq_len, k, v, torch.from_numpy(pf.rot_k).cuda(),
                       torch.from_numpy(pf.rot_v).cuda(), cbuf.pool, cbuf.page_table, cbuf.window, token_bits=tb,
                       page_table4=cbuf.page_table4, n_int4_out=cbuf.n_int4)
        caches.append(cbuf)
    torch.cuda.synchronize()
    a, b = caches
    assert torch.equal(a.pool, b.pool) and torch.equal(a.window, b.window) and torch.equal(a.n_int4, b.n_int4)
    expect = [int((P.token_bits(w, bb, w.seq_lens[bb])[64:w.seq_lens[bb] - 256] == 4).sum()) for bb in range(w.batch)]
    assert a.n_int4.cpu().tolist() == expect
