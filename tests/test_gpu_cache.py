"""GPU cache writers against the oracle: prefill windows (exact), prefill history (codes within one
level on at most 0.1% of elements, scale/zero within one bf16 step), and the per-step demote
reproducing the prefill state bit for bit."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_amd as brk
import gpu_util as G
import layout_ref
import oracle
import problem as P
import synth

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-ref": lambda: synth.workload(1),
    "d128-gqa4-ragged": lambda: synth.workload(2, batch=3, num_q_heads=8, num_kv_heads=2, seq_lens=(1000, 337, 2000),
                                               cal_tokens=1500, cal_ctx=512),
    "d128-mixed": lambda: synth.workload(5, batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(1500, 900),
                                         cal_tokens=1500, cal_ctx=512),
    # INT2-only at d 64 with histories 580 and 13 (a last chunk of 4 rows, a request shorter than a chunk)
    "d64-int2-ragged": lambda: synth.workload(1, batch=2, num_q_heads=4, num_kv_heads=2, seq_lens=(900, 333)),
    "d64-mixed": lambda: synth.workload(5, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, group_size=64,
                                        seq_lens=(1300, 800), cal_tokens=1500, cal_ctx=512),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def prefilled(request):
    print(f"case {request.param}", flush=True)
    p = P.make_problem(CASES[request.param]())
    cb, rk, rv = G.build_cache(p, oracle_written=False)
    return p, cb


def test_prefill_window_exact(prefilled):
    p, cb = prefilled
    w = p.w
    d = w.head_dim
    W = 20
    win = cb.window.cpu().numpy().view(np.uint16).reshape(w.batch, w.num_kv_heads, W, 32 * d)
    kb, vb = P.kv_bits_tensor(p, "k"), P.kv_bits_tensor(p, "v")
    for b in range(w.batch):
        T = w.seq_lens[b]
        for kv in range(w.num_kv_heads):
            held = layout_ref.read_window(win[b, kv], d, 64, 256, T)
            (s0, s1), _, (r0, r1) = oracle.segments(T)
            assert sorted(held) == list(range(s0, s1)) + list(range(r0, r1))
            for pos, (kk, vv) in held.items():
                assert np.array_equal(kk, kb[b, kv, pos]) and np.array_equal(vv, vb[b, kv, pos])


def _history_check(p, cb):
    w = p.w
    d = w.head_dim
    pool = cb.pool.cpu().numpy()
    pt2 = cb.page_table.cpu().numpy()
    pt4 = None if cb.page_table4 is None else cb.page_table4.cpu().numpy()
    off4 = cb.layout.int4_page_offset if p.mixed else cb.layout.pool_pages
    n_el = n_diff = 0
    for b in range(w.batch):
        c = p.caches[b]
        for kv in range(w.num_kv_heads):
            for bits, pt in ((2, pt2), (4, pt4)):
                if bits == 4 and not p.mixed:
                    continue
                ok, ov, osk, osv = P.oracle_history(c, kv, bits)
                gk, gv, gsk, gsv = layout_ref.read_history(pool, d, w.num_kv_heads, off4, kv, bits, pt[b], len(ok))
                for gc, oc in ((gk, ok), (gv, ov)):
                    diff = np.abs(gc.astype(int) - oc.astype(int))
                    assert diff.max(initial=0) <= 1, (b, kv, bits)
                    n_el += diff.size
                    n_diff += int((diff > 0).sum())
                for gs, os_ in ((gsk, osk), (gsv, osv)):
                    assert np.abs(gs.astype(np.int64) - os_.astype(np.int64)).max(initial=0) <= 1
    return n_el, n_diff


def test_prefill_history_matches_oracle(prefilled):
    p, cb = prefilled
    n_el, n_diff = _history_check(p, cb)
    print(f"history elements {n_el}, codes off by one level: {n_diff}")
    assert n_el > 0 and n_diff <= 1e-3 * n_el


def test_prefill_ints4_count(prefilled):
    p, cb = prefilled
    if p.mixed:
        assert cb.n_int4.cpu().tolist() == G.n_int4_counts(p)


@pytest.mark.parametrize("base,kw,steps", [
    (2, dict(batch=2, num_q_heads=4, num_kv_heads=2, seq_lens=(40, 330)), 300),
    (5, dict(batch=2, num_q_heads=4, num_kv_heads=2, seq_lens=(500, 700)), 80),
    (1, dict(seq_lens=(1000,)), 40),
])
def test_demote_steps_equal_prefill(base, kw, steps):
    """Prefill to T0, then `steps` demote/append steps == prefill to T0 + steps (bit for bit), and the
    history written step by step matches the oracle's step-by-step cache."""
    print(f"case base={base} {kw} steps={steps}", flush=True)
    t0 = kw["seq_lens"]
    full = dict(kw, seq_lens=tuple(t + steps for t in t0), cal_tokens=1500, cal_ctx=512)
    w_full = synth.workload(base, **full)
    pf = P.make_problem(w_full)
    tmax = max(w_full.seq_lens)
    # reference: prefill at the final lengths
    cb_ref, rk, rv = G.build_cache(pf, oracle_written=False)
    # step by step: prefill at T0, then demote with the next tokens
    cb = brk.allocate_cache(w_full.num_q_heads, w_full.num_kv_heads, w_full.head_dim, w_full.batch, tmax,
                            mixed=pf.mixed, pages2_per_request=pf.pages2, pages4_per_request=pf.pages4,
                            page_order2=pf.order2, page_order4=pf.order4)
    kfull = G.bf16_tensor(P.kv_bits_tensor(pf, "k"))
    vfull = G.bf16_tensor(P.kv_bits_tensor(pf, "v"))
    tb = torch.from_numpy(P.bits_tensor(pf)).cuda() if pf.mixed else None
    cb.seq_len.copy_(torch.tensor(list(t0), dtype=torch.int32))
    brk.kv_prefill(cb.layout, cb.seq_len, kfull, vfull, rk, rv, cb.pool, cb.page_table, cb.window, token_bits=tb,
                   page_table4=cb.page_table4, n_int4_out=cb.n_int4)
    seq = [cb.seq_len, torch.zeros_like(cb.seq_len)]
    n4 = [cb.n_int4, torch.zeros_like(cb.n_int4)] if pf.mixed else [None, None]
    for i in range(steps):
        pos = [t + i for t in t0]
        nk = torch.stack([kfull[b, :, pos[b]] for b in range(w_full.batch)]).contiguous()
        nv = torch.stack([vfull[b, :, pos[b]] for b in range(w_full.batch)]).contiguous()
        db = None
        if pf.mixed:
            db = torch.tensor([int(pf.bits[b][pos[b] - 256]) if pos[b] >= 320 else 2 for b in range(w_full.batch)],
                              dtype=torch.uint8, device="cuda")
        brk.kv_demote(cb.layout, seq[i % 2], nk, nv, rk, rv, cb.pool, cb.page_table, cb.window, n_int4=n4[i % 2],
                      demote_bits=db, page_table4=cb.page_table4, seq_len_out=seq[(i + 1) % 2],
                      n_int4_out=n4[(i + 1) % 2])
    torch.cuda.synchronize()
    assert seq[steps % 2].cpu().tolist() == list(w_full.seq_lens)
    assert torch.equal(cb.window, cb_ref.window)
    assert torch.equal(cb.pool, cb_ref.pool)
    if pf.mixed:
        assert n4[steps % 2].cpu().tolist() == G.n_int4_counts(pf)
    # and the step-by-step oracle agrees with the GPU history (one-level tolerance)
    n_el, n_diff = _history_check(pf, cb)
    assert n_diff <= 1e-3 * max(n_el, 1)
