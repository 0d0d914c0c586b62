"""The fused decode step (oscar_decode_step: split + merge, the demote riding along in the split)
against the two entry points it fuses, over several steps: the cache it leaves (pool, window,
lengths) bit for bit after every step, its output to fp32 rounding (the demoted and the appended
token enter as one-token partials there, through the page and window paths in the two-call
sequence); and its last output against the oracle's attention over the final cache (same bar as
the decode tests)."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_amd as brk
import gpu_util as G
import oracle
import problem as P
import synth

pytestmark = pytest.mark.gpu

STEPS = 6
# agreement of the fused step with the two-call sequence: one token's logit differs by the history
# or window path's rounding (~1e-5 in log2 units at most), and the two calls cut the history into
# different work units (the step's cost sequence holds the step segment), so the fp32 merge orders
# differ
REL_STEP, ABS_STEP = 5e-5, 2e-3

CASES = {
    "int2-d128-gq4": dict(base=2, batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(1000, 400)),
    "int2-d64-gq8": dict(base=1, batch=2, num_q_heads=16, num_kv_heads=2, seq_lens=(330, 900)),
    "mixed-d128-gq4": dict(base=5, batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(1200, 700)),
    "mixed-d64-gq8": dict(base=5, batch=2, num_q_heads=16, num_kv_heads=2, head_dim=64, group_size=64,
                          seq_lens=(900, 500)),
    # the first demote (T = 320) and the sink boundary (T = 64) inside the stepped range
    "int2-d128-gq4-boundaries": dict(base=2, batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(317, 61)),
    "int2-d128-gq1": dict(base=2, batch=1, num_q_heads=2, num_kv_heads=2, seq_lens=(500,)),
    # 24 (request, kv-head) pairs: GQA 4 in 4-wavefront split workgroups
    "int2-d128-gq4-b3": dict(base=2, batch=3, num_q_heads=32, num_kv_heads=8, seq_lens=(700, 333, 1200)),
}


def _prefilled(pf, t0, tmax):
    w = pf.w
    cb = brk.allocate_cache(w.num_q_heads, w.num_kv_heads, w.head_dim, w.batch, tmax, mixed=pf.mixed,
                            pages2_per_request=pf.pages2, pages4_per_request=pf.pages4, page_order2=pf.order2,
                            page_order4=pf.order4)
    k = G.bf16_tensor(P.kv_bits_tensor(pf, "k"))
    v = G.bf16_tensor(P.kv_bits_tensor(pf, "v"))
    tb = torch.from_numpy(P.bits_tensor(pf)).cuda() if pf.mixed else None
    cb.seq_len.copy_(torch.tensor(list(t0), dtype=torch.int32))
    rk = torch.from_numpy(pf.rot_k).cuda()
    rv = torch.from_numpy(pf.rot_v).cuda()
    brk.kv_prefill(cb.layout, cb.seq_len, k, v, rk, rv, cb.pool, cb.page_table, cb.window, token_bits=tb,
                   page_table4=cb.page_table4, n_int4_out=cb.n_int4)
    return cb, k, v, rk, rv


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_step_equals_demote_then_decode(name):
    kw = dict(CASES[name])
    base = kw.pop("base")
    print(f"case {name}", flush=True)
    t0 = kw["seq_lens"]
    w = synth.workload(base, **dict(kw, seq_lens=tuple(t + STEPS for t in t0), cal_tokens=1500, cal_ctx=512))
    pf = P.make_problem(w)
    tmax = max(w.seq_lens)
    a, k, v, rk, rv = _prefilled(pf, t0, tmax)
    b, _, _, _, _ = _prefilled(pf, t0, tmax)
    q = G.bf16_tensor(oracle.bf16_bits(pf.q))
    ws_a = torch.zeros(brk.decode_workspace_bytes(a.layout, w.batch, tmax), dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    seq_a = [a.seq_len, torch.zeros_like(a.seq_len)]
    seq_b = [b.seq_len, torch.zeros_like(b.seq_len)]
    n4_a = [a.n_int4, torch.zeros_like(a.n_int4)] if pf.mixed else [None, None]
    n4_b = [b.n_int4, torch.zeros_like(b.n_int4)] if pf.mixed else [None, None]
    for i in range(STEPS):
        pos = [t + i for t in t0]
        nk = torch.stack([k[bb, :, pos[bb]] for bb in range(w.batch)]).contiguous()
        nv = torch.stack([v[bb, :, pos[bb]] for bb in range(w.batch)]).contiguous()
        db = None
        if pf.mixed:
            db = torch.tensor([int(pf.bits[bb][pos[bb] - 256]) if pos[bb] >= 320 else 2 for bb in range(w.batch)],
                              dtype=torch.uint8, device="cuda")
        cur, nxt = i % 2, (i + 1) % 2
        brk.kv_demote(a.layout, seq_a[cur], nk, nv, rk, rv, a.pool, a.page_table, a.window, n_int4=n4_a[cur],
                      demote_bits=db, page_table4=a.page_table4, seq_len_out=seq_a[nxt], n_int4_out=n4_a[nxt])
        out_a = brk.decode_attn(a.layout, q, seq_a[nxt], a.window, a.pool, a.page_table, rk, rv, ws_a, tmax,
                                n_int4=n4_a[nxt], page_table4=a.page_table4)
        out_b = brk.decode_step(b.layout, seq_b[cur], nk, nv, q, rk, rv, b.pool, b.page_table, b.window, seq_b[nxt],
                                ws_b, tmax, n_int4=n4_b[cur], n_int4_out=n4_b[nxt], demote_bits=db,
                                page_table4=b.page_table4)
        torch.cuda.synchronize()
        assert torch.equal(seq_a[nxt], seq_b[nxt]), f"{name}: step {i} lengths differ"
        assert torch.equal(a.pool, b.pool), f"{name}: step {i} history pages differ"
        assert torch.equal(a.window, b.window), f"{name}: step {i} window differs"
        if pf.mixed:
            assert torch.equal(n4_a[nxt], n4_b[nxt]), f"{name}: step {i} INT4 counts differ"
        G.check_close(out_b.cpu().numpy().astype(np.float64), out_a.cpu().numpy().astype(np.float64),
                      rel=REL_STEP, abs_=ABS_STEP, tag=f"{name} step {i} vs demote + decode")
    assert seq_b[STEPS % 2].cpu().tolist() == list(w.seq_lens)
    # last output against the oracle's attention over the final cache
    ref = np.stack([oracle.decode_attention(pf.caches[bb], pf.q[bb]) for bb in range(w.batch)])
    worst, mab = G.check_close(out_b.cpu().numpy().astype(np.float64), ref, tag=name)
    print(f"{name}: worst rel-L2 {worst:.2e} max-abs {mab:.2e}")


def test_decode_step_rejects_missing_outputs():
    w = synth.workload(2, batch=1, num_q_heads=8, num_kv_heads=2, seq_lens=(400,), cal_tokens=1500, cal_ctx=512)
    pf = P.make_problem(w, with_oracle=False)
    cb, k, v, rk, rv = _prefilled(pf, (399,), 400)
    q = G.bf16_tensor(oracle.bf16_bits(pf.q))
    ws = torch.zeros(brk.decode_workspace_bytes(cb.layout, 1, 400), dtype=torch.uint8, device="cuda")
    nk = k[:, :, 399].contiguous()
    with pytest.raises(RuntimeError):   # seq_len_out must not alias seq_len
        brk.decode_step(cb.layout, cb.seq_len, nk, nk, q, rk, rv, cb.pool, cb.page_table, cb.window, cb.seq_len,
                        ws, 400)


@pytest.mark.parametrize("t_full", [600, 650])
def test_decode_step_leaves_a_request_without_room(t_full):
    """A request whose cache has no room for the new token (seq_len >= max_seq_len) is left as it
    is -- no demote, no append, its length unchanged, flag bit 1 -- and attends over its cache as it
    stands (lengths clamped to max_seq_len); the other requests step as usual."""
    tmax = 600
    w = synth.workload(2, batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(tmax, 401), cal_tokens=1500,
                       cal_ctx=512)
    print(f"case no room, seq_len {t_full}, max_seq_len {tmax}", flush=True)
    pf = P.make_problem(w, with_oracle=False)
    a, k, v, rk, rv = _prefilled(pf, (tmax, 400), tmax)
    b, _, _, _, _ = _prefilled(pf, (tmax, 400), tmax)
    for c in (a, b):
        c.seq_len[0] = t_full
    q = G.bf16_tensor(oracle.bf16_bits(pf.q))
    nk = torch.stack([k[0, :, 0], k[1, :, 400]]).contiguous()
    nv = torch.stack([v[0, :, 0], v[1, :, 400]]).contiguous()
    # reference: request 1 alone through the demote, then decode over both requests
    out1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    win = a.window.view(2, -1)
    brk.kv_demote(a.layout, a.seq_len[1:2], nk[1:2], nv[1:2], rk, rv, a.pool, a.page_table[1:2], win[1],
                  seq_len_out=out1)
    lens_a = torch.stack([a.seq_len[0], out1[0]]).contiguous()
    ws_a = torch.zeros(brk.decode_workspace_bytes(a.layout, 2, tmax), dtype=torch.uint8, device="cuda")
    out_a = brk.decode_attn(a.layout, q, lens_a, a.window, a.pool, a.page_table, rk, rv, ws_a, tmax)
    ws_b = torch.zeros_like(ws_a)
    lens_b = torch.zeros_like(b.seq_len)
    out_b = brk.decode_step(b.layout, b.seq_len, nk, nv, q, rk, rv, b.pool, b.page_table, b.window, lens_b, ws_b,
                            tmax)
    torch.cuda.synchronize()
    assert lens_b.cpu().tolist() == [t_full, 401]
    assert torch.equal(a.pool, b.pool) and torch.equal(a.window, b.window)
    assert int(ws_b[:4].view(torch.int32).item()) & 2
    G.check_close(out_b.cpu().numpy().astype(np.float64), out_a.cpu().numpy().astype(np.float64),
                  rel=REL_STEP, abs_=ABS_STEP, tag="no room vs demote + decode")
