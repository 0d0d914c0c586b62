"""oscar_decode_step_noalloc (the decode step with the library's own per-device workspace, for
callers that cannot allocate) against oscar_decode_step with a caller workspace: two calls in a
row on one device, the second smaller than the first (fewer requests, shorter histories, the other
split width), each on caches prefilled alike. Both run the same kernels on the same plan, so the
cache they leave and their outputs agree bit for bit."""
import pytest
import torch

import bit_rotated_kv_amd as brk
import gpu_util as G
import oracle
import problem as P
import synth

pytestmark = pytest.mark.gpu


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


# first call: 3 requests x 8 kv-heads (4-wavefront split workgroups); second: 1 request (16-wavefront)
CALLS = [
    dict(base=2, batch=3, num_q_heads=32, num_kv_heads=8, seq_lens=(1400, 333, 2100)),
    dict(base=3, batch=1, num_q_heads=32, num_kv_heads=8, seq_lens=(900,)),
]


def test_noalloc_step_matches_the_workspace_step_twice():
    for n, kw in enumerate(CALLS):
        kw = dict(kw)
        base = kw.pop("base")
        print(f"no-alloc call {n}: batch {kw['batch']} seq_lens {kw['seq_lens']}", flush=True)
        t0 = tuple(t - 1 for t in kw["seq_lens"])
        w = synth.workload(base, **dict(kw, cal_tokens=1500, cal_ctx=512))
        pf = P.make_problem(w, with_oracle=False)
        tmax = max(w.seq_lens)
        a, k, v, rk, rv = _prefilled(pf, t0, tmax)
        b, _, _, _, _ = _prefilled(pf, t0, tmax)
        q = G.bf16_tensor(oracle.bf16_bits(pf.q))
        nk = torch.stack([k[bb, :, t0[bb]] for bb in range(w.batch)]).contiguous()
        nv = torch.stack([v[bb, :, t0[bb]] for bb in range(w.batch)]).contiguous()
        ws = torch.zeros(brk.decode_workspace_bytes(a.layout, w.batch, tmax), dtype=torch.uint8, device="cuda")
        assert ws.numel() <= brk.ops.NOALLOC_SCRATCH_BYTES
        lens_a = torch.zeros_like(a.seq_len)
        lens_b = torch.zeros_like(b.seq_len)
        out_a = brk.decode_step(a.layout, a.seq_len, nk, nv, q, rk, rv, a.pool, a.page_table, a.window, lens_a, ws,
                                tmax)
        out_b = torch.full_like(out_a, float("nan"))
        brk.decode_step_noalloc(b.layout, b.seq_len, nk, nv, q, rk, rv, b.pool, b.page_table, b.window, lens_b,
                                tmax, out_b)
        torch.cuda.synchronize()
        assert lens_b.cpu().tolist() == list(w.seq_lens)
        assert torch.equal(lens_a, lens_b)
        assert torch.equal(a.pool, b.pool), f"call {n}: history pages differ"
        assert torch.equal(a.window, b.window), f"call {n}: window differs"
        assert torch.isfinite(out_b).all()
        assert torch.equal(out_a, out_b), f"call {n}: outputs differ, max {(out_a - out_b).abs().max().item()}"
