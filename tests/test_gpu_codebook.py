"""The Lloyd-Max INT2 codebook on the GPU against the oracle: the codebook quantiser bit for bit on
the same fp32 rotated rows (also next to every decision threshold), decode attention over
oracle-written and GPU-written codebook caches (rel-L2 <= 5e-3, max-abs <= 1e-2), the prefill and
the per-step demote writing the same cache bit for bit, the fused step against demote + decode,
and the uniform levels reproducing the uniform codec."""
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


def _cases_levels():
    r = np.random.default_rng(77)
    out = [("uniform", oracle.fp16_levels(oracle.UNIFORM_LEVELS)),
           ("lloyd-gauss", oracle.fp16_levels([0.55, 1.21, 1.79, 2.45])),
           ("skewed", oracle.fp16_levels([0.02, 0.4, 1.3, 2.97]))]
    for i in range(3):
        out.append((f"random{i}", oracle.fp16_levels(np.sort(r.uniform(-0.2, 3.2, 4)) + np.arange(4) * 1e-2)))
    return out


def gpu_qp_cb(x, group, clip, levels):
    codes, sz = brk.quantize_pack_codebook(torch.from_numpy(x).cuda(), group, clip, oracle.fp16_patterns(levels))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sz.cpu().numpy().view(np.uint16)


def oracle_qp_cb(x, group, clip, levels):
    c, sz = oracle.quantize_rows_codebook(x, group, clip, levels)
    return oracle.pack_codes(c, 2), sz


@pytest.mark.parametrize("name,levels", _cases_levels())
@pytest.mark.parametrize("dim,group,clip", [(128, 128, 0.96), (128, 32, 0.92), (64, 64, 1.0), (96, 16, 0.9)])
def test_quantize_pack_codebook_bit_exact(name, levels, dim, group, clip):
    print(f"case {name} dim {dim} group {group}", flush=True)
    x = synth.standard_rows(31 + dim + group, 700, dim, scale=2.5)
    x[::9, :3] *= 40.0                       # outliers: clipping at both ends
    gc, gs = gpu_qp_cb(x, group, clip, levels)
    oc, os_ = oracle_qp_cb(x, group, clip, levels)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


def test_quantize_pack_codebook_next_to_thresholds():
    """Coordinates on, and 2^-24 .. 2^-11 away from, every threshold (where the reciprocal estimate
    must defer to the exact division), for several scales."""
    levels = oracle.fp16_levels([0.3, 1.1, 1.75, 2.6])
    t = oracle.thresholds_fp32(levels).astype(np.float64)
    rows = []
    for s in (0.7109375, 0.01171875, 13.5, 1.0):          # bf16 scales: hi = 3 s with lo = 0, clip 1
        row = [0.0, 3.0 * s]
        for tj in t:
            for k in range(-14, 15):
                d = 0.0 if k == 0 else np.sign(k) * 2.0 ** (-24 + 1 * (abs(k) - 1))
                row.append((tj + d) * s)
        row = np.array(row, np.float32)
        row = np.concatenate([row, np.full(128 - len(row) % 128, 0.5 * s, np.float32)]) if len(row) % 128 else row
        rows.append(row[:128])
    x = np.stack(rows).astype(np.float32)
    gc, gs = gpu_qp_cb(x, 128, 1.0, levels)
    oc, os_ = oracle_qp_cb(x, 128, 1.0, levels)
    assert np.array_equal(gs, os_) and np.array_equal(gc, oc)


def test_uniform_codebook_equals_uniform_quantiser():
    x = synth.standard_rows(5, 500, 128, scale=3.0)
    a, sa = gpu_qp_cb(x, 32, 0.96, oracle.fp16_levels(oracle.UNIFORM_LEVELS))
    b, sb = brk.quantize_pack(torch.from_numpy(x).cuda(), 32, 2, 0.96)
    torch.cuda.synchronize()
    assert np.array_equal(a, b.cpu().numpy()) and np.array_equal(sa, sb.cpu().numpy().view(np.uint16))


def small(base, **kw):
    kw.setdefault("cal_tokens", 1500)
    kw.setdefault("cal_ctx", 512)
    return synth.workload(base, **kw)


DECODE = {
    "d128-gq4": lambda: small(2, batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(1800, 1000)),
    "d128-gq8": lambda: small(4, batch=2, num_q_heads=16, num_kv_heads=2, seq_lens=(1200, 2500)),
    "d128-gq1": lambda: small(2, batch=1, num_q_heads=2, num_kv_heads=2, seq_lens=(1500,)),
    "d128-gq2": lambda: small(2, batch=1, num_q_heads=4, num_kv_heads=2, seq_lens=(1100,)),
    "d64-gq4": lambda: synth.workload(1, num_q_heads=8, num_kv_heads=2, batch=2, seq_lens=(900, 2100)),
    "edge-lengths": lambda: small(2, batch=12, num_q_heads=4, num_kv_heads=1,
                                  seq_lens=(0, 1, 64, 319, 320, 321, 336, 337, 352, 353, 700, 1500)),
    "mixed": lambda: small(5, batch=3, num_q_heads=8, num_kv_heads=2, seq_lens=(1500, 700, 2300)),
}


@pytest.fixture(scope="module", params=sorted(DECODE))
def prob(request):
    print(f"case {request.param}", flush=True)
    p = P.make_problem(DECODE[request.param](), codebook="fit")
    ref = np.stack([oracle.decode_attention(p.caches[b], p.q[b]) for b in range(p.w.batch)])
    return request.param, p, ref


def test_codebook_decode_oracle_written_cache(prob):
    name, p, ref = prob
    cb, rk, rv = G.build_cache(p, oracle_written=True)
    got, ws = G.decode(p, cb, rk, rv)
    worst, mab = G.check_close(got, ref, tag=name)
    # same codes on both sides: the level products are rounded in fp32 (not exact as for the
    # uniform codes), still far inside the bar
    assert worst <= 5e-4, f"{name}: {worst:.2e}"
    assert int(ws[:4].view(torch.int32).item()) == 0
    print(f"{name}: codebook oracle-written worst rel-L2 {worst:.2e} max-abs {mab:.2e}")


def test_codebook_decode_gpu_written_cache(prob):
    name, p, ref = prob
    cb, rk, rv = G.build_cache(p, oracle_written=False)
    got, _ = G.decode(p, cb, rk, rv)
    worst, mab = G.check_close(got, ref, tag=name)
    print(f"{name}: codebook gpu-written worst rel-L2 {worst:.2e} max-abs {mab:.2e}")


def test_codebook_prefill_history_matches_oracle():
    p = P.make_problem(small(2, batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(2000, 700)), codebook="fit")
    cb, rk, rv = G.build_cache(p, oracle_written=False)
    pool = cb.pool.cpu().numpy()
    pt2 = cb.page_table.cpu().numpy()
    n_el = n_diff = 0
    for b in range(p.w.batch):
        for kv in range(p.w.num_kv_heads):
            ok, ov, osk, osv = P.oracle_history(p.caches[b], kv, 2)
            gk, gv, gsk, gsv = layout_ref.read_history(pool, p.w.head_dim, p.w.num_kv_heads, cb.layout.pool_pages,
                                                       kv, 2, pt2[b], len(ok))
            for gc, oc in ((gk, ok), (gv, ov)):
                diff = np.abs(gc.astype(int) - oc.astype(int))
                assert diff.max(initial=0) <= 1
                n_el += diff.size
                n_diff += int((diff > 0).sum())
            for gs, os_ in ((gsk, osk), (gsv, osv)):
                assert np.abs(gs.astype(np.int64) - os_.astype(np.int64)).max(initial=0) <= 1
    print(f"history elements {n_el}, codes off by one level: {n_diff}")
    assert n_el > 0 and n_diff <= 1e-3 * n_el


def _prefill(p, t0, tmax):
    cb = G.allocate(p, tmax)
    k = G.bf16_tensor(P.kv_bits_tensor(p, "k"))
    v = G.bf16_tensor(P.kv_bits_tensor(p, "v"))
    tb = torch.from_numpy(P.bits_tensor(p)).cuda() if p.mixed else None
    cb.seq_len.copy_(torch.tensor(list(t0), dtype=torch.int32))
    rk = torch.from_numpy(p.rot_k).cuda()
    rv = torch.from_numpy(p.rot_v).cuda()
    brk.kv_prefill(cb.layout, cb.seq_len, k, v, rk, rv, cb.pool, cb.page_table, cb.window, token_bits=tb,
                   page_table4=cb.page_table4, n_int4_out=cb.n_int4)
    return cb, k, v, rk, rv


def _demote_bits(p, pos):
    if not p.mixed:
        return None
    return torch.tensor([int(p.bits[b][pos[b] - 256]) if pos[b] >= 320 else 2 for b in range(p.w.batch)],
                        dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("base,kw,steps", [
    (2, dict(batch=2, num_q_heads=4, num_kv_heads=2, seq_lens=(300, 500)), 40),
    (5, dict(batch=2, num_q_heads=4, num_kv_heads=2, seq_lens=(500, 700)), 30),
])
def test_codebook_demote_steps_equal_prefill(base, kw, steps):
    print(f"case base={base} steps={steps}", flush=True)
    t0 = kw["seq_lens"]
    w = small(base, **dict(kw, seq_lens=tuple(t + steps for t in t0)))
    p = P.make_problem(w, with_oracle=False, codebook="fit")
    tmax = max(w.seq_lens)
    ref, _, _ = G.build_cache(p, oracle_written=False)
    cb, k, v, rk, rv = _prefill(p, t0, tmax)
    seq = [cb.seq_len, torch.zeros_like(cb.seq_len)]
    n4 = [cb.n_int4, torch.zeros_like(cb.n_int4)] if p.mixed else [None, None]
    for i in range(steps):
        pos = [t + i for t in t0]
        nk = torch.stack([k[b, :, pos[b]] for b in range(w.batch)]).contiguous()
        nv = torch.stack([v[b, :, pos[b]] for b in range(w.batch)]).contiguous()
        brk.kv_demote(cb.layout, seq[i % 2], nk, nv, rk, rv, cb.pool, cb.page_table, cb.window, n_int4=n4[i % 2],
                      demote_bits=_demote_bits(p, pos), page_table4=cb.page_table4, seq_len_out=seq[(i + 1) % 2],
                      n_int4_out=n4[(i + 1) % 2])
    torch.cuda.synchronize()
    assert torch.equal(cb.window, ref.window)
    assert torch.equal(cb.pool, ref.pool)


@pytest.mark.parametrize("name,base,kw", [
    ("int2-d128-gq4", 2, dict(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(1000, 400))),
    ("int2-d64-gq8", 1, dict(batch=2, num_q_heads=16, num_kv_heads=2, seq_lens=(330, 900))),
    ("mixed-d128-gq4", 5, dict(batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(1200, 700))),
])
def test_codebook_step_equals_demote_then_decode(name, base, kw):
    print(f"case {name}", flush=True)
    steps = 4
    t0 = kw["seq_lens"]
    w = small(base, **dict(kw, seq_lens=tuple(t + steps for t in t0)))
    p = P.make_problem(w, codebook="fit")
    tmax = max(w.seq_lens)
    a, k, v, rk, rv = _prefill(p, t0, tmax)
    b, _, _, _, _ = _prefill(p, t0, tmax)
    q = G.bf16_tensor(oracle.bf16_bits(p.q))
    ws_a = torch.zeros(brk.decode_workspace_bytes(a.layout, w.batch, tmax), dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    seq_a = [a.seq_len, torch.zeros_like(a.seq_len)]
    seq_b = [b.seq_len, torch.zeros_like(b.seq_len)]
    n4_a = [a.n_int4, torch.zeros_like(a.n_int4)] if p.mixed else [None, None]
    n4_b = [b.n_int4, torch.zeros_like(b.n_int4)] if p.mixed else [None, None]
    for i in range(steps):
        pos = [t + i for t in t0]
        nk = torch.stack([k[bb, :, pos[bb]] for bb in range(w.batch)]).contiguous()
        nv = torch.stack([v[bb, :, pos[bb]] for bb in range(w.batch)]).contiguous()
        db = _demote_bits(p, pos)
        cur, nxt = i % 2, (i + 1) % 2
        brk.kv_demote(a.layout, seq_a[cur], nk, nv, rk, rv, a.pool, a.page_table, a.window, n_int4=n4_a[cur],
                      demote_bits=db, page_table4=a.page_table4, seq_len_out=seq_a[nxt], n_int4_out=n4_a[nxt])
        out_a = brk.decode_attn(a.layout, q, seq_a[nxt], a.window, a.pool, a.page_table, rk, rv, ws_a, tmax,
                                n_int4=n4_a[nxt], page_table4=a.page_table4)
        out_b = brk.decode_step(b.layout, seq_b[cur], nk, nv, q, rk, rv, b.pool, b.page_table, b.window, seq_b[nxt],
                                ws_b, tmax, n_int4=n4_b[cur], n_int4_out=n4_b[nxt], demote_bits=db,
                                page_table4=b.page_table4)
        torch.cuda.synchronize()
        assert torch.equal(a.pool, b.pool) and torch.equal(a.window, b.window), f"{name}: step {i} cache differs"
        G.check_close(out_b.cpu().numpy().astype(np.float64), out_a.cpu().numpy().astype(np.float64),
                      rel=1e-4, abs_=2e-3, tag=f"{name} step {i} vs demote + decode")
    ref = np.stack([oracle.decode_attention(p.caches[bb], p.q[bb]) for bb in range(w.batch)])
    worst, mab = G.check_close(out_b.cpu().numpy().astype(np.float64), ref, tag=name)
    print(f"{name}: codebook step worst rel-L2 {worst:.2e} max-abs {mab:.2e}")


def test_uniform_codebook_table_reproduces_the_uniform_codec():
    """A table holding the levels 0, 1, 2, 3 writes the uniform cache byte for byte, and its decode
    (levels through the byte permute) agrees with the uniform decode to fp32 rounding."""
    w = small(2, batch=2, num_q_heads=8, num_kv_heads=2, seq_lens=(1500, 800))
    uni = np.broadcast_to(oracle.fp16_levels(oracle.UNIFORM_LEVELS), (2, 2, 4)).copy()
    pu = P.make_problem(w, with_oracle=False, codebook=uni)
    pn = P.make_problem(w, with_oracle=False)
    cu, rk, rv = G.build_cache(pu, oracle_written=False)
    cn, _, _ = G.build_cache(pn, oracle_written=False)
    assert torch.equal(cu.pool, cn.pool) and torch.equal(cu.window, cn.window)
    gu, _ = G.decode(pu, cu, rk, rv)
    gn, _ = G.decode(pn, cn, rk, rv)
    # the two decodes differ only in how the low parts of the query operands are scaled into fp16
    # (per code bit position, or not at all): fp32-rounding-level differences of the logits
    G.check_close(gu, gn, rel=5e-5, abs_=2e-3, tag="uniform table vs uniform codec")


# ---------------------------------------------------------------- Lloyd-Max fit on the GPU
def _fit_inputs(w, n_rows, which, identity):
    """Calibration rows [Hkv, n, d] (bf16 values) of the workload's channel law and the rotations."""
    rk, rv = P.rotations(w) if not identity else (None, None)
    d, hkv = w.head_dim, w.num_kv_heads
    rows = np.zeros((hkv, n_rows, d), np.float32)
    rot = np.zeros((hkv, d, d), np.float32)
    for kv in range(hkv):
        kc, vc = synth.calibration_context(w, kv)
        x = (kc if which == "k" else vc)[:n_rows]
        rows[kv, :len(x)] = oracle.bf16_round(x.astype(np.float32))
        rot[kv] = np.eye(d, dtype=np.float32) if identity else (rk if which == "k" else rv)[kv]
    return rows, rot


def _gpu_fit(rows, rot, clip, max_iter=100, tol=1e-7):
    x = G.bf16_tensor(oracle.bf16_bits(rows))
    r = torch.from_numpy(rot).cuda()
    lv, pats, it = brk.codebook_fit(x, r, clip, max_iter=max_iter, tol=tol)
    return lv, pats.view(np.uint16), it


@pytest.mark.parametrize("which,clip,n_rows", [("k", 0.96, 512), ("v", 0.92, 500), ("k", 1.0, 77)])
def test_codebook_fit_identity_rotation_matches_oracle(which, clip, n_rows):
    """With R = I the writers' rotation is exact, so the GPU sees the oracle's coordinates bit for
    bit: the fits differ only in the order of the fp64 cell sums."""
    print(f"case identity {which} n={n_rows}", flush=True)
    w = small(2, num_q_heads=8, num_kv_heads=2)
    rows, rot = _fit_inputs(w, n_rows, which, identity=True)
    lv, pats, it = _gpu_fit(rows, rot, clip)
    for kv in range(w.num_kv_heads):
        u, ok = oracle.group_coordinates(rows[kv], w.group_size, clip)
        ref, rit, _ = oracle.lloyd_max(u[ok], max_iter=100, tol=1e-7)
        assert np.allclose(lv[kv], ref, rtol=0, atol=1e-12), (kv, lv[kv], ref)
        assert np.array_equal(pats[kv], oracle.fp16_patterns(ref))
        assert it[kv] == rit
    print(f"levels {lv.tolist()} iterations {it.tolist()}")


@pytest.mark.parametrize("which,clip", [("k", 0.96), ("v", 0.92)])
def test_codebook_fit_with_rotation_matches_oracle(which, clip):
    """Calibration rows rotated by the workload's OSCAR rotations: the writers' rotation and the
    oracle's fp64 one differ in the last fp32 bits, which moves a level by far less than 1e-5."""
    print(f"case rotated {which}", flush=True)
    w = small(2, num_q_heads=8, num_kv_heads=2)
    rows, rot = _fit_inputs(w, 512, which, identity=False)
    lv, pats, it = _gpu_fit(rows, rot, clip)
    for kv in range(w.num_kv_heads):
        ref, ref16, rit = oracle.fit_codebook(oracle.rotate_rows_fp32(rows[kv], rot[kv]), w.group_size, clip)
        assert np.abs(lv[kv] - ref).max() < 1e-5, (kv, lv[kv], ref)
        gp = pats[kv].astype(np.int64)
        rp = oracle.fp16_patterns(ref).astype(np.int64)
        assert np.abs(gp - rp).max() <= 1
    print(f"levels {lv.tolist()} iterations {it.tolist()}")


def test_codebook_fit_edge_rows():
    """Constant rows (scale 0) carry no coordinates; a ragged row count; one iteration only."""
    w = small(2, num_q_heads=4, num_kv_heads=1)
    rows, rot = _fit_inputs(w, 130, "k", identity=True)
    rows[0, 5:40] = 1.5                              # constant rows: no coordinates
    lv, pats, it = _gpu_fit(rows, rot, 0.96, max_iter=1)
    u, ok = oracle.group_coordinates(rows[0], w.group_size, 0.96)
    assert (~ok).sum() == 35 * w.head_dim
    ref, rit, _ = oracle.lloyd_max(u[ok], max_iter=1)
    assert it[0] == 1 == rit and np.allclose(lv[0], ref, rtol=0, atol=1e-12)
    # all rows constant: the uniform levels come back after one iteration
    rows[0, :] = -0.25
    lv, pats, it = _gpu_fit(rows, rot, 0.96)
    assert lv[0].tolist() == [0.0, 1.0, 2.0, 3.0] and it[0] == 1
