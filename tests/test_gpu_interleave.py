"""The one-request launch with interleaved history pages (a batch of one, GQA 4 at 8 kv-heads,
INT2-only, max_seq_len long enough for it): decode attention against the oracle at short and
edge lengths (units and wavefronts without pages, a lone page, ragged last pages), skipped page
ids at several positions of the interleave, determinism, and the fused step against demote +
decode over several steps (caches bit for bit, outputs to fp32 rounding)."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_amd as brk
import gpu_util as G
import oracle
import problem as P
import synth

pytestmark = pytest.mark.gpu

HQ, HKV = 32, 8
# max_seq_len of the buffers: its history (2,480 pages) gives the 31 history units of each kv-head
# more than 64 pages each, which selects the interleaved launch; the requests themselves are shorter
TMAX = 40_000


def _workload(T, base=2, **kw):
    return synth.workload(base, batch=1, num_q_heads=HQ, num_kv_heads=HKV, seq_lens=(T,), cal_tokens=1500,
                          cal_ctx=512, **kw)


def _cache(p, oracle_written, tmax=TMAX, t0=None):
    """Buffers for TMAX tokens (a page table covering all of them, a seeded permutation of the
    pool), filled with the problem's tokens up to its length (or t0)."""
    w = p.w
    hp = (tmax - 320 + 15) // 16
    order = np.random.default_rng(11).permutation(hp)
    cb = brk.allocate_cache(HQ, HKV, w.head_dim, 1, tmax, pages2_per_request=hp, page_order2=order)
    T = w.seq_lens[0] if t0 is None else t0
    cb.seq_len.fill_(T)
    rk = torch.from_numpy(p.rot_k).cuda()
    rv = torch.from_numpy(p.rot_v).cuda()
    if oracle_written:
        pool, win = P.oracle_pool_and_window(p, cb.layout, cb.page_table.cpu().numpy(), None, cb.pool.numel(),
                                             cb.window.numel())
        cb.pool.copy_(torch.from_numpy(pool))
        cb.window.copy_(torch.from_numpy(np.ascontiguousarray(win)))
        k = v = None
    else:
        k = G.bf16_tensor(P.kv_bits_tensor(p, "k"))
        v = G.bf16_tensor(P.kv_bits_tensor(p, "v"))
        pad = tmax - k.shape[2]
        kp = torch.nn.functional.pad(k, (0, 0, 0, pad)).contiguous()
        vp = torch.nn.functional.pad(v, (0, 0, 0, pad)).contiguous()
        brk.kv_prefill(cb.layout, cb.seq_len, kp, vp, rk, rv, cb.pool, cb.page_table, cb.window)
    torch.cuda.synchronize()
    return cb, rk, rv, k, v


def _decode(p, cb, rk, rv, max_seq_len=TMAX):
    """decode_attn over the buffers; max_seq_len = TMAX selects the interleaved launch, the
    request's own length the general plan."""
    q = G.bf16_tensor(oracle.bf16_bits(p.q))
    ws = torch.zeros(brk.decode_workspace_bytes(cb.layout, 1, TMAX), dtype=torch.uint8, device="cuda")
    out = brk.decode_attn(cb.layout, q, cb.seq_len, cb.window, cb.pool, cb.page_table, rk, rv, ws, max_seq_len)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), ws


# 0 and 1 token; the sink boundary; one history token (one page on one unit); 24 history pages (some
# units with one page, most with none); a ragged last page over every unit; several pages per
# wavefront on some units (9,000: 543 pages)
LENGTHS = [0, 1, 64, 321, 700, 5_000, 9_000]


@pytest.mark.parametrize("T", LENGTHS)
def test_interleaved_decode_matches_oracle(T):
    print(f"case interleaved decode T={T}", flush=True)
    p = P.make_problem(_workload(T))
    ref = oracle.decode_attention(p.caches[0], p.q[0])[None]
    cb, rk, rv, _, _ = _cache(p, oracle_written=True)
    got, ws = _decode(p, cb, rk, rv)
    worst, mab = G.check_close(got, ref, tag=f"interleaved T={T}")
    # Same codes on both sides. At 8 kv-heads this workload has heads whose error against the oracle
    # reaches 1.2e-4 whatever the history length, on the general plan too: held to 5e-4 here, and
    # the interleaved launch is held to the general plan's result on the same buffers to 1e-5.
    assert worst <= 5e-4, f"T={T}: {worst:.2e}"
    assert int(ws[:4].view(torch.int32).item()) == 0
    gen, _ = _decode(p, cb, rk, rv, max_seq_len=max(T, 1))
    G.check_close(got, gen, rel=1e-5, abs_=5e-4, tag=f"interleaved vs general plan T={T}")
    cb, rk, rv, _, _ = _cache(p, oracle_written=False)
    got2, _ = _decode(p, cb, rk, rv)
    G.check_close(got2, ref, tag=f"interleaved gpu-written T={T}")
    print(f"T={T}: oracle-written worst rel-L2 {worst:.2e} max-abs {mab:.2e}")


def test_interleaved_decode_is_deterministic():
    p = P.make_problem(_workload(6_000), with_oracle=False)
    cb, rk, rv, _, _ = _cache(p, oracle_written=False)
    a, _ = _decode(p, cb, rk, rv)
    b, _ = _decode(p, cb, rk, rv)
    assert np.array_equal(a, b)


# history page indices whose ids are replaced by ids beyond the pool: pages of the first unit's
# first and second list entries (0, 31 * 16 = 496), of unit 30 (30), and of consecutive units (7, 8)
@pytest.mark.parametrize("bad", [(0,), (30,), (7, 8), (496,), (0, 496, 31)])
def test_interleaved_decode_skips_out_of_range_page_ids(bad):
    print(f"case interleaved skip {bad}", flush=True)
    p = P.make_problem(_workload(9_000))
    cb, rk, rv, _, _ = _cache(p, oracle_written=True)
    for i in bad:
        cb.page_table[0, i] = cb.layout.pool_pages + i
    got, ws = _decode(p, cb, rk, rv)
    assert int(ws[:4].view(torch.int32).item()) & 1
    assert np.all(np.isfinite(got))
    c = p.caches[0]
    keep = np.ones(len(c.hist_pos), bool)
    order = np.argsort(c.hist_pos)
    for i in bad:
        keep[order[16 * i:16 * (i + 1)]] = False
    for attr in ("hist_pos", "hist_bits"):
        setattr(c, attr, getattr(c, attr)[keep])
    for attr in ("k_codes", "v_codes", "k_sz", "v_sz"):
        setattr(c, attr, getattr(c, attr)[:, keep])
    G.check_close(got, oracle.decode_attention(c, p.q[0])[None], tag=f"interleaved skip {bad}")


STEPS = 4
REL_STEP, ABS_STEP = 5e-5, 2e-3


@pytest.mark.parametrize("t0", [317, 3_000])
def test_interleaved_step_equals_demote_then_decode(t0):
    """The fused step in the interleaved launch (step and window on unit 0) against kv_demote +
    decode_attn (itself interleaved): caches bit for bit after every step, outputs to fp32 rounding,
    the last output against the oracle."""
    print(f"case interleaved step t0={t0}", flush=True)
    p = P.make_problem(_workload(t0 + STEPS))
    a, rk, rv, k, v = _cache(p, oracle_written=False, t0=t0)
    b, _, _, _, _ = _cache(p, oracle_written=False, t0=t0)
    q = G.bf16_tensor(oracle.bf16_bits(p.q))
    ws_a = torch.zeros(brk.decode_workspace_bytes(a.layout, 1, TMAX), dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    seq_a = [a.seq_len, torch.zeros_like(a.seq_len)]
    seq_b = [b.seq_len, torch.zeros_like(b.seq_len)]
    for i in range(STEPS):
        nk = k[:, :, t0 + i].contiguous()
        nv = v[:, :, t0 + i].contiguous()
        cur, nxt = i % 2, (i + 1) % 2
        brk.kv_demote(a.layout, seq_a[cur], nk, nv, rk, rv, a.pool, a.page_table, a.window, seq_len_out=seq_a[nxt])
        out_a = brk.decode_attn(a.layout, q, seq_a[nxt], a.window, a.pool, a.page_table, rk, rv, ws_a, TMAX)
        out_b = brk.decode_step(b.layout, seq_b[cur], nk, nv, q, rk, rv, b.pool, b.page_table, b.window, seq_b[nxt],
                                ws_b, TMAX)
        torch.cuda.synchronize()
        assert torch.equal(seq_a[nxt], seq_b[nxt]), f"step {i} lengths differ"
        assert torch.equal(a.pool, b.pool), f"step {i} history pages differ"
        assert torch.equal(a.window, b.window), f"step {i} window differs"
        G.check_close(out_b.cpu().numpy().astype(np.float64), out_a.cpu().numpy().astype(np.float64),
                      rel=REL_STEP, abs_=ABS_STEP, tag=f"interleaved step {i} vs demote + decode")
    assert seq_b[STEPS % 2].cpu().tolist() == [t0 + STEPS]
    ref = oracle.decode_attention(p.caches[0], p.q[0])[None]
    worst, mab = G.check_close(out_b.cpu().numpy().astype(np.float64), ref, tag=f"interleaved step t0={t0}")
    print(f"t0={t0}: worst rel-L2 {worst:.2e} max-abs {mab:.2e}")


def test_interleaved_decode_reuses_a_dirty_workspace():
    """A workspace holding garbage (report word aside), reused call after call, gives the
    fresh-workspace result every time in the interleaved launch."""
    p = P.make_problem(_workload(5_000), with_oracle=False)
    cb, rk, rv, _, _ = _cache(p, oracle_written=False)
    ref, _ = _decode(p, cb, rk, rv)
    q = G.bf16_tensor(oracle.bf16_bits(p.q))
    for fill in (0x5A, 0x00, 0xFF):
        ws = torch.full((brk.decode_workspace_bytes(cb.layout, 1, TMAX),), fill, dtype=torch.uint8, device="cuda")
        ws[:4] = 0
        for _ in range(3):
            out = brk.decode_attn(cb.layout, q, cb.seq_len, cb.window, cb.pool, cb.page_table, rk, rv, ws, TMAX)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().astype(np.float64), ref), f"fill {fill:#x}"
        assert int(ws[:4].view(torch.int32).item()) == 0
