"""Pins of the oracle's quantiser, bf16 rounding and packing (no GPU)."""
import numpy as np
import pytest
import torch

import oracle
import synth


def test_bf16_known_patterns():
    vals = np.array([1.0, -2.0, 0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                     3.140625, 65504.0], np.float32)
    bits = oracle.bf16_bits(vals)
    # ties go to the even pattern: 1+2^-8 is halfway between 0x3F80 and 0x3F81
    assert list(bits[:6]) == [0x3F80, 0xC000, 0x0000, 0x3F80, 0x3F82, 0x3F81]
    assert oracle.bf16_from_bits(np.uint16(0x4049))[()] == np.float32(3.140625)


def test_bf16_matches_torch():
    x = synth.standard_rows(1, 200, 64, scale=30.0).ravel()
    x = np.concatenate([x, np.float32(1.0) + np.arange(-300, 300, dtype=np.float32) * np.float32(2 ** -9)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits(x), ref)


def _brute_codes(x, bits, clip):
    """Nearest level by exhaustive search in fp64, ties to the even code, on the grid the
    stored (bf16) scale and zero define; also returns the gap to the runner-up."""
    x = np.asarray(x, np.float32)
    lo = np.float32(np.float32(clip) * x.min())
    hi = np.float32(np.float32(clip) * x.max())
    s = oracle.bf16_round(np.float32((hi - lo) / np.float32((1 << bits) - 1)))[()]
    z = oracle.bf16_round(lo)[()]
    codes, gaps = [], []
    for xi in x:
        xc = min(max(float(xi), float(lo)), float(hi))
        dist = [abs(xc - (float(z) + k * float(s))) for k in range(1 << bits)]
        order = sorted(range(1 << bits), key=lambda k: (dist[k], k % 2, k))
        codes.append(order[0])
        gaps.append((dist[order[1]] - dist[order[0]]) / float(s))
    return np.array(codes), np.array(gaps), s, z


@pytest.mark.parametrize("bits,clip", [(2, 0.96), (2, 0.92), (2, 1.0), (4, 1.0), (4, 0.9)])
def test_quantize_group_brute_force(bits, clip):
    r = np.random.default_rng(11 + bits)
    for trial in range(60):
        g = (r.standard_normal(64) * r.uniform(0.01, 50)).astype(np.float32)
        codes, s_b, z_b = oracle.quantize_group(g, bits, clip)
        ref, gaps, s, z = _brute_codes(g, bits, clip)
        assert oracle.bf16_from_bits(s_b)[()] == s and oracle.bf16_from_bits(z_b)[()] == z
        clear = gaps > 1e-4      # away from a tie the answer is unique
        assert np.array_equal(codes[clear], ref[clear])
        assert codes.max() <= (1 << bits) - 1


def test_quantize_exact_ties_go_even():
    # s = 1, z = 0 after bf16 rounding; points exactly half-way between levels
    g = np.array([0.0, 3.0, 0.5, 1.5, 2.5, 1.0], np.float32)
    codes, s_b, z_b = oracle.quantize_group(g, 2, 1.0)
    assert oracle.bf16_from_bits(s_b)[()] == 1.0 and oracle.bf16_from_bits(z_b)[()] == 0.0
    assert list(codes) == [0, 3, 0, 2, 2, 1]
    rc, rsz = oracle.quantize_rows(g[None], 6, 2, 1.0)
    assert list(rc[0]) == [0, 3, 0, 2, 2, 1]


def test_quantize_constant_group_is_zero_codes():
    for v in (0.0, 3.7, -1e-3):
        codes, s_b, z_b = oracle.quantize_group(np.full(32, v, np.float32), 2, 0.96)
        assert np.all(codes == 0) and oracle.bf16_from_bits(s_b)[()] == 0.0
        assert np.allclose(oracle.dequantize_rows(codes[None], np.array([[[s_b, z_b]]], np.uint16), 32),
                           oracle.bf16_round(np.float32(0.96) * np.float32(v)))


def test_quantize_on_grid_reconstructs_exactly():
    g = np.array([-1.0, -0.5, 0.0, 0.5, -1.0, 0.5, 0.0, -0.5], np.float32)
    codes, sz = oracle.quantize_rows(g[None], 8, 2, 1.0)
    assert list(codes[0]) == [0, 1, 2, 3, 0, 3, 2, 1]
    assert np.array_equal(oracle.dequantize_rows(codes, sz, 8)[0], g.astype(np.float64))


def test_quantize_clip_saturates():
    g = np.array([-10.0, -1.0, 0.0, 1.0, 10.0, 9.9, -9.9, 5.0], np.float32)
    codes, s_b, z_b = oracle.quantize_group(g, 2, 0.5)
    assert codes[0] == 0 and codes[4] == 3 and codes[5] == 3 and codes[6] == 0


@pytest.mark.parametrize("bits", [2, 4])
def test_quantize_rows_equals_groupwise(bits):
    x = synth.standard_rows(3, 40, 128, scale=4.0)
    for group in (32, 64, 128):
        codes, sz = oracle.quantize_rows(x, group, bits, 0.96)
        for i in range(0, 40, 7):
            for gi in range(128 // group):
                c, s_b, z_b = oracle.quantize_group(x[i, gi * group:(gi + 1) * group], bits, 0.96)
                assert np.array_equal(codes[i, gi * group:(gi + 1) * group], c)
                assert sz[i, gi, 0] == s_b and sz[i, gi, 1] == z_b


def test_pack_known_bytes():
    assert oracle.pack_codes(np.array([[0, 1, 2, 3]]), 2)[0, 0] == 0xE4
    assert oracle.pack_codes(np.array([[1, 2]]), 4)[0, 0] == 0x21
    assert oracle.pack_codes(np.array([[3, 0, 0, 0, 0, 0, 0, 2]]), 2).tolist() == [[0x03, 0x80]]


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_round_trip(bits):
    r = np.random.default_rng(12)
    c = r.integers(0, 1 << bits, size=(17, 128)).astype(np.uint8)
    p = oracle.pack_codes(c, bits)
    assert p.shape == (17, 128 * bits // 8)
    assert np.array_equal(oracle.unpack_codes(p, bits, 128), c)


def test_rotate_rows_rounds_once():
    r = np.random.default_rng(13)
    x = oracle.bf16_round(r.standard_normal((5, 16)).astype(np.float32))
    rot = synth.random_orthogonal(r, 16).astype(np.float32)
    got = oracle.rotate_rows_fp32(x, rot)
    for i in range(5):
        for j in range(16):
            exact = sum(float(x[i, k]) * float(rot[k, j]) for k in range(16))
            assert got[i, j] == np.float32(exact) or abs(float(got[i, j]) - exact) <= 6e-8 * abs(exact)


def test_bitrev_only_permutes_codes_when_group_is_full_row():
    """With one group per row, rotating by an extra P_br only reorders the codes."""
    d = 64
    r = np.random.default_rng(14)
    x = r.standard_normal((20, d)).astype(np.float32)
    p = oracle.bitrev_indices(d)
    xp = x[:, np.argsort(p)]          # x . P_br: entry rev(i) takes x[i]
    assert np.array_equal(xp[:, p], x)
    c1, s1 = oracle.quantize_rows(x, d, 2, 0.96)
    c2, s2 = oracle.quantize_rows(xp, d, 2, 0.96)
    assert np.array_equal(c2[:, p], c1) and np.array_equal(s1, s2)
