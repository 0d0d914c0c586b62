"""CPU checks of the test-side layout helper against the properties the header states."""
import numpy as np
import pytest

import layout_ref


@pytest.mark.parametrize("d,bits", [(64, 2), (128, 2), (64, 4), (128, 4)])
def test_code_positions_are_a_bijection(d, bits):
    nbits = 2 * d * bits * 16
    used = np.zeros(nbits, np.int32)
    for byte, bit in (layout_ref.key_offsets(d, bits), layout_ref.value_offsets(d, bits)):
        for k in range(bits):
            np.add.at(used, (byte * 8 + bit + k).ravel(), 1)
    assert used.min() == 1 and used.max() == 1        # every code bit exactly once, codes region full


@pytest.mark.parametrize("d,bits", [(64, 2), (128, 2), (64, 4), (128, 4)])
def test_key_lane_part_belongs_to_one_slot(d, bits):
    byte, _ = layout_ref.key_offsets(d, bits)
    cb = d * bits // 32
    if bits == 2:                                     # lane chunks: key part, then value part
        lane = byte // (2 * cb)
        assert np.all((byte % (2 * cb)) < cb)
    else:                                             # INT4: the 64 key parts, then the 64 value parts
        lane = byte // cb
        assert np.all(byte < 64 * cb)
    for t in range(16):
        assert set(np.unique(lane[t] % 16)) == {t}    # lane 16g+t holds slot t only


@pytest.mark.parametrize("d", [64, 128])
def test_int4_value_parts_follow_the_key_parts(d):
    byte, _ = layout_ref.value_offsets(d, 4)
    cb = d * 4 // 32
    assert np.all(byte >= 64 * cb) and np.all(byte < 128 * cb)
    lane = byte // cb - 64
    nb_c = np.arange(d) % 16                          # value lane 16*(t/4) + ch%16
    for t in range(16):
        assert np.array_equal(lane[t], 16 * (t // 4) + nb_c)


@pytest.mark.parametrize("d,bits", [(64, 2), (128, 2), (64, 4), (128, 4)])
def test_pack_round_trip(d, bits):
    r = np.random.default_rng(3)
    ck = r.integers(0, 1 << bits, (16, d)).astype(np.uint8)
    cv = r.integers(0, 1 << bits, (16, d)).astype(np.uint8)
    sk = r.integers(0, 65535, (16, 2)).astype(np.uint16)
    sv = r.integers(0, 65535, (16, 2)).astype(np.uint16)
    raw = layout_ref.pack_page_head(d, bits, ck, cv, sk, sv)
    assert raw.size == 4 * d * bits + 128
    a, b, c, e = layout_ref.unpack_page_head(d, bits, raw)
    assert np.array_equal(a, ck) and np.array_equal(b, cv) and np.array_equal(c, sk) and np.array_equal(e, sv)


def test_bf16_indices_are_a_bijection():
    for d in (64, 128):
        idx = np.concatenate([layout_ref.bf16_key_index(d).ravel(), layout_ref.bf16_value_index(d).ravel()])
        assert np.array_equal(np.sort(idx), np.arange(32 * d))


def test_window_positions():
    for T in (0, 1, 63, 64, 100, 319, 320, 321, 1000, 1001):
        held = sorted(p for j in range(20) for t in range(16)
                      if (p := layout_ref.window_position(j, t, T, 64, 256)) >= 0)
        expect = list(range(min(T, 64))) + list(range(max(64, T - 256), T))
        assert held == expect, T
