"""The lane-major group-block layout: every (position, channel) owns its own
b bits (b = 2, 3, 4), and the readers invert the writer's index maps."""
import numpy as np
import pytest

from decode_attention_kvq_amd import layout


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("which", ["key", "value"])
def test_layout_is_a_bijection(d, which, bits):
    pos = (layout._key_bits if which == "key" else layout._value_bits)(d, bits)
    assert pos.shape == (32, d)
    assert np.all(pos % bits == 0)
    slots = pos // bits
    assert slots.min() == 0 and slots.max() == 32 * d - 1
    assert np.unique(slots).size == 32 * d


@pytest.mark.parametrize("d", [64, 128])
def test_two_bit_key_layout_matches_header_formula(d):
    pos = layout._key_bits(d, 2)
    W = d // 8
    for t, c in [(0, 0), (5, 37), (17, 99 % d), (31, d - 1)]:
        lane = ((c % 32) // 8) * 16 + t % 16
        assert pos[t, c] // 8 == lane * W + (t // 16) * (d // 16) + (c // 32) * 2 + (c % 8) // 4
        assert pos[t, c] % 8 == 2 * (c % 4)


@pytest.mark.parametrize("d", [64, 128])
def test_two_bit_value_layout_groups_four_positions_per_byte(d):
    pos = layout._value_bits(d, 2)
    for t in range(0, 32, 4):
        for c in range(d):
            assert len(set(pos[t:t + 4, c] // 8)) == 1
            assert list(pos[t:t + 4, c] % 8) == [0, 2, 4, 6]


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_lanes_own_operand_units_of_eight_codes(d, bits):
    """Lane L's stream holds, unit after unit, the 8 codes one matrix-core
    operand needs: 8 consecutive channels of one position (keys) or 8
    positions of one channel (values)."""
    per_lane = bits * d // 16 * 8
    kp, vp = layout._key_bits(d, bits), layout._value_bits(d, bits)
    for t in range(32):
        for c in range(0, d, 8):
            lanes = kp[t, c:c + 8] // per_lane
            assert len(set(lanes)) == 1
            offs = kp[t, c:c + 8] % per_lane
            assert list(offs - offs[0]) == [bits * k for k in range(8)] and offs[0] % (8 * bits) == 0
    for c in range(d):
        for q in range(4):
            ts = [4 * q + r for r in range(4)] + [16 + 4 * q + r for r in range(4)]
            offs = vp[ts, c] % per_lane
            assert len(set(vp[ts, c] // per_lane)) == 1
            assert list(offs - offs[0]) == [bits * k for k in range(8)] and offs[0] % (8 * bits) == 0


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_unpack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(3, 32, 128)).astype(np.uint8)
    kb = layout.pack_key_codes(codes, 128, bits)
    vb = layout.pack_value_codes(codes, 128, bits)
    assert kb.shape == (3, 4 * bits * 128)
    np.testing.assert_array_equal(layout.unpack_key_blocks(kb, 128, bits), codes)
    np.testing.assert_array_equal(layout.unpack_value_blocks(vb, 128, bits), codes)
