"""The lane-major group-block layout: every (position, channel) owns its own
two bits, and the readers invert the writer's index maps."""
import numpy as np
import pytest

from decode_attention_kvq_amd import layout


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("which", ["key", "value"])
def test_layout_is_a_bijection(d, which):
    byte, shift = (layout._key_index if which == "key" else layout._value_index)(d)
    slots = byte * 4 + shift // 2
    assert byte.shape == (32, d)
    assert slots.min() == 0 and slots.max() == 32 * d - 1
    assert np.unique(slots).size == 32 * d


@pytest.mark.parametrize("d", [64, 128])
def test_key_layout_matches_header_formula(d):
    byte, shift = layout._key_index(d)
    W = d // 8
    for t, c in [(0, 0), (5, 37), (17, 99 % d), (31, d - 1)]:
        lane = ((c % 32) // 8) * 16 + t % 16
        assert byte[t, c] == lane * W + (t // 16) * (d // 16) + (c // 32) * 2 + (c % 8) // 4
        assert shift[t, c] == 2 * (c % 4)


@pytest.mark.parametrize("d", [64, 128])
def test_value_layout_groups_four_positions_per_byte(d):
    byte, shift = layout._value_index(d)
    for t in range(0, 32, 4):
        for c in range(d):
            assert len(set(byte[t:t + 4, c])) == 1
            assert list(shift[t:t + 4, c]) == [0, 2, 4, 6]


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 4, size=(3, 32, 128)).astype(np.uint8)
    blocks = layout.pack_key_codes(codes, 128)
    np.testing.assert_array_equal(layout.unpack_key_blocks(blocks, 128), codes)
