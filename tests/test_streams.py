"""The seeded omni-stream generator: determinism and the configured shapes."""
import numpy as np

from omnistream import (CONFIGS, MOD_AUDIO, MOD_TEXT, MOD_VIDEO, bf16_bits_to_f64,
                        f64_to_bf16_bits, generate, workload_digest)


def test_generator_is_deterministic():
    a, b = generate(1, length=3000), generate(1, length=3000)
    assert workload_digest(a) == workload_digest(b)
    assert workload_digest(a) != workload_digest(generate(2, length=3000))


def test_block84_interleave_and_fp32():
    w = generate(0)
    m = w.modality[0]
    assert m.size == 2048 and w.k[0].dtype == np.float32 and w.k[0].shape == (2048, 1, 64)
    np.testing.assert_array_equal(m[:84], [MOD_VIDEO] * 64 + [MOD_AUDIO] * 16 + [MOD_TEXT] * 4)
    assert w.q.shape == (1, 2, 64) and w.q.dtype == np.float32


def test_chunk_recipes():
    w = generate(1)
    m = w.modality[0]
    assert m.size == 16384 and w.k[0].dtype == np.uint16
    np.testing.assert_array_equal(m[:665], [MOD_VIDEO] * 640 + [MOD_AUDIO] * 25)
    w2 = generate(2, length=20000)
    runs = np.flatnonzero(np.diff(w2.modality[0].astype(int)) != 0) + 1
    first_video = runs[0]
    assert 640 <= first_video <= 2304


def test_stream_loop_append_chunk():
    w = generate(4, length=2048)
    m = w.modality[0]
    assert m.size == 2048 + 1024
    tail = m[2048:]
    assert (tail == MOD_VIDEO).sum() == 640 and (tail == MOD_AUDIO).sum() == 25
    assert (tail == MOD_TEXT).sum() == 359


def test_paged_sessions_table_is_a_permutation():
    w = generate(3, batch=6, len_range=(300, 1200))
    used = w.page_table[w.page_table >= 0]
    assert sorted(used.tolist()) == list(range(w.num_pages))
    for b in range(6):
        assert (w.page_table[b] >= 0).sum() == -(-int(w.lengths[b]) // 256)
        assert 300 <= w.lengths[b] <= 1200


def test_bf16_roundtrip():
    x = np.array([1.0, -2.5, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 3.14159])
    r = bf16_bits_to_f64(f64_to_bf16_bits(x))
    np.testing.assert_array_equal(r[:2], x[:2])
    assert r[2] == 1.0                      # tie to even
    assert r[3] == 1.0 + 2 ** -7            # rounds up
    assert abs(r[4] - 3.14159) < 2 ** -7 * 2


def test_config_table_matches_descriptions():
    c = CONFIGS
    assert (c[2].head_dim, c[2].n_q_heads, c[2].n_kv_heads, c[2].length) == (128, 28, 4, 81920)
    assert (c[3].batch, c[3].n_q_heads, c[3].n_kv_heads, c[3].len_range) == (32, 16, 2, (8192, 65536))
    assert (c[4].n_q_heads, c[4].n_kv_heads, c[4].length, c[4].append_tokens) == (32, 8, 131072, 1024)
