"""Host-side checks of the seeded input generator (no attention arithmetic here)."""
import numpy as np

import workloads as G


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, 1.0 + 2**-9, -2.5, np.inf, np.nan,
                  3.4028235e38], dtype=np.float32)
    b = G.bf16_bits(x)
    back = G.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                     # exact tie -> even (mantissa ...0)
    assert back[3] == 1.0                     # below the tie -> down
    assert back[2] == 1.0 + 2**-7             # above the tie -> up
    assert back[4] == -2.5 and np.isinf(back[5]) and np.isnan(back[6])
    assert np.isinf(back[7])                  # overflow rounds to inf


def test_decode_case_deterministic_and_poisoned():
    a = G.decode_case(3, 4, 8, 2, [5, 0, 3], G.BF16, seed=7)
    b = G.decode_case(3, 4, 8, 2, [5, 0, 3], G.BF16, seed=7)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.cache, b.cache)
    f = G.to_f64(a.cache, G.BF16)
    assert np.all(np.isfinite(f[0, :5])) and np.all(np.isnan(f[2, 3:])) and np.all(np.isnan(f[1]))


def test_single_sequence_regenerates_alone():
    a = G.decode_case(4, 2, 8, 2, [6, 6, 6, 6], G.F32, seed=3)
    b = G.decode_case(2, 2, 8, 2, [6, 6], G.F32, seed=3)
    assert np.array_equal(a.cache[:2], b.cache) and np.array_equal(a.q[:2], b.q)


def test_paged_layout_matches_dense():
    lens = [1, 64, 65, 130, 0]
    d = G.decode_case(5, 2, 16, 4, lens, G.BF16, seed=11)
    p = G.decode_case(5, 2, 16, 4, lens, G.BF16, seed=11, page_size=64)
    assert np.array_equal(d.q, p.q)
    assert p.pages.shape[0] == sum((l + 63) // 64 for l in lens)
    used = p.block_table[p.block_table >= 0]
    assert sorted(used.tolist()) == list(range(p.pages.shape[0]))   # a permutation of the pool
    for b, l in enumerate(lens):
        assert np.array_equal(G.seq_rows(p, b), d.cache[b, :l])
    # unused slots of each last page are NaN
    last = p.pages[p.block_table[2, 1]]
    assert np.all(np.isnan(G.bf16_bits_to_f32(last[1:])))


def test_config4_lengths_range():
    lens = G.config4_lengths(0)
    assert lens.shape == (128,) and lens.min() >= 1 and lens.max() <= 32768


def test_rms_and_rope_properties():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 512))
    c = G.rms_normalise(z)
    np.testing.assert_allclose(np.sqrt(np.mean(c * c, axis=1)), 1.0, rtol=1e-5)
    x = rng.standard_normal((7, 64))
    r = G.rope_interleaved(x, np.arange(7))
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    np.testing.assert_array_equal(r[0], x[0])  # position 0 is the identity


def test_paged_layout_matches_decode_case():
    lens = [64, 1, 130, 0, 200, 65]
    c = G.decode_case(6, 2, 8, 2, lens, G.BF16, seed=31, page_size=64)
    table, P = G.paged_layout(lens, 64, seed=31)
    assert np.array_equal(table, c.block_table) and P == c.pages.shape[0]
