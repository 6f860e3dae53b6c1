"""The seeded input generators: bf16 rounding and the Philox uniforms.

Philox4x64-10 is written out here from its published definition (Salmon et
al., SC'11: two 64x64->128 multiplies per round with multipliers
0xD2E7470EE14C6C93 / 0xCA5A826395121157, Weyl key increments
0x9E3779B97F4A7C15 / 0xBB67AE8584CAA73B, ten rounds) and compared with the
generator, which takes its blocks from numpy.random.Philox.
"""

import numpy as np

import dsa_inputs as I

M64 = (1 << 64) - 1


def philox4x64_10(ctr, key):
    x = [int(c) & M64 for c in ctr]
    k0, k1 = int(key[0]) & M64, int(key[1]) & M64
    for r in range(10):
        if r:
            k0 = (k0 + 0x9E3779B97F4A7C15) & M64
            k1 = (k1 + 0xBB67AE8584CAA73B) & M64
        p0 = 0xD2E7470EE14C6C93 * x[0]
        p1 = 0xCA5A826395121157 * x[2]
        hi0, lo0 = p0 >> 64, p0 & M64
        hi1, lo1 = p1 >> 64, p1 & M64
        x = [hi1 ^ x[1] ^ k0, lo1, hi0 ^ x[3] ^ k1, lo0]
    return x


def test_philox_matches_published_definition():
    rng = np.random.default_rng(0)
    cases = [((0, 0, 0, 0), 0), ((M64, M64, M64, M64), M64), ((0, 3, 7, 1), 12345)]
    for _ in range(20):
        cases.append((tuple(int(v) for v in rng.integers(0, 2**63, 4)), int(rng.integers(0, 2**63))))
    for ctr, seed in cases:
        got = [int(v) for v in I.philox_block(seed, ctr)]
        assert got == philox4x64_10(ctr, (seed, 0))


def test_uniform_layout():
    seed, off = 77, 5
    ua, us = I.verify_uniforms(seed, off, 3, 2)
    for b in range(3):
        for j in range(3):
            x = philox4x64_10((off, b, j, 1), (seed, 0))[0]
            assert us[b, j] == np.float32((x >> 40) / 2**24)
            if j < 2:
                x = philox4x64_10((off, b, j, 0), (seed, 0))[0]
                assert ua[b, j] == np.float32((x >> 40) / 2**24)
    assert np.all((ua >= 0) & (ua < 1)) and np.all((us >= 0) & (us < 1))


def test_bf16_rounding():
    vals = np.array([1.0, -2.5, 1.0 + 2**-8, 1.0 + 3 * 2**-9, 3.0e38, 1e-40, 0.0, -0.0], np.float32)
    bits = I.bf16_bits(vals)
    back = I.bf16_value(bits)
    assert back[0] == 1.0 and back[1] == -2.5
    assert back[2] == 1.0                    # tie rounds to even (down)
    assert back[3] == 1.0 + 2**-7            # above the tie rounds up
    assert np.signbit(back[7]) and back[7] == 0
    # integers in [-4, 4] are exact in bf16
    ints = np.arange(-4, 5, dtype=np.float32)
    assert np.all(I.bf16_value(I.bf16_bits(ints)) == ints)
    assert I.bf16_bits(np.array([np.nan], np.float32))[0] == I.BF16_NAN


def test_draft_inputs_layout_roundtrip():
    d = I.draft_inputs(3, [100, 70], H_I=2, D_I=8, H_q=4, H_kv=2, D_qk=16, D_v=8,
                       k=16, G=3, page=16, shuffle_pages=True, poison=True)
    assert d.block_table.shape == (2, 7)
    used = d.block_table[d.block_table >= 0]
    assert len(set(used.tolist())) == used.size          # pages are distinct
    for b, L in enumerate(d.lens):
        for t in (0, 17, int(L) - 1):
            pg, row = d.block_table[b, t // 16], t % 16
            np.testing.assert_array_equal(I.bf16_value(d.kidx_bits[pg, row]), d.keys[b][t])
            np.testing.assert_array_equal(I.bf16_value(d.k_bits[pg, row]), d.K[b][t])
            np.testing.assert_array_equal(I.bf16_value(d.v_bits[pg, row]), d.V[b][t])
        # draft-written slots are poisoned
        t = int(L)
        pg, row = d.block_table[b, t // 16], t % 16
        assert np.all(np.isnan(I.bf16_value(d.k_bits[pg, row])))


def test_gumbel_draw_distribution():
    from scipy import stats
    rng = np.random.default_rng(9)
    logits = np.array([0.0, 1.0, -1.0, 2.0])
    counts = np.zeros(4)
    for _ in range(20000):
        counts[I.gumbel_draw(rng, logits)] += 1
    p = np.exp(logits) / np.exp(logits).sum()
    assert stats.chisquare(counts, p * counts.sum()).pvalue > 1e-3
