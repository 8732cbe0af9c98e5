"""The seeded input generators: shapes, storage precision and the stated distributions."""
import numpy as np

from synth import bf16_rne, gen_coupled_tokens


def test_bf16_rne_ties_to_even_and_exact_values():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    a = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0], dtype=np.float32)
    bits, vals = bf16_rne(a)
    assert vals.tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, -2.5, 0.0]
    assert bits[0] == 0x3F80 and bits[3] == 0xC020


def test_coupled_tokens_correlate_by_rho():
    for rho in (0.0, 0.5, 0.9):
        vals, bits = gen_coupled_tokens(np.random.default_rng(7), 64, 2048, rho)
        assert vals.shape == (64, 2048) and bits.dtype == np.uint16
        assert np.array_equal(bf16_rne(vals)[1], vals)   # already bf16 values
        assert abs(float(vals.std()) - 1.0) < 0.05
        c = np.corrcoef(vals.astype(np.float64))
        off = c[np.triu_indices(64, 1)]
        assert abs(float(off.mean()) - rho) < 0.03
