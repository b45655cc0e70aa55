"""The input generators: deterministic, and their bf16 rounding agrees with
the oracle's exact rounding."""
import numpy as np

import synth
from oracle import formats as F


def test_bf16_rounding_matches_oracle():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000) * 30, rng.standard_t(3, 100_000),
                        [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0, -0.0]])
    np.testing.assert_array_equal(synth.bf16_bits(x), F.f64_to_bf16_rne(x))


def test_seeded_and_shaped():
    a = synth.activations(1, 8, 32, outliers=2, outlier_mult=20.0)
    b = synth.activations(1, 8, 32, outliers=2, outlier_mult=20.0)
    assert a.dtype == np.uint16 and a.shape == (8, 32)
    np.testing.assert_array_equal(a, b)
    w = synth.weight(1, 0, 16, 32)
    assert abs(F.bf16_to_f64(w).std() - 0.02) < 0.005
