"""The rounding-aware error bound used by GPU tests, checked on the CPU
against numpy's own format spacing."""

import numpy as np

from tests.gpu_helpers import half_ulp, max_err_stored


def test_half_ulp_matches_numpy_spacing():
    x = np.array([1e-3, 0.3, 1.0, 1.5, 2.0, 3.99, 4.0, 7.5, 100.0, -5.0])
    assert np.array_equal(half_ulp(x, "f16"), np.spacing(np.abs(x).astype(np.float16)).astype(np.float64) / 2)
    assert np.array_equal(half_ulp(x, "f32"), np.spacing(np.abs(x).astype(np.float32)).astype(np.float64) / 2)
    # bf16 keeps the f32 exponent with 16 fewer mantissa bits
    assert np.array_equal(half_ulp(x, "bf16"),
                          np.spacing(np.abs(x).astype(np.float32)).astype(np.float64) * 2 ** 16 / 2)


def test_max_err_stored_forgives_exactly_one_rounding():
    ref = np.array([4.0 + 2 ** -6 - 1e-9])       # just below the bf16 midpoint of [4, 4 + 2^-5]
    got = np.array([4.0])
    assert max_err_stored(got, ref, "bf16") <= 0.0
    assert max_err_stored(np.array([4.0 - 2 ** -5]), ref, "bf16") > 0.03
