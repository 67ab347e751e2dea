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
    assert max_err_stored(got, ref, "bf16", 1e-2) <= 0.0
    assert max_err_stored(np.array([4.0 - 2 ** -5]), ref, "bf16", 1e-2) > 0.03


def test_max_err_stored_allowance_only_where_rounding_exceeds_half_the_bound():
    """bf16, bound 1e-2: half an ulp is 2^-8 (< 5e-3) on [1, 2) and 2^-7 (> 5e-3)
    on [2, 4); f16, bound 2e-3: 2^-10 on [2, 4) (< 1e-3), 2^-9 on [4, 8)."""
    # on [1, 2) the plain error counts: 9e-3 passes 1e-2, 1.1e-2 fails
    assert abs(max_err_stored(np.array([1.5]), np.array([1.5 + 9e-3]), "bf16", 1e-2) - 9e-3) < 1e-15
    assert max_err_stored(np.array([1.5]), np.array([1.5 + 1.1e-2]), "bf16", 1e-2) > 1e-2
    # on [2, 4) the half ulp 2^-7 is forgiven
    e = max_err_stored(np.array([3.0]), np.array([3.0 + 1.2e-2]), "bf16", 1e-2)
    assert abs(e - (1.2e-2 - 2 ** -7)) < 1e-15
    # f16 bound 2e-3: no allowance at 3.0 (half ulp 2^-10 < 1e-3), allowance at 5.0
    assert abs(max_err_stored(np.array([3.0]), np.array([3.0 + 1.5e-3]), "f16", 2e-3) - 1.5e-3) < 1e-15
    e = max_err_stored(np.array([5.0]), np.array([5.0 + 2.5e-3]), "f16", 2e-3)
    assert abs(e - (2.5e-3 - 2 ** -9)) < 1e-15
    # the same elements under the fp8-KV bound 3e-2 with bf16 outputs: only
    # |x| >= 4 (half ulp 2^-6 > 1.5e-2) gets the allowance
    assert abs(max_err_stored(np.array([3.0]), np.array([3.02]), "bf16", 3e-2) - 0.02) < 1e-12
    e = max_err_stored(np.array([6.0]), np.array([6.04]), "bf16", 3e-2)
    assert abs(e - (0.04 - 2 ** -6)) < 1e-12
