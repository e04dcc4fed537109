"""CPU checks of the parity diagnostics the GPU tests report (cosine
similarity, pass rate at 3e-3, max relative error) and of the comparison
that applies them."""

import numpy as np
import pytest

import gpu_util as U


def test_identical_arrays():
    x = np.random.default_rng(0).standard_normal((3, 5, 128))
    rel, cos, rate = U.diagnostics(x, x)
    assert rel == 0.0 and cos == pytest.approx(1.0, abs=1e-15) and rate == 1.0
    assert U.compare(x, x, 0.0, "identical") == 0.0


def test_pass_rate_and_relative_error():
    ref = np.ones(1000)
    got = ref.copy()
    got[:10] += 1e-2    # 1 % of the elements beyond 3e-3
    rel, cos, rate = U.diagnostics(got, ref)
    assert rate == pytest.approx(0.99)
    assert rel == pytest.approx(1e-2)
    assert cos > 0.999


def test_zero_rows_count_as_matching():
    z = np.zeros((4, 128))
    assert U.diagnostics(z, z)[1] == 1.0


def test_compare_rejects_a_sign_flip_within_the_bound():
    # a small output flipped in sign passes a loose absolute bound but not the cosine check
    ref = np.full(256, 1e-3)
    with pytest.raises(AssertionError, match="cosine"):
        U.compare(-ref, ref, 1e-2, "flipped")
