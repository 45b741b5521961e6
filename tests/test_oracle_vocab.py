"""Pins for the oracle's temperature softmax / argmax."""
import numpy as np
import pytest
import scipy.special

import oracle


@pytest.mark.parametrize("T", [0.3, 1.0, 2.5])
def test_softmax_matches_scipy_and_sums_to_one(T):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(1000) * 3).astype(np.float32)
    p = oracle.target_distribution(x, T)
    ref = scipy.special.softmax(x.astype(np.float64) / T)
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=0)
    assert abs(p.sum() - 1) < 1e-12


def test_softmax_log_ratio_closed_form():
    x = np.array([0.5, -1.25, 3.0, 2.0], dtype=np.float32)
    T = 0.7
    p = oracle.target_distribution(x, T)
    for a in range(4):
        for b in range(4):
            assert np.isclose(np.log(p[a] / p[b]), (float(x[a]) - float(x[b])) / T, rtol=0, atol=1e-12)


def test_two_token_softmax_is_sigmoid():
    for d in [-3.0, 0.0, 0.4, 5.0]:
        p = oracle.target_distribution(np.array([d, 0.0]), 1.3)
        assert np.isclose(p[0], 1 / (1 + np.exp(-d / 1.3)), rtol=1e-13)


def test_temperature_zero_is_onehot_argmax_lowest_tie():
    x = np.array([1.0, 4.0, 4.0, -2.0], dtype=np.float32)
    p = oracle.target_distribution(x, 0.0)
    assert list(p) == [0.0, 1.0, 0.0, 0.0]
    assert oracle.argmax_lowest(x) == 1
    rng = np.random.default_rng(3)
    y = rng.standard_normal(5000).astype(np.float32)
    assert oracle.argmax_lowest(y) == int(np.argmax(y))  # numpy's argmax also keeps the first


def test_low_temperature_approaches_argmax():
    x = np.array([0.1, 0.9, 0.5], dtype=np.float32)
    p = oracle.target_distribution(x, 1e-3)
    assert p[1] > 1 - 1e-15 and p[0] < 1e-100


def test_rejects_bad_inputs():
    with pytest.raises(ValueError):
        oracle.target_distribution(np.array([np.nan, 0.0]), 1.0)
    with pytest.raises(ValueError):
        oracle.target_distribution(np.array([0.0, 0.0]), -1.0)
