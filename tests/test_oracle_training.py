"""Pins for the oracle's loss scaling and fp32 master-weight SGD (CPU only).

The dynamic loss-scale procedure of the mixed-precision page is a small state
machine; its pins are the sequences it must produce.  SGD is pinned by exact
dyadic cases (every rounding exact, so the fp32 result equals the rational
one), the skip on an overflowed step, and exact power-of-two loss scaling.
"""
import math
from fractions import Fraction

import numpy as np
import pytest


def test_loss_scale_grows_after_interval_clean_steps(oracle):
    ls = oracle.LossScale(65536.0, interval=5)
    seq = []
    for _ in range(12):
        ls.update([1.0, 0.5, 3.0])
        seq.append(float(ls.state[0]))
        assert not ls.found_inf
    assert seq == [65536.0] * 4 + [131072.0] * 5 + [262144.0] * 3


@pytest.mark.parametrize("bad", [math.inf, -math.inf, math.nan])
def test_loss_scale_backs_off_and_flags_overflow(oracle, bad):
    ls = oracle.LossScale(1024.0, interval=3)
    ls.update([1.0])
    ls.update([1.0])
    assert ls.state[1] == 2.0
    ls.update([2.0, bad, 1.0])
    assert ls.found_inf and ls.state[0] == 512.0 and ls.state[1] == 0.0
    assert ls.state[3] == 1024.0                      # the overflowed step carried the old S
    ls.update([1.0])
    assert not ls.found_inf and ls.state[3] == 512.0


def test_sgd_exact_dyadic_cases(oracle):
    rng = np.random.default_rng(3)
    n = 4096
    # few-bit dyadic values: every product and difference below is exact in fp32
    w = (rng.integers(-64, 64, n) * 2.0 ** rng.integers(-6, 2, n)).astype(np.float32)
    g = (rng.integers(-64, 64, n) * 2.0 ** rng.integers(10, 14, n)).astype(np.float32)
    ls = oracle.LossScale(2.0 ** 16)
    ls.update([1.0])
    lr = 2.0 ** -10
    w0 = w.copy()
    oracle.sgd(w, g, lr, ls)
    for i in range(0, n, 97):
        want = Fraction(float(w0[i])) - Fraction(lr) * Fraction(float(g[i])) / Fraction(2 ** 16)
        assert Fraction(float(w[i])) == want


def test_sgd_skipped_after_overflow(oracle):
    w = np.arange(16, dtype=np.float32)
    g = np.ones(16, dtype=np.float32)
    ls = oracle.LossScale()
    ls.update([np.inf])
    oracle.sgd(w, g, 0.1, ls)
    assert np.array_equal(w, np.arange(16, dtype=np.float32))


def test_sgd_unscales_by_the_scale_the_gradients_carry(oracle):
    """A gradient g produced under scale S moves the weight by lr * g / S even
    when the update of the same step changes S (growth after the interval)."""
    ls = oracle.LossScale(8.0, interval=1)
    ls.update([1.0])                                  # S grows to 16 now, the step carried 8
    w = np.array([1.0], np.float32)
    oracle.sgd(w, np.array([8.0], np.float32), 0.5, ls)
    assert w[0] == 0.5


def test_scale_by_power_of_two_is_exact(oracle):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.scale_by(x, 2.0 ** 16), x * np.float32(2.0 ** 16))
    xb = oracle.bf16_from_f32(x)
    got = oracle.bf16_to_f64(oracle.scale_by(xb, 2.0 ** -3))
    assert np.array_equal(got, oracle.bf16_to_f64(xb) * 2.0 ** -3)
