"""GPU parity: amax and the delayed-scaling update against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
from helpers import assert_bits_equal, dev, np_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [0, 1, 17, 1024, 999_999, 1 << 24])
def test_amax_matches_oracle(oracle, dtype, n):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * np.exp2(rng.uniform(-40, 40, n))).astype(np.float32)
    if dtype == "bf16":
        x = oracle.bf16_from_f32(x)
    slot = torch.zeros(1, dtype=torch.float32, device="cuda")
    F.fp8_amax(dev(x), slot)
    assert_bits_equal(np_of(slot)[0], oracle.amax(x), f"{dtype} n={n}")


def test_amax_special_values_and_merge(oracle):
    cases = [np.array([1.0, -np.inf, 3.0], np.float32), np.array([1.0, np.nan, -2.0] * 100, np.float32),
             np.array([-0.0] * 33, np.float32), np.array([1e-45, -3e-45] * 20, np.float32)]
    for x in cases:
        slot = torch.zeros(1, dtype=torch.float32, device="cuda")
        F.fp8_amax(dev(x), slot)
        assert_bits_equal(np_of(slot)[0], oracle.amax(x))
    # merging keeps the larger value already in the slot
    slot = torch.full((1,), 100.0, dtype=torch.float32, device="cuda")
    F.fp8_amax(dev(np.array([3.0, -7.0] * 50, np.float32)), slot)
    assert np_of(slot)[0] == 100.0
    F.fp8_amax(dev(np.array([3.0, -700.0] * 50, np.float32)), slot)
    assert np_of(slot)[0] == 700.0


@pytest.mark.parametrize("L", [1, 16, 255, 1024, 1500])
@pytest.mark.parametrize("margin", [0, 3])
def test_scale_update_matches_oracle(oracle, L, margin):
    rng = np.random.default_rng(L * 7 + margin)
    n = 13
    fmts = [F.E4M3 if i % 3 else F.E5M2 for i in range(n)]
    ofmts = [0 if f == F.E4M3 else 1 for f in fmts]
    hist = (rng.uniform(0, 1, (n, L)) * np.exp2(rng.integers(-30, 30, (n, L)))).astype(np.float32)
    hist[1] = 0.0                                   # nothing recorded yet: keep the scale
    hist[2, :] = np.inf                             # only non-finite entries: keep
    hist[3, 0] = np.nan                             # NaN is skipped
    hist[4, L // 2] = np.inf
    hist[5, :] = 1e-44                              # quotient overflows: FLT_MAX
    hist[6, 0] = 3.0e38
    scale = rng.uniform(0.5, 2, n).astype(np.float32)
    sinv = (1 / scale).astype(np.float32)
    dh, ds, di = dev(hist), dev(scale), dev(sinv)
    recipe = F.Recipe(F.FORMAT_HYBRID, L, F.AMAX_MAX, margin)
    for _ in range(3):                              # three consecutive steps (the history rolls)
        F.fp8_amax_scale_update(dh, ds, di, fmts, recipe)
        oracle.scale_update(hist, scale, sinv, ofmts, margin)
        assert_bits_equal(np_of(dh), hist, "history")
        assert_bits_equal(np_of(ds), scale, "scale")
        assert_bits_equal(np_of(di), sinv, "scale_inv")
        # a new step's amax lands in slot 0
        new = rng.uniform(0, 10, n).astype(np.float32)
        hist[:, 0] = new
        dh[:, 0] = dev(new)


def test_scale_from_current_amax_matches_oracle(oracle):
    """fp8_scale_from_current_amax over a bank of 40 tensors whose slot-0
    amaxes span normal, subnormal, huge, zero, Inf and NaN values (the last
    three keep the old scale), margins 0 and 3; histories are not rolled."""
    rng = np.random.default_rng(8)
    n, L = 40, 8
    fmts = [int(v) for v in rng.integers(0, 2, n)]
    hist = (np.abs(rng.standard_normal((n, L))) * np.exp2(rng.uniform(-30, 30, (n, L)))).astype(np.float32)
    hist[0, 0], hist[1, 0], hist[2, 0], hist[3, 0] = 0.0, np.inf, np.nan, 1e-44
    hist[4, 0], hist[5, 0] = 3.0e38, 2.0 ** -149
    for margin in (0, 3):
        bank = F.MetaBank([F.E4M3 if f == 0 else F.E5M2 for f in fmts], L)
        bank.amax_history.copy_(torch.from_numpy(hist))
        bank.scale.fill_(2.0)
        bank.scale_inv.fill_(0.5)
        bank.scale_from_current(F.Recipe(F.FORMAT_HYBRID, L, F.AMAX_MAX, margin))
        for t in range(n):
            m = oracle.Meta(L, fmts[t])
            m.hist = hist[t].copy()
            m.scale, m.scale_inv = np.float32(2.0), np.float32(0.5)
            oracle.scale_from_current(m, margin)
            assert_bits_equal(np_of(bank.scale[t]), m.scale, f"margin {margin} scale {t}")
            assert_bits_equal(np_of(bank.scale_inv[t]), m.scale_inv, f"margin {margin} scale_inv {t}")
        assert_bits_equal(np_of(bank.amax_history), hist, "history untouched")
