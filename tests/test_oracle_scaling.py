"""Pins for the oracle's amax, delayed-scaling update and history (CPU only).

The pins are closed forms of the scale rule, a brute-force sliding window over
the amax sequence, special values, and the data-parallel invariant.
"""
import math

import numpy as np
import pytest

FLT_MAX = np.float32(3.4028234663852886e38)


def _bf16(x):
    """bf16 bit patterns by truncating exact-in-bf16 values (test inputs only)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


# ------------------------------------------------------------------ amax ----

def test_amax_bruteforce_and_permutation(oracle):
    rng = np.random.default_rng(0)
    for n in (1, 7, 1000, 100003):
        x = (rng.standard_normal(n) * np.exp2(rng.uniform(-30, 30, n))).astype(np.float32)
        a = oracle.amax(x)
        assert a == np.max(np.abs(x.astype(np.float64)))
        assert oracle.amax(rng.permutation(x)) == a


def test_amax_special_values(oracle):
    assert oracle.amax(np.zeros(17, np.float32)) == 0.0
    assert not math.copysign(1.0, oracle.amax(np.array([-0.0], np.float32))) < 0   # -0 counts as +0
    assert oracle.amax(np.array([1.0, -np.inf, 3.0], np.float32)) == np.inf
    assert math.isnan(oracle.amax(np.array([1.0, np.nan, np.inf], np.float32)))
    assert oracle.amax(np.array([-5.0, 4.0], np.float32)) == 5.0
    assert oracle.amax(np.zeros(0, np.float32)) == 0.0
    d = np.array([1e-45, -3e-45], np.float32)                 # fp32 subnormals
    assert oracle.amax(d) == np.float32(3e-45)


def test_amax_bf16_widening(oracle):
    x = np.array([0.5, -2.0, 3.0, -1024.0], np.float32)
    assert oracle.amax(_bf16(x)) == 1024.0
    assert oracle.amax(_bf16(x[:3])) == 3.0


def test_amax_data_parallel_invariant(oracle):
    """The max over shards of per-shard amaxes equals the amax of the whole
    batch, so one MAX all-reduce gives every rank the same scale."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 96)) * 10).astype(np.float32)
    for shards in (2, 4, 8):
        parts = np.array_split(x, shards, axis=0)
        assert max(oracle.amax(p) for p in parts) == oracle.amax(x)


# ------------------------------------------------------------ scale rule ----

def _update(oracle, hist_rows, fmts, margin=0, scale=None, sinv=None):
    hist = np.array(hist_rows, dtype=np.float32)
    n = hist.shape[0]
    s = np.ones(n, np.float32) if scale is None else np.array(scale, np.float32)
    si = np.ones(n, np.float32) if sinv is None else np.array(sinv, np.float32)
    oracle.scale_update(hist, s, si, fmts, margin)
    return hist, s, si


@pytest.mark.parametrize("fmt,mx", [(0, 448.0), (1, 57344.0)])
def test_scale_closed_forms(oracle, fmt, mx):
    h, s, si = _update(oracle, [[mx, 0, 0, 0]], [fmt])
    assert s[0] == 1.0 and si[0] == 1.0
    for k in range(-40, 40, 3):
        h, s, si = _update(oracle, [[2.0 ** k, 0.5 * 2.0 ** k, 0, 0]], [fmt])
        assert s[0] == np.float32(mx * 2.0 ** -k)
        assert si[0] == np.float32(2.0 ** k / mx)
    for m in range(0, 9):
        base = _update(oracle, [[3.7, 1.0]], [fmt])[1][0]
        got = _update(oracle, [[3.7, 1.0]], [fmt], margin=m)[1][0]
        assert got == base * np.float32(2.0 ** -m)


def test_scale_is_fp32_division(oracle):
    rng = np.random.default_rng(9)
    amaxes = (rng.uniform(0.5, 2.0, 200) * np.exp2(rng.integers(-60, 60, 200))).astype(np.float32)
    for a in amaxes:
        _, s, si = _update(oracle, [[a, 0, 0]], [0])
        # fp32 IEEE division of fp32 operands == the fp64 quotient rounded once to fp32
        assert s[0] == np.float32(np.float64(448.0) / np.float64(a))
        assert si[0] == np.float32(np.float64(1.0) / np.float64(s[0]))


def test_scale_degenerate_cases(oracle):
    # all-zero history: scale kept
    _, s, si = _update(oracle, [[0, 0, 0]], [0], scale=[5.0], sinv=[0.2])
    assert s[0] == np.float32(5.0) and si[0] == np.float32(0.2)
    # only non-finite entries: kept
    _, s, si = _update(oracle, [[np.inf, np.nan, 0]], [0], scale=[5.0], sinv=[0.2])
    assert s[0] == np.float32(5.0) and si[0] == np.float32(0.2)
    # non-finite entries are skipped, the finite max is used
    _, s, _ = _update(oracle, [[np.inf, 2.0, np.nan, 7.0]], [0])
    assert s[0] == np.float32(448.0 / 7.0)
    # a quotient beyond fp32 becomes FLT_MAX
    _, s, si = _update(oracle, [[1e-44, 0]], [0])
    assert s[0] == FLT_MAX and si[0] == np.float32(1.0 / np.float64(FLT_MAX))


def test_history_roll(oracle):
    rows = [[1, 2, 3, 4], [9, 8, 7, 6]]
    h, _, _ = _update(oracle, rows, [0, 1])
    assert h.tolist() == [[0, 1, 2, 3], [0, 9, 8, 7]]


@pytest.mark.parametrize("L", [1, 4, 16])
def test_scale_follows_sliding_window(oracle, L):
    """Driving the update with a known amax sequence, the scale after step t is
    fp8_max / max(amax[t-L+1 .. t]) -- a window of exactly the last L amaxes."""
    rng = np.random.default_rng(L)
    T = 60
    seq = (rng.uniform(0.1, 1.0, T) * np.exp2(rng.integers(-8, 8, T))).astype(np.float32)
    hist = np.zeros((1, L), np.float32)
    s = np.ones(1, np.float32)
    si = np.ones(1, np.float32)
    for t in range(T):
        hist[0, 0] = seq[t]                      # the step's amax lands in slot 0
        oracle.scale_update(hist, s, si, [1], 0)
        window = seq[max(0, t - L + 1): t + 1]
        assert s[0] == np.float32(57344.0 / np.float64(window.max()))


def test_spike_recovery_reading(oracle):
    """A x100 amax spike at step 10 with history 1024: the scale drops by ~100 at
    the next update and stays down for the rest of a 20-step run."""
    L = 1024
    hist = np.zeros((1, L), np.float32)
    s = np.ones(1, np.float32)
    si = np.ones(1, np.float32)
    scales = []
    for t in range(20):
        hist[0, 0] = np.float32(3.0 * (100 if t == 10 else 1))
        oracle.scale_update(hist, s, si, [0], 0)
        scales.append(float(s[0]))
    assert all(x == scales[0] for x in scales[:10])
    assert all(abs(x * 100 / scales[0] - 1) < 1e-6 for x in scales[10:])


# --------------------------------------------------------- cast and dequant ----

def test_cast_constant_tensor_at_steady_state(oracle):
    """A constant tensor c scaled by fp8_max/c lands on the largest code."""
    for fmt, maxc, mx in ((0, 0x7E, 448.0), (1, 0x7B, 57344.0)):
        for c in (1e-7, 3.3e-3, 0.1, 1.7, 1234.5):
            x = np.full(33, c, np.float32)
            s = np.float32(np.float32(mx) / np.float32(c))
            assert np.all(oracle.cast(x, fmt, s) == maxc)
            assert np.all(oracle.cast(-x, fmt, s) == maxc | 0x80)


def test_cast_identity_on_representable_inputs(oracle):
    for fmt in (0, 1):
        vals = np.array([oracle.decode(c, fmt) for c in range(256)])
        ok = np.isfinite(vals)
        codes = np.arange(256, dtype=np.uint8)[ok]
        x = vals[ok].astype(np.float32)
        assert np.array_equal(oracle.cast(x, fmt, 1.0), codes)
        back = oracle.dequant(codes, fmt, 1.0)
        assert np.array_equal(back, x)


def test_cast_is_two_roundings(oracle):
    """x*s is rounded to fp32 first; then the FP8 rounding applies to that product."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal(4096).astype(np.float32)
    s = np.float32(3.3)
    prod = (x * s).astype(np.float32)                   # numpy fp32 multiply (IEEE RNE)
    for fmt in (0, 1):
        assert np.array_equal(oracle.cast(x, fmt, s), oracle.encode_array(prod, fmt))


def test_cast_transpose_and_dequant(oracle):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((48, 80)).astype(np.float32)
    q, qt = oracle.cast_transpose(x, 0, 2.0)
    assert np.array_equal(qt, q.T)
    d = oracle.dequant(q, 0, 0.5)
    err = np.abs(d - x) / np.maximum(np.abs(x), 2.0 ** -6)
    assert err.max() <= 2.0 ** -4 + 1e-7                      # half an E4M3 ulp, relative
    db = oracle.dequant(q, 0, 0.5, out_dtype=1)
    assert np.array_equal(db, oracle.bf16_from_f32(d))


def test_colsum(oracle):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1000, 37)).astype(np.float32)
    assert np.allclose(oracle.colsum(x), x.astype(np.float64).sum(axis=0), rtol=1e-13, atol=1e-12)
