"""Pins for just-in-time scaling in the oracle (CPU only).

Just-in-time scaling ([TE-KR] "Scaling factor" strategy) takes the factor
from the amax of the tensor being cast.  Closed forms: the scale is
fl32(fp8_max / amax); the element of largest magnitude lands on the largest
code (it maps to fp8_max up to one rounding of the scale, and the cast
saturates); with a power-of-two amax the scale is exact and every element is
x * fp8_max / amax before rounding.  Behaviour pins: the first backward step of
the 768-wide linear no longer underflows (the delayed step 0 does, a pin of its
own), and a x100 spike saturates the delayed cast but not the just-in-time one.
"""
import numpy as np
import pytest

MAXCODE = {0: 0x7E, 1: 0x7B}


@pytest.mark.parametrize("fmt", [0, 1])
def test_jit_scale_closed_form_and_top_code(oracle, fmt):
    rng = np.random.default_rng(10 + fmt)
    x = (rng.standard_normal((64, 96)) * 3e-3).astype(np.float32)
    m = oracle.Meta(8, fmt)
    m.record(x)
    oracle.scale_from_current(m)
    a = np.abs(x).max()
    assert m.scale == np.float32(oracle.fp8_max(fmt) / np.float64(a))
    assert m.scale_inv == np.float32(1.0 / np.float64(m.scale))
    q = oracle.cast(x, fmt, m.scale)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[i] & 0x7F == MAXCODE[fmt]
    assert np.all(m.hist[1:] == 0) and m.hist[0] == a          # no roll


def test_jit_power_of_two_amax_is_exact_rescale(oracle):
    x = np.array([[0.25, -0.125, 0.0625, 1.0 / 3.0]], dtype=np.float32)   # amax 1/3 is not a power of two
    x[0, 3] = 0.5                                                          # now amax = 0.5
    m = oracle.Meta(4, 0)
    m.record(x)
    oracle.scale_from_current(m)
    assert m.scale == np.float32(896.0)
    want = oracle.encode_array(x.astype(np.float64) * 896.0, 0)
    assert np.array_equal(oracle.cast(x, 0, m.scale), want)


def test_jit_keeps_scale_for_zero_or_nonfinite_amax(oracle):
    for bad in (0.0, np.inf, np.nan):
        m = oracle.Meta(4, 1)
        m.scale, m.scale_inv = np.float32(8.0), np.float32(0.125)
        m.hist[0] = bad
        oracle.scale_from_current(m)
        assert m.scale == np.float32(8.0) and m.scale_inv == np.float32(0.125), bad


def test_jit_first_backward_step_does_not_underflow(oracle):
    import synth
    w, b = synth.linear768_weights()
    x, dy = synth.linear768_x(0).numpy(), synth.linear768_dy(0).numpy()
    for jit, expect_zero in ((False, True), (True, False)):
        mx, mw, mg = oracle.Meta(16, 0), oracle.Meta(16, 0), oracle.Meta(16, 1)
        fw = oracle.linear_fwd(x, w.numpy(), mx, mw, rows=np.arange(4), jit=jit)
        bw = oracle.linear_bwd(dy, fw, mg, rows_dx=np.arange(4), rows_dw=np.arange(4), jit=jit)
        assert (not np.any(bw["gq"] & 0x7F)) == expect_zero
        assert (not np.any(bw["dw"])) == expect_zero


def test_jit_spike_does_not_saturate_but_delayed_does(oracle):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((256, 64)).astype(np.float32)
    m = oracle.Meta(16, 0)
    m.record(x)
    oracle.update_metas([m])                          # delayed scale from the clean step
    spike = x * np.float32(100.0)
    delayed = oracle.cast(spike, 0, m.scale)
    jm = m.copy()
    jm.record(spike)
    oracle.scale_from_current(jm)
    jit = oracle.cast(spike, 0, jm.scale)
    sat = lambda q: int(np.count_nonzero((q & 0x7F) == 0x7E))
    assert sat(delayed) > 0.5 * x.size
    assert sat(jit) <= 2                              # only the amax element (and a tie) reach 448
