"""GPU: the SGD step fused with the next forward's weight cast
(fp8_sgd_step_cast) and the forward that takes W pre-cast (fp8_linear_fwd with
w = None).

The fused call must equal fp8_sgd_step followed by fp8_cast_transpose of the
updated masters bit for bit: masters, codes both ways, amax slot and, with a
counter registered, the saturated-code count; on a found_inf step the masters
stay and are still cast.  The updated masters are also checked against the
oracle's SGD and cast.  A forward with W pre-cast equals the forward that casts
W itself, output and saved state alike."""
import numpy as np
import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
import synth
from helpers import assert_bits_equal, np_of

pytestmark = pytest.mark.gpu


def _state(s, found_inf=0.0):
    return torch.tensor([s, 0.0, found_inf, s], dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("shape", [(272, 400), (1024, 768), (16, 16)], ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("found_inf", [0.0, 1.0], ids=["step", "skipped"])
def test_sgd_step_cast_equals_sgd_then_cast(oracle, shape, found_inf):
    rows, cols = shape
    seed = synth.seed_of(6, 0, rows % 97 + int(found_inf))
    w0 = synth.normal((rows, cols), 0.05, seed, device="cuda")
    g = synth.normal((rows, cols), 2.0 ** 10, seed + 1, device="cuda")     # gradients carry the loss scale
    lr, S = 2.0 ** -10, 2.0 ** 16
    state = _state(S, found_inf)
    scale = torch.tensor([448.0 / 0.12], dtype=torch.float32, device="cuda")   # saturates the tails
    u8 = dict(dtype=torch.uint8, device="cuda")
    # reference: the two separate calls
    w_ref = w0.clone()
    F.fp8_sgd_step(w_ref, g, lr, state)
    q_ref, qt_ref = torch.empty(rows, cols, **u8), torch.empty(cols, rows, **u8)
    slot_ref = torch.zeros(1, device="cuda")
    F.fp8_cast_transpose(w_ref, F.E4M3, scale, q_ref, qt_ref, slot_ref)
    # fused, with a saturation counter on its slot
    w = w0.clone()
    q, qt = torch.empty(rows, cols, **u8), torch.empty(cols, rows, **u8)
    slot = torch.zeros(1, device="cuda")
    ctr = torch.zeros(1, dtype=torch.int32, device="cuda")
    F.count_saturation(slot, ctr)
    try:
        F.fp8_sgd_step_cast(w, g, lr, state, scale, q, qt, slot)
        torch.cuda.synchronize()
    finally:
        F.count_saturation(slot, None)
    assert_bits_equal(np_of(w), np_of(w_ref), "masters")
    assert_bits_equal(np_of(q), np_of(q_ref), "codes")
    assert_bits_equal(np_of(qt), np_of(qt_ref), "transposed codes")
    assert_bits_equal(np_of(slot), np_of(slot_ref), "amax slot")
    # against the oracle: its SGD on the host copies, then its cast
    W, G = np_of(w0).ravel().copy(), np_of(g).ravel()
    ls = oracle.LossScale(S)
    ls.state[2] = np.float32(found_inf)
    oracle.sgd(W, G, lr, ls)
    W = W.reshape(rows, cols)
    assert_bits_equal(np_of(w), W, "masters vs oracle")
    wq, wqt = oracle.cast_transpose(W, 0, np.float32(np_of(scale)[0]))
    assert_bits_equal(np_of(q), wq, "codes vs oracle")
    assert_bits_equal(np_of(qt), wqt, "transposed codes vs oracle")
    assert int(ctr.item()) == oracle.count_saturated(W, 0, np_of(scale)[0])
    if found_inf:
        assert_bits_equal(np_of(w), np_of(w0), "skipped step leaves the masters")


def test_forward_with_precast_weights(oracle):
    """fp8_linear_fwd(x, None, ...) after fp8_sgd_step_cast equals the forward
    that casts the same updated W itself: Y, the saved codes, the inverse
    scales it snapshots and the amax histories (W's recorded once by the fused
    step, X's by the forward)."""
    m, n, k = 272, 400, 208
    x = synth.normal((m, k), 1.0, synth.seed_of(6, 1, 0), torch.bfloat16, "cuda")
    w0 = synth.normal((n, k), 0.05, synth.seed_of(6, 1, 1), device="cuda")
    g = synth.normal((n, k), 2.0 ** 10, synth.seed_of(6, 1, 2), device="cuda")
    lr, state = 2.0 ** -10, _state(2.0 ** 16)
    recipe = F.Recipe(F.FORMAT_HYBRID, 16, F.AMAX_MAX, 0)
    outs = {}
    for mode in ("cast", "precast"):
        bank = F.MetaBank([F.E4M3, F.E4M3], 16)
        bank.scale.copy_(torch.tensor([448.0 / 4.0, 448.0 / 0.2], device="cuda"))
        bank.scale_inv.copy_(1.0 / bank.scale)
        saved = F.Saved(m, n, k)
        w = w0.clone()
        y = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
        if mode == "cast":
            F.fp8_sgd_step(w, g, lr, state)
            F.fp8_linear_fwd(x, w, y, recipe, bank.meta(0), bank.meta(1), saved)
        else:
            F.fp8_sgd_step_cast(w, g, lr, state, bank.scale[1:2], saved.wq, saved.wq_t, bank.amax_history[1, 0:1])
            F.fp8_linear_fwd(x, None, y, recipe, bank.meta(0), bank.meta(1), saved)
        torch.cuda.synchronize()
        outs[mode] = (y, saved, bank, w)
    (y0, s0, b0, w_0), (y1, s1, b1, w_1) = outs["cast"], outs["precast"]
    assert_bits_equal(np_of(w_1), np_of(w_0), "masters")
    assert_bits_equal(np_of(y1), np_of(y0), "Y")
    for attr in ("xq", "xq_t", "wq", "wq_t", "sinv"):
        assert_bits_equal(np_of(getattr(s1, attr)), np_of(getattr(s0, attr)), attr)
    assert_bits_equal(np_of(b1.amax_history), np_of(b0.amax_history), "histories")
    # the forward's inputs against the oracle: X's and W's codes
    wq = oracle.cast_transpose(np_of(w_0), 0, np.float32(448.0 / 0.2))[0]
    assert_bits_equal(np_of(s1.wq), wq, "W codes vs oracle")
