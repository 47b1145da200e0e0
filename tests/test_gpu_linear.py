"""GPU parity of the layer calls, step by step against the oracle.

linear768 forward (4 steps on the same inputs, history 16, E4M3) and
forward + backward in HYBRID (16 iterations with fresh X and dY each step).
Every step compares: the FP8 codes of X, W, dY (row-major and transposed),
the inverse scales saved by the forward, the amax histories and scales after
the update (all bit-exact) and Y, dX, dW, dbias (GEMM tolerances).
"""
import numpy as np
import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
import synth
from helpers import assert_bits_equal, assert_gemm_f32, np_of

pytestmark = pytest.mark.gpu


def _metas_equal(bank, om, what):
    for i, m in enumerate(om):
        assert_bits_equal(np_of(bank.amax_history[i]), m.hist, f"{what}: history {i}")
        assert_bits_equal(np_of(bank.scale[i]), m.scale, f"{what}: scale {i}")
        assert_bits_equal(np_of(bank.scale_inv[i]), m.scale_inv, f"{what}: scale_inv {i}")


def test_linear768_forward_four_steps(oracle):
    m, n, k, L = 1024, 768, 768, 16
    w, b = synth.linear768_weights()
    x = synth.linear768_x(0)
    recipe = F.Recipe(F.FORMAT_E4M3, L, F.AMAX_MAX, 0)
    bank = F.MetaBank([F.E4M3, F.E4M3], L)
    mx, mw = bank.meta(0), bank.meta(1)
    ox, ow = oracle.Meta(L, 0), oracle.Meta(L, 0)
    saved = F.Saved(m, n, k, transposes=False)
    y = torch.empty(m, n, dtype=torch.float32, device="cuda")
    xd, wd, bd = x.cuda(), w.cuda(), b.cuda()
    for step in range(4):
        F.fp8_linear_fwd(xd, wd, y, recipe, mx, mw, saved, bias=bd)
        ref = oracle.linear_fwd(x.numpy(), w.numpy(), ox, ow, bias=b.numpy())
        assert_bits_equal(np_of(saved.xq), ref["xq"], f"step {step} xq")
        assert_bits_equal(np_of(saved.wq), ref["wq"], f"step {step} wq")
        assert_bits_equal(np_of(saved.sinv), np.array([ref["sinv_x"], ref["sinv_w"]]), f"step {step} sinv")
        assert_gemm_f32(np_of(y), ref["y"], f"step {step} y")
        bank.update(recipe)
        oracle.update_metas([ox, ow])
        _metas_equal(bank, [ox, ow], f"step {step}")
    # steady state from step 1 on: the same inputs give the same scale
    assert np_of(bank.scale)[0] == np.float32(448.0 / np.float64(x.max().item()))


def test_linear768_forward_backward_hybrid(oracle):
    m, n, k, L = 1024, 768, 768, 16
    w, b = synth.linear768_weights()
    recipe = F.Recipe(F.FORMAT_HYBRID, L, F.AMAX_MAX, 0)
    bank = F.MetaBank([F.E4M3, F.E4M3, F.E5M2], L)
    mx, mw, mg = bank.meta(0), bank.meta(1), bank.meta(2)
    ox, ow, og = oracle.Meta(L, 0), oracle.Meta(L, 0), oracle.Meta(L, 1)
    saved = F.Saved(m, n, k)
    dev = dict(device="cuda")
    y = torch.empty(m, n, dtype=torch.float32, **dev)
    dx = torch.empty(m, k, dtype=torch.float32, **dev)
    dw = torch.empty(n, k, dtype=torch.float32, **dev)
    db = torch.empty(n, dtype=torch.float32, **dev)
    gq = torch.empty(m, n, dtype=torch.uint8, **dev)
    gqt = torch.empty(n, m, dtype=torch.uint8, **dev)
    ws = torch.empty(F.dbias_workspace_bytes(m, n) // 4, dtype=torch.float32, **dev)
    wd, bd = w.cuda(), b.cuda()
    rows = np.arange(0, m, 37)
    for it in range(16):
        x, dy = synth.linear768_x(it), synth.linear768_dy(it)
        F.fp8_linear_fwd(x.cuda(), wd, y, recipe, mx, mw, saved, bias=bd)
        F.fp8_linear_bwd(dy.cuda(), k, recipe, mg, saved, gq, gqt, dx, dw, dbias=db, dbias_ws=ws)
        fw = oracle.linear_fwd(x.numpy(), w.numpy(), ox, ow, bias=b.numpy(), rows=rows)
        bw = oracle.linear_bwd(dy.numpy(), fw, og, rows_dx=rows)
        tag = f"iteration {it}"
        assert_bits_equal(np_of(saved.xq), fw["xq"], tag + " xq")
        assert_bits_equal(np_of(saved.xq_t), fw["xqt"], tag + " xq_t")
        assert_bits_equal(np_of(saved.wq_t), fw["wqt"], tag + " wq_t")
        assert_bits_equal(np_of(gq), bw["gq"], tag + " dYq")
        assert_bits_equal(np_of(gqt), bw["gqt"], tag + " dYq_t")
        assert_gemm_f32(np_of(y)[rows], fw["y"], tag + " y")
        assert_gemm_f32(np_of(dx)[rows], bw["dx"], tag + " dx")
        assert_gemm_f32(np_of(dw), bw["dw"], tag + " dw")
        ref_db = bw["dbias"]
        assert np.all(np.abs(np_of(db) - ref_db) <= 1e-5 * np.abs(dy.numpy()).sum(0)), tag + " dbias"
        if it == 0:     # dY ~ 2^-20 underflows E5M2 at the initial scale 1: zero gradients
            assert not np.any(np_of(gq) & 0x7F) and not np.any(np_of(dw))
        bank.update(recipe)
        oracle.update_metas([ox, ow, og])
        _metas_equal(bank, [ox, ow, og], tag)
    assert np.count_nonzero(np_of(gq) & 0x7F) > 0.99 * m * n      # the delayed scale lifted dY into range


def test_linear768_forward_backward_all_e4m3(oracle):
    """The all-E4M3 recipe: the gradient is cast to E4M3 as well (fp8_max 448
    in its scale update); 6 iterations, bit-exact codes and metas, GEMM
    tolerances on Y, dX, dW."""
    m, n, k, L = 1024, 768, 768, 16
    w, b = synth.linear768_weights()
    recipe = F.Recipe(F.FORMAT_E4M3, L, F.AMAX_MAX, 0)
    bank = F.MetaBank([F.E4M3, F.E4M3, F.E4M3], L)
    mx, mw, mg = bank.meta(0), bank.meta(1), bank.meta(2)
    ox, ow, og = oracle.Meta(L, 0), oracle.Meta(L, 0), oracle.Meta(L, 0)
    saved = F.Saved(m, n, k)
    dev = dict(device="cuda")
    y = torch.empty(m, n, dtype=torch.float32, **dev)
    dx = torch.empty(m, k, dtype=torch.float32, **dev)
    dw = torch.empty(n, k, dtype=torch.float32, **dev)
    gq = torch.empty(m, n, dtype=torch.uint8, **dev)
    gqt = torch.empty(n, m, dtype=torch.uint8, **dev)
    wd, bd = w.cuda(), b.cuda()
    rows = np.arange(0, m, 41)
    for it in range(6):
        x, dy = synth.linear768_x(it), synth.linear768_dy(it)
        F.fp8_linear_fwd(x.cuda(), wd, y, recipe, mx, mw, saved, bias=bd)
        F.fp8_linear_bwd(dy.cuda(), k, recipe, mg, saved, gq, gqt, dx, dw)
        fw = oracle.linear_fwd(x.numpy(), w.numpy(), ox, ow, bias=b.numpy(), rows=rows)
        bw = oracle.linear_bwd(dy.numpy(), fw, og, rows_dx=rows)
        tag = f"iteration {it}"
        assert_bits_equal(np_of(gq), bw["gq"], tag + " dYq (E4M3)")
        assert_bits_equal(np_of(gqt), bw["gqt"], tag + " dYq_t (E4M3)")
        assert_gemm_f32(np_of(y)[rows], fw["y"], tag + " y")
        assert_gemm_f32(np_of(dx)[rows], bw["dx"], tag + " dx")
        assert_gemm_f32(np_of(dw), bw["dw"], tag + " dw")
        bank.update(recipe)
        oracle.update_metas([ox, ow, og])
        _metas_equal(bank, [ox, ow, og], tag)
    assert np_of(bank.scale)[2] == np.float32(448.0 / np.float64(og.hist[og.hist > 0].max()))


@pytest.mark.parametrize("mode", ["every_step", "first_step"])
def test_linear768_just_in_time(oracle, mode):
    """Just-in-time scaling (recipe.just_in_time) on every step, or on the
    first step only (the initial-amax behaviour) followed by delayed scaling.
    Bit-exact codes, saved inverse scales and metas; GEMM tolerances; the
    first step's E5M2 gradient does not underflow."""
    m, n, k, L = 1024, 768, 768, 16
    w, b = synth.linear768_weights()
    bank = F.MetaBank([F.E4M3, F.E4M3, F.E5M2], L)
    mx, mw, mg = bank.meta(0), bank.meta(1), bank.meta(2)
    ox, ow, og = oracle.Meta(L, 0), oracle.Meta(L, 0), oracle.Meta(L, 1)
    saved = F.Saved(m, n, k)
    dev = dict(device="cuda")
    y = torch.empty(m, n, dtype=torch.float32, **dev)
    dx = torch.empty(m, k, dtype=torch.float32, **dev)
    dw = torch.empty(n, k, dtype=torch.float32, **dev)
    gq = torch.empty(m, n, dtype=torch.uint8, **dev)
    gqt = torch.empty(n, m, dtype=torch.uint8, **dev)
    wd, bd = w.cuda(), b.cuda()
    rows = np.arange(0, m, 53)
    for it in range(4):
        jit = mode == "every_step" or it == 0
        recipe = F.Recipe(F.FORMAT_HYBRID, L, F.AMAX_MAX, 0, just_in_time=jit)
        x, dy = synth.linear768_x(it), synth.linear768_dy(it)
        F.fp8_linear_fwd(x.cuda(), wd, y, recipe, mx, mw, saved, bias=bd)
        F.fp8_linear_bwd(dy.cuda(), k, recipe, mg, saved, gq, gqt, dx, dw)
        fw = oracle.linear_fwd(x.numpy(), w.numpy(), ox, ow, bias=b.numpy(), rows=rows, jit=jit)
        bw = oracle.linear_bwd(dy.numpy(), fw, og, rows_dx=rows, jit=jit)
        tag = f"{mode} iteration {it}"
        assert_bits_equal(np_of(saved.xq), fw["xq"], tag + " xq")
        assert_bits_equal(np_of(saved.wq_t), fw["wqt"], tag + " wq_t")
        assert_bits_equal(np_of(saved.sinv), np.array([fw["sinv_x"], fw["sinv_w"]]), tag + " saved sinv")
        assert_bits_equal(np_of(gq), bw["gq"], tag + " dYq")
        assert_bits_equal(np_of(gqt), bw["gqt"], tag + " dYq_t")
        assert_gemm_f32(np_of(y)[rows], fw["y"], tag + " y")
        assert_gemm_f32(np_of(dx)[rows], bw["dx"], tag + " dx")
        assert_gemm_f32(np_of(dw), bw["dw"], tag + " dw")
        _metas_equal(bank, [ox, ow, og], tag + " before update")
        if it == 0:
            assert np.count_nonzero(np_of(gq) & 0x7F) > 0.99 * m * n     # no underflow at step 0
        bank.update(recipe)
        oracle.update_metas([ox, ow, og])
        _metas_equal(bank, [ox, ow, og], tag)
