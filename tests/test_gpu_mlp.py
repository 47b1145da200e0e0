"""GPU parity of the FP8 MLP block (FC1 -> GeLU -> FC2, HYBRID, delayed
scaling) step by step against the oracle.

Each sub-step is checked on the GPU's own inputs to that sub-step (stepwise
parity): the oracle casts the GPU's H and dZ, so a one-ulp difference in an
upstream bf16 value cannot cascade.  Bit-exact: every FP8 code (row-major and
transposed), the saved inverse scales, every amax, history and scale.  GEMM
tolerances (tests/helpers.py): H, Z, Y, dH, dX (bf16) and dW1, dW2 (fp32) on
the rows the oracle recomputes.  The full-size case is the benchmark's block
(8192 tokens, hidden 4096, FFN 14336) in the same launch configuration.
"""
import numpy as np
import pytest
import torch

import synth
from fp8_mixed_precision_reduce_amd.blocks import MLP_TENSORS, Fp8MlpBlock
from helpers import assert_bits_equal, assert_gemm_bf16, assert_gemm_f32, np_of

pytestmark = pytest.mark.gpu
E4, E5 = 0, 1


def _bf16_ulps(a, b):
    a, b = a.astype(np.int64), b.astype(np.int64)
    return np.abs(np.where(a & 0x8000, -(a & 0x7FFF), a & 0x7FFF) - np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF))


def _check_step(oracle, blk, om, rows, wrows, tag):
    X, W1, W2, dY = (np_of(t) for t in (blk.x, blk.w1, blk.w2, blk.dy))
    s1, s2 = blk.saved1, blk.saved2
    # forward FC1: casts and the GEMM with its GeLU epilogue
    xq, xqt = oracle.cast_transpose(X, E4, om["x"].scale)
    w1q, w1qt = oracle.cast_transpose(W1, E4, om["w1"].scale)
    assert_bits_equal(np_of(s1.xq), xq, tag + " Xq")
    assert_bits_equal(np_of(s1.xq_t), xqt, tag + " Xq^T")
    assert_bits_equal(np_of(s1.wq), w1q, tag + " W1q")
    assert_bits_equal(np_of(s1.wq_t), w1qt, tag + " W1q^T")
    assert_bits_equal(np_of(s1.sinv), np.array([om["x"].scale_inv, om["w1"].scale_inv]), tag + " saved sinv 1")
    h_ref, z_ref = oracle.gemm(xq, E4, w1q, E4, om["x"].scale_inv, om["w1"].scale_inv, gelu=True, rows=rows,
                               want_pre=True)
    H, Z = np_of(blk.h), np_of(blk.z)
    sel = slice(None) if rows is None else rows
    assert_gemm_bf16(H[sel], h_ref, oracle, tag + " H")
    assert_gemm_bf16(Z[sel], z_ref, oracle, tag + " Z")
    # forward FC2 on the GPU's H
    hq, hqt = oracle.cast_transpose(H, E4, om["h"].scale)
    w2q, w2qt = oracle.cast_transpose(W2, E4, om["w2"].scale)
    assert_bits_equal(np_of(s2.xq), hq, tag + " Hq")
    assert_bits_equal(np_of(s2.xq_t), hqt, tag + " Hq^T")
    assert_bits_equal(np_of(s2.wq), w2q, tag + " W2q")
    assert_bits_equal(np_of(s2.wq_t), w2qt, tag + " W2q^T")
    y_ref = oracle.gemm(hq, E4, w2q, E4, om["h"].scale_inv, om["w2"].scale_inv, rows=rows)
    assert_gemm_bf16(np_of(blk.y)[sel], y_ref, oracle, tag + " Y")
    # backward FC2
    gq, gqt = oracle.cast_transpose(dY, E5, om["dy"].scale)
    assert_bits_equal(np_of(blk.dyq), gq, tag + " dYq")
    assert_bits_equal(np_of(blk.dyq_t), gqt, tag + " dYq^T")
    dh_ref = oracle.gemm(gq, E5, w2qt, E4, om["dy"].scale_inv, om["w2"].scale_inv, rows=rows)
    dH = np_of(blk.dh)
    assert_gemm_bf16(dH[sel], dh_ref, oracle, tag + " dH")
    dw2_ref = oracle.gemm(gqt, E5, hqt, E4, om["dy"].scale_inv, om["h"].scale_inv, rows=wrows)
    assert_gemm_f32(np_of(blk.dw2)[slice(None) if wrows is None else wrows], dw2_ref, tag + " dW2")
    # GeLU backward fused into the dZ cast, on the GPU's dH and Z
    dZ = np_of(blk.dz)
    assert _bf16_ulps(dZ, oracle.gelu_bwd(dH, Z)).max() <= 1, tag + " dZ"
    zq, zqt = oracle.cast_transpose(dZ, E5, om["dz"].scale)
    assert_bits_equal(np_of(blk.dzq), zq, tag + " dZq")
    assert_bits_equal(np_of(blk.dzq_t), zqt, tag + " dZq^T")
    dx_ref = oracle.gemm(zq, E5, w1qt, E4, om["dz"].scale_inv, om["w1"].scale_inv, rows=rows)
    assert_gemm_bf16(np_of(blk.dx)[sel], dx_ref, oracle, tag + " dX")
    dw1_ref = oracle.gemm(zqt, E5, xqt, E4, om["dz"].scale_inv, om["x"].scale_inv, rows=wrows)
    assert_gemm_f32(np_of(blk.dw1)[slice(None) if wrows is None else wrows], dw1_ref, tag + " dW1")
    # amaxes of the step (slot 0, before the update), from the same tensors
    for name, t in (("x", X), ("w1", W1), ("h", H), ("w2", W2), ("dy", dY), ("dz", dZ)):
        om[name].record(t)
    return om


def _run_steps(oracle, blk, steps, rows, wrows):
    om = {name: oracle.Meta(blk.bank.history_len, E5 if name.startswith("d") else E4) for name in MLP_TENSORS}
    for step in range(steps):
        tag = f"step {step}"
        blk.forward()
        blk.backward()
        torch.cuda.synchronize()
        _check_step(oracle, blk, om, rows, wrows, tag)
        for i, name in enumerate(MLP_TENSORS):
            assert_bits_equal(np_of(blk.bank.amax_history[i, 0]), om[name].hist[0], f"{tag} amax {name}")
        blk.update()
        oracle.update_metas([om[n] for n in MLP_TENSORS])
        for i, name in enumerate(MLP_TENSORS):
            assert_bits_equal(np_of(blk.bank.amax_history[i]), om[name].hist, f"{tag} history {name}")
            assert_bits_equal(np_of(blk.bank.scale[i]), om[name].scale, f"{tag} scale {name}")
            assert_bits_equal(np_of(blk.bank.scale_inv[i]), om[name].scale_inv, f"{tag} scale_inv {name}")


@pytest.mark.parametrize("fused", [False, True], ids=["separate_casts", "fused_h_cast"])
def test_mlp_block_small_ragged_all_outputs(oracle, fused):
    m, hidden, ffn = 272, 208, 464
    x, w1, w2, dy = synth.mlp_inputs(0, device="cpu", m=m, hidden=hidden, ffn=ffn)
    blk = Fp8MlpBlock(x.cuda(), w1.cuda(), w2.cuda(), dy.cuda(), history_len=16, keep_dz=True, keep_h=True,
                      fuse_casts=fused)
    _run_steps(oracle, blk, steps=4, rows=None, wrows=None)


def test_mlp_block_full_size_sampled(oracle):
    """8192 tokens x hidden 4096 x FFN 14336 (the benchmark's block), 2 steps."""
    x, w1, w2, dy = synth.mlp_inputs(0, device="cuda")
    blk = Fp8MlpBlock(x, w1, w2, dy, history_len=1024, keep_dz=True, keep_h=True)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(8192, 12, replace=False))
    wrows = np.sort(rng.choice(4096, 4, replace=False))
    _run_steps(oracle, blk, steps=2, rows=rows, wrows=wrows)
