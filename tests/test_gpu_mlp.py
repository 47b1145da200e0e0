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
from helpers import (GELU_LIPSCHITZ, assert_bits_equal, assert_fast_bf16, assert_fast_f32, assert_gemm_bf16,
                     assert_gemm_f32, fast_accum_bound, np_of)

pytestmark = pytest.mark.gpu
E4, E5 = 0, 1


def _bf16_ulps(a, b):
    a, b = a.astype(np.int64), b.astype(np.int64)
    return np.abs(np.where(a & 0x8000, -(a & 0x7FFF), a & 0x7FFF) - np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF))


class _GemmCheck:
    """The GEMM comparisons of one step: the fp32-accumulation tolerances of
    tests/helpers.py for the exact inner product, the group-truncation bound
    for the fast one (recipe.fast_accum)."""

    def __init__(self, oracle, fast):
        self.o, self.fast = oracle, fast

    def __call__(self, got, a, af, b, bf, sa, sb, rows, tag, gelu=False, aux=None, f32=False):
        o = self.o
        res = o.gemm(a, af, b, bf, sa, sb, gelu=gelu, rows=rows, want_pre=gelu)
        y, pre = res if gelu else (res, None)
        sel = slice(None) if rows is None else rows
        if not self.fast:
            if f32:
                assert_gemm_f32(got[sel], y, tag)
            else:
                assert_gemm_bf16(got[sel], y, o, tag)
                if aux is not None:
                    assert_gemm_bf16(aux[sel], pre, o, tag + " (pre-GeLU)")
            return
        a_rows = a if rows is None else a[rows]
        bound = fast_accum_bound(o.decode_table(af)[a_rows], o.decode_table(bf)[b], sa, sb)
        if f32:
            assert_fast_f32(got[sel], y, bound, tag)
        else:
            assert_fast_bf16(got[sel], y, bound, tag, lipschitz=GELU_LIPSCHITZ if gelu else 1.0)
            if aux is not None:
                assert_fast_bf16(aux[sel], pre, bound, tag + " (pre-GeLU)")


def _check_step(oracle, blk, om, rows, wrows, tag, fast=False):
    X, W1, W2, dY = (np_of(t) for t in (blk.x, blk.w1, blk.w2, blk.dy))
    s1, s2 = blk.saved1, blk.saved2
    gemm = _GemmCheck(oracle, fast)
    # forward FC1: casts and the GEMM with its GeLU epilogue
    xq, xqt = oracle.cast_transpose(X, E4, om["x"].scale)
    w1q, w1qt = oracle.cast_transpose(W1, E4, om["w1"].scale)
    assert_bits_equal(np_of(s1.xq), xq, tag + " Xq")
    assert_bits_equal(np_of(s1.xq_t), xqt, tag + " Xq^T")
    assert_bits_equal(np_of(s1.wq), w1q, tag + " W1q")
    assert_bits_equal(np_of(s1.wq_t), w1qt, tag + " W1q^T")
    assert_bits_equal(np_of(s1.sinv), np.array([om["x"].scale_inv, om["w1"].scale_inv]), tag + " saved sinv 1")
    H, Z = np_of(blk.h), np_of(blk.z)
    gemm(H, xq, E4, w1q, E4, om["x"].scale_inv, om["w1"].scale_inv, rows, tag + " H", gelu=True, aux=Z)
    # forward FC2 on the GPU's H
    hq, hqt = oracle.cast_transpose(H, E4, om["h"].scale)
    w2q, w2qt = oracle.cast_transpose(W2, E4, om["w2"].scale)
    assert_bits_equal(np_of(s2.xq), hq, tag + " Hq")
    assert_bits_equal(np_of(s2.xq_t), hqt, tag + " Hq^T")
    assert_bits_equal(np_of(s2.wq), w2q, tag + " W2q")
    assert_bits_equal(np_of(s2.wq_t), w2qt, tag + " W2q^T")
    gemm(np_of(blk.y), hq, E4, w2q, E4, om["h"].scale_inv, om["w2"].scale_inv, rows, tag + " Y")
    # backward FC2
    gq, gqt = oracle.cast_transpose(dY, E5, om["dy"].scale)
    assert_bits_equal(np_of(blk.dyq), gq, tag + " dYq")
    assert_bits_equal(np_of(blk.dyq_t), gqt, tag + " dYq^T")
    dH = np_of(blk.dh)
    gemm(dH, gq, E5, w2qt, E4, om["dy"].scale_inv, om["w2"].scale_inv, rows, tag + " dH")
    gemm(np_of(blk.dw2), gqt, E5, hqt, E4, om["dy"].scale_inv, om["h"].scale_inv, wrows, tag + " dW2", f32=True)
    # GeLU backward fused into the dZ cast, on the GPU's dH and Z
    dZ = np_of(blk.dz)
    assert _bf16_ulps(dZ, oracle.gelu_bwd(dH, Z)).max() <= 1, tag + " dZ"
    zq, zqt = oracle.cast_transpose(dZ, E5, om["dz"].scale)
    assert_bits_equal(np_of(blk.dzq), zq, tag + " dZq")
    assert_bits_equal(np_of(blk.dzq_t), zqt, tag + " dZq^T")
    gemm(np_of(blk.dx), zq, E5, w1qt, E4, om["dz"].scale_inv, om["w1"].scale_inv, rows, tag + " dX")
    gemm(np_of(blk.dw1), zqt, E5, xqt, E4, om["dz"].scale_inv, om["x"].scale_inv, wrows, tag + " dW1", f32=True)
    # amaxes of the step (slot 0, before the update), from the same tensors
    for name, t in (("x", X), ("w1", W1), ("h", H), ("w2", W2), ("dy", dY), ("dz", dZ)):
        om[name].record(t)
    return om


def _run_steps(oracle, blk, steps, rows, wrows, fast=False):
    om = {name: oracle.Meta(blk.bank.history_len, E5 if name.startswith("d") else E4) for name in MLP_TENSORS}
    for step in range(steps):
        tag = f"step {step}"
        blk.forward()
        blk.backward()
        torch.cuda.synchronize()
        _check_step(oracle, blk, om, rows, wrows, tag, fast=fast)
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


def test_mlp_block_small_ragged_fast_accum(oracle):
    """The block with the fast inner product (recipe.fast_accum): every code,
    amax, history and scale bit-exact as with the exact one (stepwise), the
    GEMM outputs within the group-truncation bound."""
    m, hidden, ffn = 272, 208, 464
    x, w1, w2, dy = synth.mlp_inputs(0, device="cpu", m=m, hidden=hidden, ffn=ffn)
    blk = Fp8MlpBlock(x.cuda(), w1.cuda(), w2.cuda(), dy.cuda(), history_len=16, keep_dz=True, keep_h=True,
                      fast_accum=True)
    _run_steps(oracle, blk, steps=4, rows=None, wrows=None, fast=True)


@pytest.mark.parametrize("fast", [False, True], ids=["exact", "fast_accum"])
def test_mlp_block_full_size_sampled(oracle, fast):
    """8192 tokens x hidden 4096 x FFN 14336 (the benchmark's block), 2 steps,
    with either inner product."""
    x, w1, w2, dy = synth.mlp_inputs(0, device="cuda")
    blk = Fp8MlpBlock(x, w1, w2, dy, history_len=1024, keep_dz=True, keep_h=True, fast_accum=fast)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(8192, 12 if not fast else 6, replace=False))
    wrows = np.sort(rng.choice(4096, 4 if not fast else 3, replace=False))
    _run_steps(oracle, blk, steps=2, rows=rows, wrows=wrows, fast=fast)


def test_mlp_block_end_to_end_from_inputs_alone(oracle):
    """The oracle runs the whole block from the seeded inputs alone, 4 steps,
    with no GPU value entering it (the stepwise tests above feed each sub-step
    the GPU's own inputs).  Everything that depends only on the inputs and
    their histories is bit-exact: the codes of X, W1, W2 and dY and their
    amaxes, histories and scales.  The chained tensors may differ where a
    one-ulp bf16 difference upstream crosses an FP8 rounding boundary: H and
    Z stay within one bf16 ulp (their inputs are exact), a differing H or dZ
    code is an adjacent code and at most 1% of them differ, and Y, dH, dX,
    dW1, dW2 agree to 1e-2 normwise, far below the FP8 quantisation step
    (2^-4 relative for E4M3)."""
    m, hidden, ffn, L = 272, 208, 464, 16
    x, w1, w2, dy = synth.mlp_inputs(0, device="cpu", m=m, hidden=hidden, ffn=ffn)
    blk = Fp8MlpBlock(x.cuda(), w1.cuda(), w2.cuda(), dy.cuda(), history_len=L, keep_dz=True, keep_h=True)
    X, W1, W2, DY = (np_of(t) for t in (x, w1, w2, dy))
    metas = oracle.mlp_metas(L)
    idx = {name: i for i, name in enumerate(MLP_TENSORS)}

    def ranks(fmt):
        # position of each code's value among the format's distinct finite values (+0 and -0 share one)
        vals = np.array([oracle.decode(c, fmt) for c in range(256)])
        finite = np.unique(vals[np.isfinite(vals)])
        return np.array([np.searchsorted(finite, v) if np.isfinite(v) else -10 for v in vals])

    rank = {E4: ranks(E4), E5: ranks(E5)}

    def code_diff(got, want, fmt, tag):
        d = got != want
        if d.any():
            step = np.abs(rank[fmt][got[d]] - rank[fmt][want[d]])
            assert np.all(step <= 1), tag + ": a differing code is not a neighbouring value"
        assert d.mean() <= 0.01, f"{tag}: {d.mean():.4f} of the codes differ"

    def normwise(got64, want64, tag):
        err = np.linalg.norm(got64 - want64) / np.linalg.norm(want64)
        assert err <= 1e-2, f"{tag}: normwise error {err:.2e}"

    for step in range(4):
        tag = f"step {step}"
        blk.forward()
        blk.backward()
        torch.cuda.synchronize()
        hist_before = np_of(blk.bank.amax_history[:, 0])
        ref = oracle.mlp_step(X, W1, W2, DY, metas)
        blk.update()
        torch.cuda.synchronize()
        # input-only quantities: bit-exact
        assert_bits_equal(np_of(blk.saved1.xq), ref["fw1"]["xq"], tag + " Xq")
        assert_bits_equal(np_of(blk.saved1.wq), ref["fw1"]["wq"], tag + " W1q")
        assert_bits_equal(np_of(blk.saved2.wq), ref["fw2"]["wq"], tag + " W2q")
        assert_bits_equal(np_of(blk.dyq), ref["bw2"]["gq"], tag + " dYq")
        for name in ("x", "w1", "w2", "dy"):
            i = idx[name]
            assert_bits_equal(hist_before[i], np.float32(metas[name].hist[1]), f"{tag} amax {name}")
            assert_bits_equal(np_of(blk.bank.amax_history[i]), metas[name].hist, f"{tag} history {name}")
            assert_bits_equal(np_of(blk.bank.scale[i]), metas[name].scale, f"{tag} scale {name}")
        # chained quantities
        assert _bf16_ulps(np_of(blk.h), ref["h"]).max() <= 1, tag + " H"
        assert _bf16_ulps(np_of(blk.z), ref["z"]).max() <= 1, tag + " Z"
        code_diff(np_of(blk.saved2.xq), ref["fw2"]["xq"], E4, tag + " Hq")
        code_diff(np_of(blk.dzq), ref["bw1"]["gq"], E5, tag + " dZq")
        for name in ("y", "dh", "dx"):
            normwise(oracle.bf16_to_f64(np_of(getattr(blk, name))), oracle.bf16_to_f64(ref[name]), f"{tag} {name}")
        normwise(np_of(blk.dw1).astype(np.float64), ref["dw1"], tag + " dW1")
        normwise(np_of(blk.dw2).astype(np.float64), ref["dw2"], tag + " dW2")
        for name in ("h", "dz"):
            i = idx[name]
            got, want = np_of(blk.bank.scale[i]).astype(np.float64), np.float64(metas[name].scale)
            assert abs(got - want) <= 2.0 ** -7 * want, f"{tag} scale {name}: {got} vs {want}"
