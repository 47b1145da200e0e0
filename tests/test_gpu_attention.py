"""Parity of the bf16 attention core (bf16_attention_fwd / _bwd through the C
ABI) with the fp64 oracle.

Tolerance, derived from the arithmetic (every element, bf16 unit roundoff
u = 2^-9):
* O = sum_k p_k v_k / l with p_k rounded to bf16 for the product (relative
  error <= u each), fp32 sums and exp2, then one rounding of O to bf16:
  |O_gpu - O| <= u * A + u * |O| + (fp32 terms), A = sum_k P |V| (the
  oracle's absolute-term sum).  Tested with 2u: |err| <= 2^-8 (A + |O|).
* dV, dK, dQ: one bf16 rounding of P or dS per term of the final contraction
  plus the output rounding; dS = P (dP - D) is formed in fp32 from fp32 dP and D
  (their rounding errors are ~2^-24 of |dP| + |D|), so with
  T = sum of |P| (|dP| + |D|) |operand| (the oracle's t*) the same 2^-8 (T + |x|)
  bound holds.
* lse: the kernel's base-2 value times ln 2 against the natural-log LSE,
  |err| <= 2^-16 (1 + |lse|) (fp32 sums, exp2/log2 to about an ulp).
The oracle's backward takes the GPU's bf16 O as the saved forward output (the
method's backward works from the saved O)."""
import numpy as np
import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
import synth
from oracle import attention as A
from helpers import assert_within_terms as _assert_within, bf16_bits_to_f64, np_of

pytestmark = pytest.mark.gpu
LN2 = float(np.log(2.0))


def _run_fwd(qkv, batch, heads):
    seq = qkv.shape[0] // batch
    hd = qkv.shape[1] // 3
    ctx = torch.empty(qkv.shape[0], hd, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(batch, heads, seq, dtype=torch.float32, device="cuda")
    ws = torch.empty(F.attention_workspace_bytes(batch, seq, heads), dtype=torch.uint8, device="cuda")
    F.bf16_attention_fwd(qkv, batch, heads, ctx, lse, ws)
    return ctx, lse


def _run_bwd(qkv, ctx, lse, dctx, batch, heads):
    seq = qkv.shape[0] // batch
    dqkv = torch.full_like(qkv, float("nan"))
    ws = torch.empty(F.attention_workspace_bytes(batch, seq, heads, backward=True), dtype=torch.uint8, device="cuda")
    F.bf16_attention_bwd(qkv, ctx, lse, dctx, batch, heads, dqkv, ws)
    return dqkv


@pytest.mark.parametrize("batch,seq,heads,std", [(1, 256, 2, 1.0), (2, 512, 3, 1.0), (1, 768, 2, 3.0)],
                         ids=["b1s256h2", "b2s512h3", "b1s768h2_peaky"])
def test_attention_matches_oracle(batch, seq, heads, std):
    qkv, dctx = synth.attention_inputs(batch, seq, heads, std=std, seed=synth.seed_of(5, 0, 20) + seq + heads)
    qkv_d, dctx_d = qkv.cuda(), dctx.cuda()
    ctx, lse = _run_fwd(qkv_d, batch, heads)
    dqkv = _run_bwd(qkv_d, ctx, lse, dctx_d, batch, heads)
    torch.cuda.synchronize()

    qkv_b = np_of(qkv)
    o_ref, lse_ref, a_ref = A.attention_fwd(qkv_b, batch, seq, heads)
    _assert_within(np_of(ctx), o_ref, a_ref, "ctx")
    lse_got = lse.cpu().numpy().astype(np.float64) * LN2
    assert np.all(np.abs(lse_got - lse_ref) <= 2.0 ** -16 * (1 + np.abs(lse_ref))), "lse"

    d_ref, t_ref = A.attention_bwd(qkv_b, np_of(ctx), np_of(dctx), batch, seq, heads)
    got = np_of(dqkv)
    hd = heads * 128
    for part, name in enumerate(("dq", "dk", "dv")):
        sl = slice(part * hd, (part + 1) * hd)
        _assert_within(got[:, sl], d_ref[:, sl], t_ref[:, sl], name)


def test_attention_full_size_sampled():
    """The layer's attention (batch 2, seq 4096, 64 heads of 128) in the
    launch configuration the layer step uses; the oracle checks the forward on
    64 query rows of two heads and the whole backward of one head."""
    batch, seq, heads = 2, 4096, 64
    qkv, dctx = synth.attention_inputs(batch, seq, heads, device="cuda")
    ctx, lse = _run_fwd(qkv, batch, heads)
    dqkv = _run_bwd(qkv, ctx, lse, dctx, batch, heads)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    hd = heads * 128
    for b, h in ((0, 0), (1, 37)):
        rows = np.sort(rng.choice(seq, 64, replace=False))
        tok = b * seq + rows
        # the head's slices of qkv, ctx, dctx as a one-batch, one-head problem
        cols = [p * hd + h * 128 + np.arange(128) for p in range(3)]
        sub = np_of(qkv[b * seq:(b + 1) * seq])[:, np.concatenate(cols)]
        q, k, v = A.split_heads(sub, 1, seq, 1)
        o, l, a = A.head_fwd(q[0, 0], k[0, 0], v[0, 0], rows=rows)
        got_o = np_of(ctx[torch.as_tensor(tok, device="cuda")])[:, h * 128:(h + 1) * 128]
        _assert_within(got_o, o, a, f"ctx b{b} h{h}")
        got_l = lse[b, h].cpu().numpy().astype(np.float64)[rows] * LN2
        assert np.all(np.abs(got_l - l) <= 2.0 ** -16 * (1 + np.abs(l))), "lse"
        if (b, h) == (1, 37):
            o_saved = bf16_bits_to_f64(np_of(ctx[b * seq:(b + 1) * seq])[:, h * 128:(h + 1) * 128])
            do = bf16_bits_to_f64(np_of(dctx[b * seq:(b + 1) * seq])[:, h * 128:(h + 1) * 128])
            g = A.head_bwd(q[0, 0], k[0, 0], v[0, 0], o_saved, do)
            got = np_of(dqkv[b * seq:(b + 1) * seq])
            for p, name in enumerate(("dq", "dk", "dv")):
                _assert_within(got[:, cols[p]], g[name], g["t" + name[1]], f"{name} b{b} h{h}")


def test_attention_shapes_rejected_before_launch():
    qkv = torch.zeros(256, 3 * 2 * 64, dtype=torch.bfloat16, device="cuda")
    ctx = torch.zeros(256, 2 * 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 2, 256, device="cuda")
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(F.Fp8LinError) as e:
        F.bf16_attention_fwd(qkv, 1, 2, ctx, lse, ws)
    assert e.value.status == F.ERR_UNSUPPORTED
    qkv = torch.zeros(200, 3 * 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(F.Fp8LinError) as e:
        F.bf16_attention_fwd(qkv, 1, 1, ctx, lse, ws)
    assert e.value.status == F.ERR_SHAPE
