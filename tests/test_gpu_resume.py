"""Checkpoint / resume and determinism.

The training state of the layer is plain device buffers (fp32 masters, the
twelve amax histories with their scales, the loss-scale state); a run saved
after step k and restored into freshly built buffers must continue bit for bit
like the uninterrupted run.  The kernels use no atomics on floating point
values, so two runs of the same step on the same inputs give identical bytes.
"""
import io

import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
import synth
from fp8_mixed_precision_reduce_amd.blocks import Fp8MlpBlock, Fp8TransformerLayer
from helpers import assert_bits_equal, np_of

pytestmark = pytest.mark.gpu


def _roundtrip(state):
    """Through a checkpoint file: torch.save, then the loader that executes nothing."""
    buf = io.BytesIO()
    torch.save(state, buf)
    buf.seek(0)
    return torch.load(buf, weights_only=True)


def _layer(inp, **kw):
    d = {k: v.cuda() for k, v in inp.items()}
    return Fp8TransformerLayer(d["x"], d["ctx"], d["g"], d["dqkv"], d["wqkv"], d["wo"], d["w1"], d["w2"],
                               history_len=16, lr=2.0 ** -10, **kw), d


@pytest.mark.parametrize("attention", [False, True], ids=["stand_in", "attention_core"])
def test_layer_resume_is_bit_identical(attention):
    """Steps 0..5 with the x100 spike at step 3: uninterrupted, and saved after
    step 2 then restored into a fresh layer for steps 3..5."""
    shape = dict(m=512, hidden=256, ffn=464) if attention else dict(m=272, hidden=208, ffn=464)
    kw = dict(heads=2, batch=2) if attention else {}
    inp = synth.layer_inputs(device="cpu", **shape)
    spiked = synth.layer_spike(inp["x"]).cuda()

    whole, _ = _layer(inp, **kw)
    for step in range(6):
        whole.step(spiked if step == 3 else None)
    first, _ = _layer(inp, **kw)
    for step in range(3):
        first.step()
    state = _roundtrip(first.state_dict())
    del first
    resumed, _ = _layer(inp, **kw)
    resumed.load_state_dict(state)
    for step in range(3, 6):
        resumed.step(spiked if step == 3 else None)
    torch.cuda.synchronize()
    for name in ("master", "ls_state", "y", "dx", "dqkv", "grad"):
        assert_bits_equal(np_of(getattr(resumed, name)), np_of(getattr(whole, name)), name)
    for what in ("amax_history", "scale", "scale_inv"):
        assert_bits_equal(np_of(getattr(resumed.bank, what)), np_of(getattr(whole.bank, what)), what)
    assert float(np_of(whole.ls_state)[0]) == 2.0 ** 17              # grown after five clean steps


def test_mlp_block_resume_is_bit_identical():
    x, w1, w2, dy = (t.cuda() for t in synth.mlp_inputs(device="cpu", m=272, hidden=208, ffn=464))

    def make():
        return Fp8MlpBlock(x, w1, w2, dy, history_len=16)
    whole = make()
    for _ in range(4):
        whole.step()
    first = make()
    for _ in range(2):
        first.step()
    state = _roundtrip(first.state_dict())
    resumed = make()
    resumed.load_state_dict(state)
    for _ in range(2):
        resumed.step()
    torch.cuda.synchronize()
    for name in ("y", "dx", "dw1", "dw2"):
        assert_bits_equal(np_of(getattr(resumed, name)), np_of(getattr(whole, name)), name)
    for what in ("amax_history", "scale", "scale_inv"):
        assert_bits_equal(np_of(getattr(resumed.bank, what)), np_of(getattr(whole.bank, what)), what)


def test_load_state_rejects_a_different_layout():
    inp = synth.layer_inputs(device="cpu", m=272, hidden=208, ffn=464)
    lay, _ = _layer(inp)
    state = lay.state_dict()
    state["bank"]["formats"] = torch.zeros_like(state["bank"]["formats"])
    with pytest.raises(ValueError):
        lay.load_state_dict(state)


def test_attention_is_deterministic():
    """Two runs of the attention forward and backward at the layer's full shape
    give identical bytes (no floating-point atomics anywhere)."""
    batch, seq, heads = 2, 4096, 64
    qkv, dctx = synth.attention_inputs(batch, seq, heads, device="cuda")
    ws = torch.empty(max(F.attention_workspace_bytes(batch, seq, heads, backward=bw) for bw in (False, True)),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        ctx = torch.empty(batch * seq, heads * 128, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(batch, heads, seq, device="cuda")
        dqkv = torch.empty_like(qkv)
        F.bf16_attention_fwd(qkv, batch, heads, ctx, lse, ws)
        F.bf16_attention_bwd(qkv, ctx, lse, dctx, batch, heads, dqkv, ws)
        outs.append((ctx, lse, dqkv))
    torch.cuda.synchronize()
    for a, b, name in zip(outs[0], outs[1], ("ctx", "lse", "dqkv")):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                           b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32)), name
