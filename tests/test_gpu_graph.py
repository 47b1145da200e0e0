"""The training steps under HIP graph capture.

The library allocates nothing, issues no memsets and never synchronises, so a
whole step can be captured once and replayed.  Each test captures one step of
a block into a graph, then replays it several times with eager work and
synchronisations in between, and checks every replay bit for bit against an
identical block stepped eagerly: outputs, FP8 codes, histories and scales
(and, for the layer, the loss-scale state and the fp32 masters).
"""
import numpy as np
import pytest
import torch

import synth
from fp8_mixed_precision_reduce_amd.blocks import Fp8MlpBlock, Fp8TransformerLayer
from helpers import assert_bits_equal, np_of

pytestmark = pytest.mark.gpu


def _capture(step):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # warm-up on the side stream, as capture requires
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    return g


def test_mlp_block_step_graph_replays_match_eager():
    m, hidden, ffn = 272, 208, 464
    x, w1, w2, dy = synth.mlp_inputs(0, device="cpu", m=m, hidden=hidden, ffn=ffn)
    eager = Fp8MlpBlock(x.cuda(), w1.cuda(), w2.cuda(), dy.cuda(), history_len=16)
    graphed = Fp8MlpBlock(x.cuda(), w1.cuda(), w2.cuda(), dy.cuda(), history_len=16)
    g = _capture(graphed.step)               # one warm-up step ran; the capture runs nothing
    eager.step()
    for rep in range(5):
        eager.step()
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work between replays
        tag = f"replay {rep}"
        for name in ("z", "y", "dh", "dx", "dw1", "dw2", "dyq", "dzq"):
            assert_bits_equal(np_of(getattr(graphed, name)), np_of(getattr(eager, name)), f"{tag} {name}")
        for what in ("amax_history", "scale", "scale_inv"):
            assert_bits_equal(np_of(getattr(graphed.bank, what)), np_of(getattr(eager.bank, what)), f"{tag} {what}")
        del junk


@pytest.mark.parametrize("attention", [False, True], ids=["stand_in", "attention_core"])
def test_layer_step_graph_replays_match_eager(attention):
    """The whole layer step captured once and replayed (with the attention
    core: 2 sequences of 256 tokens, two heads of 128)."""
    shape = dict(m=512, hidden=256, ffn=464) if attention else dict(m=272, hidden=208, ffn=464)
    inp = synth.layer_inputs(device="cpu", **shape)
    kw = dict(heads=2, batch=2) if attention else {}

    def make():
        d = {k: v.cuda() for k, v in inp.items()}
        return Fp8TransformerLayer(d["x"], d["ctx"], d["g"], d["dqkv"], d["wqkv"], d["wo"], d["w1"], d["w2"],
                                   history_len=16, lr=2.0 ** -10, **kw)
    eager, graphed = make(), make()
    g = _capture(graphed.step)
    eager.step()
    for rep in range(6):                     # crosses the loss-scale growth after 5 clean steps
        eager.step()
        g.replay()
        torch.cuda.synchronize()
        tag = f"replay {rep}"
        for name in ("qkv", "ctx", "y1", "z", "y", "dx", "dctx", "dqkv", "grad", "master", "ls_state"):
            assert_bits_equal(np_of(getattr(graphed, name)), np_of(getattr(eager, name)), f"{tag} {name}")
        for what in ("amax_history", "scale", "scale_inv"):
            assert_bits_equal(np_of(getattr(graphed.bank, what)), np_of(getattr(eager.bank, what)), f"{tag} {what}")
    assert float(np_of(eager.ls_state)[0]) == 2.0 ** 17
