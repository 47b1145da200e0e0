"""Pins for the oracle's transformer-layer step (CPU only).

The layer step chains pinned pieces (casts, FP8 GEMMs, GeLU, loss scaling,
SGD); what is new in it is the wiring: which tensor feeds which linear, which
meta scales which cast, where the two residual paths add their gradients and
which operands the dgrad/wgrad products take.  The pin derives that wiring
independently: the same layer written as a float64 torch autograd graph, with
each FP8 linear a custom function whose forward multiplies the dequantised FP8
copies of its input and weight and whose backward quantises the incoming
gradient with the gradient meta's scale (the backward runs on the forward's
FP8 copies, as the FP8 linear does).  Autograd then decides where every
gradient goes.  Stored activations and activation gradients are rounded to
bf16 at the places the layer stores them, so the two computations agree to
fp64 summation order.  GeLU and its derivative come from scipy here.

Further pins: an Inf in the upstream gradient skips the update and halves S;
the x100 spike saturates the input cast of the next step and its amax enters
the history.
"""
import numpy as np
import pytest
import torch
from scipy.special import erfc

E4, E5 = 0, 1
M, H, FF = 32, 16, 48


def _inputs(seed=5):
    rng = np.random.default_rng(seed)

    def bf(shape, std):
        v = (rng.standard_normal(shape) * std).astype(np.float32)
        return (v.view(np.uint32) >> 16).astype(np.uint16)       # truncation: any bf16 values will do

    masters = {"wqkv": (rng.standard_normal((3 * H, H)) * 0.2).astype(np.float32),
               "wo": (rng.standard_normal((H, H)) * 0.2).astype(np.float32),
               "w1": (rng.standard_normal((FF, H)) * 0.2).astype(np.float32),
               "w2": (rng.standard_normal((H, FF)) * 0.2).astype(np.float32)}
    return dict(x=bf((M, H), 1.0), ctx=bf((M, H), 1.0), g=bf((M, H), 2.0 ** -12),
                dqkv=bf((M, 3 * H), 2.0 ** -12)), masters


def _bits_to_f64(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _round_bf16(t, oracle):
    return torch.from_numpy(_bits_to_f64(oracle.bf16_from_f64(t.detach().numpy())))


def _autograd_layer(oracle, inp, masters, metas, S):
    """The layer as a float64 autograd graph; returns Y, dX, dctx, and the
    weight gradients divided by S."""

    def qdq(t, meta, stored):
        v = t.detach().numpy()
        arr = oracle.bf16_from_f64(v) if stored == "bf16" else v.astype(np.float32)
        codes = oracle.cast(arr, meta.fmt, meta.scale)
        return torch.from_numpy(oracle.decode_table(meta.fmt)[codes] * np.float64(meta.scale_inv))

    class Fp8Linear(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, w, mx, mw, mg, x_stored):
            xq, wq = qdq(x, mx, x_stored), qdq(w, mw, "f32")
            ctx.save_for_backward(xq, wq)
            ctx.mg = mg
            return xq @ wq.T

        @staticmethod
        def backward(ctx, gy):
            xq, wq = ctx.saved_tensors
            gq = qdq(gy, ctx.mg, "bf16")
            return gq @ wq, gq.T @ xq, None, None, None, None

    class Store(torch.autograd.Function):
        """A bf16 tensor: the value is rounded, and so is the gradient it receives."""
        @staticmethod
        def forward(ctx, t):
            return _round_bf16(t, oracle)

        @staticmethod
        def backward(ctx, g):
            return _round_bf16(g, oracle)

    class GeluStore(Function := torch.autograd.Function):
        """FC1's epilogue: H = bf16(gelu(pre)) and Z = bf16(pre) kept for the
        backward, dZ = bf16(dH * gelu'(Z))."""
        @staticmethod
        def forward(ctx, pre):
            p = pre.detach().numpy()
            z = _bits_to_f64(oracle.bf16_from_f64(p))
            ctx.z = z
            return _round_bf16(torch.from_numpy(0.5 * p * erfc(-p / np.sqrt(2.0))), oracle)

        @staticmethod
        def backward(ctx, gh):
            z = ctx.z
            dh = _round_bf16(gh, oracle).numpy()
            d = 0.5 * erfc(-z / np.sqrt(2.0)) + z * np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)
            return _round_bf16(torch.from_numpy(dh * d), oracle)

    f64 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x = f64(_bits_to_f64(inp["x"])).requires_grad_()
    ctx_in = f64(_bits_to_f64(inp["ctx"])).requires_grad_()
    w = {k: f64(v).requires_grad_() for k, v in masters.items()}
    mt = metas
    qkv = Store.apply(Fp8Linear.apply(x, w["wqkv"], mt["x"], mt["wqkv"], mt["g_qkv"], "bf16"))
    y1 = Store.apply(Fp8Linear.apply(ctx_in, w["wo"], mt["ctx"], mt["wo"], mt["g_o"], "bf16") + x)
    h = GeluStore.apply(Fp8Linear.apply(y1, w["w1"], mt["y1"], mt["w1"], mt["g_fc1"], "bf16"))
    y = Store.apply(Fp8Linear.apply(h, w["w2"], mt["h"], mt["w2"], mt["g_fc2"], "bf16") + y1)
    loss = ((y * f64(_bits_to_f64(inp["g"]))).sum() + (qkv * f64(_bits_to_f64(inp["dqkv"]))).sum()) * float(S)
    loss.backward()
    grads = {k: v.grad.numpy() for k, v in w.items()}
    return (y.detach().numpy(), _round_bf16(x.grad, oracle).numpy(), _round_bf16(ctx_in.grad, oracle).numpy(),
            grads)


def _run(oracle, steps, inp, masters, L=8):
    metas = oracle.layer_metas(L)
    ls = oracle.LossScale(2.0 ** 4, interval=5)
    outs = []
    for _ in range(steps):
        before = {k: m.copy() for k, m in metas.items()}
        w_before = {k: v.copy() for k, v in masters.items()}
        S = np.float32(ls.state[0])
        out = oracle.layer_step(inp["x"], inp["ctx"], inp["g"], inp["dqkv"], masters, metas, ls, 2.0 ** -10)
        outs.append((before, w_before, S, out))
    return outs, metas, ls


def test_layer_step_matches_autograd_wiring(oracle):
    inp, masters = _inputs()
    outs, _, _ = _run(oracle, 3, inp, masters)
    for step, (before, w_before, S, out) in enumerate(outs):
        y, dx, dctx, grads = _autograd_layer(oracle, inp, w_before, before, S)
        assert np.array_equal(_bits_to_f64(out["y"]), y), f"step {step} Y"
        assert np.array_equal(_bits_to_f64(out["dx"]), dx), f"step {step} dX"
        assert np.array_equal(_bits_to_f64(out["dctx"]), dctx), f"step {step} dctx"
        for name in oracle.LAYER_WEIGHTS:
            want = grads[name]
            got = out["grads"][name].astype(np.float64)
            err = np.linalg.norm(got - want) / np.linalg.norm(want)
            assert err <= 2.0 ** -23, (step, name, err)
    # every gradient meta saw its tensor from step 1 on (step 0 casts unscaled)
    assert all(np.any(outs[-1][3]["grads"][n] != 0) for n in oracle.LAYER_WEIGHTS)


def test_layer_step_sgd_moves_masters_by_unscaled_gradient(oracle):
    inp, masters = _inputs(7)
    outs, _, ls = _run(oracle, 2, inp, masters)
    (_, w0, S0, out0), (_, w1, _, _) = outs
    assert not ls.found_inf
    for name in oracle.LAYER_WEIGHTS:
        g = out0["grads"][name]
        want = w0[name] - np.float32(2.0 ** -10) * (g * (np.float32(1.0) / S0))
        assert np.array_equal(w1[name], want), name


def test_layer_step_inf_gradient_skips_update_and_backs_off(oracle):
    inp, masters = _inputs(9)
    outs, metas, ls = _run(oracle, 1, inp, masters)
    g_bad = inp["g"].copy()
    g_bad[3, 5] = 0x7F80                                      # +Inf
    w_before = {k: v.copy() for k, v in masters.items()}
    S = float(ls.state[0])
    oracle.layer_step(inp["x"], inp["ctx"], g_bad, inp["dqkv"], masters, metas, ls, 2.0 ** -10)
    assert ls.found_inf and ls.state[0] == S / 2 and ls.state[1] == 0.0
    assert np.isinf(metas["g_fc2"].hist[1])                   # the Inf amax is in the rolled history
    for name in oracle.LAYER_WEIGHTS:
        assert np.array_equal(masters[name], w_before[name]), name
    # the scale of dY ignores the non-finite entry: it equals the clean rule over the finite ones
    finite = metas["g_fc2"].hist[np.isfinite(metas["g_fc2"].hist)]
    assert metas["g_fc2"].scale == np.float32(57344.0 / np.float64(finite.max()))


def test_layer_step_spike_saturates_then_rescales(oracle):
    inp, masters = _inputs(11)
    outs, metas, ls = _run(oracle, 2, inp, masters)
    sx = np.float32(metas["x"].scale)
    spiked = oracle.bf16_from_f32(_bits_to_f64(inp["x"]).astype(np.float32) * np.float32(100.0))
    out = oracle.layer_step(spiked, inp["ctx"], inp["g"], inp["dqkv"], masters, metas, ls, 2.0 ** -10)
    codes = out["fwd"]["qkv"]["xq"]
    sat = np.count_nonzero((codes & 0x7F) == 0x7E)            # +-448
    assert sat > 0.5 * codes.size                             # the delayed scale saturates most of X
    a_spike = oracle.amax(spiked)
    assert metas["x"].hist[1] == a_spike                      # recorded, then rolled to slot 1
    assert metas["x"].scale == np.float32(448.0 / np.float64(a_spike)) and metas["x"].scale < sx
    out2 = oracle.layer_step(inp["x"], inp["ctx"], inp["g"], inp["dqkv"], masters, metas, ls, 2.0 ** -10)
    assert not np.any((out2["fwd"]["qkv"]["xq"] & 0x7F) == 0x7E)   # back to the clean input: no saturation
