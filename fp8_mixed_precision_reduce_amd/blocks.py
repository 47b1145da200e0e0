"""Layer compositions over the C entry points (argument marshalling only).

Fp8MlpBlock: the FC1 -> GeLU -> FC2 block of a transformer layer with FP8
linears and per-tensor delayed scaling ([TE-KR] "Using FP8 with Transformer
Engine": Linear layers under an FP8 autocast with a DelayedScaling recipe;
HYBRID formats).  One step() is the forward pass, the backward pass and the
per-step history/scale update of all six FP8 tensors (X, W1, H, W2, dY, dZ),
every part of it in the library's kernels:

  fp8_linear_fwd(X, W1, GELU)  -> H = gelu(Z) (bf16), Z kept for backward
  fp8_linear_fwd(H, W2)        -> Y (bf16)
  (fuse_casts=True: H leaves FC1's epilogue already cast to E4M3 -- codes and
  transposed codes straight into FC2's saved operands, amax(H) into H's history
  -- and FC2 skips its input cast.  Measured on MI355X the fused epilogue costs
  the GEMM about what the separate cast costs, so it is off by default.)
  fp8_linear_bwd(dY; W2)       -> dH (bf16), dW2 (fp32)
  fp8_linear_bwd(dH; W1, Z)    -> GeLU backward fused into the dZ cast, dX (bf16), dW1 (fp32)
  fp8_amax_scale_update(6 tensors)

Fp8TransformerLayer: the four FP8 linears of a transformer layer (QKV,
attention output, FC1, FC2) around the bf16 attention core, trained from fp32
master weights with dynamic loss scaling and SGD; see its docstring for the
wiring.

Page tags: [TE-KR] "Transformer Engine으로 FP8 사용하기" (coniverse.tistory.com);
[MP-KR] "LLM) Mixed-Precision 개념 및 학습 방법 알아보기" (data-newbie.tistory.com);
[PT-VI] "Các kiểu dữ liệu FP8 gốc của PyTorch" (hotroai.com).
"""
import torch

from . import (AMAX_MAX, E4M3, E5M2, EPI_GELU, FORMAT_HYBRID, MetaBank, QOut, Recipe, Saved, attention_workspace_bytes,
               bf16_attention_bwd, bf16_attention_fwd, fp8_linear_bwd, fp8_linear_fwd, fp8_loss_scale_apply,
               fp8_loss_scale_update, fp8_sgd_step, fp8_sgd_step_cast)

MLP_TENSORS = ("x", "w1", "h", "w2", "dy", "dz")


class Fp8MlpBlock:
    """Buffers, metas and one training step of the FP8 MLP block.

    x [m][hidden], w1 [ffn][hidden], w2 [hidden][ffn], dy [m][hidden]: bf16 (or
    fp32) device tensors owned by the caller.  keep_dz=True also writes the
    rounded GeLU-backward gradient dZ, keep_h=True the bf16 H (for inspection;
    with fuse_casts=False H is always written)."""

    def __init__(self, x, w1, w2, dy, history_len=1024, fast_accum=False, keep_dz=False, fuse_casts=False,
                 keep_h=False):
        m, hidden = x.shape
        ffn = w1.shape[0]
        assert w1.shape == (ffn, hidden) and w2.shape == (hidden, ffn) and dy.shape == (m, hidden)
        dev = x.device
        self.m, self.hidden, self.ffn = m, hidden, ffn
        self.x, self.w1, self.w2, self.dy = x, w1, w2, dy
        act = dict(dtype=x.dtype, device=dev)
        self.fuse_casts = fuse_casts and x.dtype == torch.bfloat16
        self.h = torch.empty(m, ffn, **act) if (keep_h or not self.fuse_casts) else None
        self.z = torch.empty(m, ffn, **act)
        self.y = torch.empty(m, hidden, **act)
        self.dh = torch.empty(m, ffn, **act)
        self.dx = torch.empty(m, hidden, **act)
        self.dz = torch.empty(m, ffn, **act) if keep_dz else None
        self.dw1 = torch.empty(ffn, hidden, dtype=torch.float32, device=dev)
        self.dw2 = torch.empty(hidden, ffn, dtype=torch.float32, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.dyq, self.dyq_t = torch.empty(m, hidden, **u8), torch.empty(hidden, m, **u8)
        self.dzq, self.dzq_t = torch.empty(m, ffn, **u8), torch.empty(ffn, m, **u8)
        self.saved1 = Saved(m, ffn, hidden, device=dev)        # X, W1 codes
        self.saved2 = Saved(m, hidden, ffn, device=dev)        # H, W2 codes
        self.bank = MetaBank([E4M3, E4M3, E4M3, E4M3, E5M2, E5M2], history_len, device=dev)
        self.meta = {name: self.bank.meta(i) for i, name in enumerate(MLP_TENSORS)}
        self.recipe = Recipe(FORMAT_HYBRID, history_len, AMAX_MAX, 0, fast_accum)

    def forward(self):
        r, mt = self.recipe, self.meta
        if self.fuse_casts and not r.just_in_time:
            hq = QOut(mt["h"].scale, self.saved2.xq, self.saved2.xq_t, E4M3)
            fp8_linear_fwd(self.x, self.w1, self.h, r, mt["x"], mt["w1"], self.saved1, epilogue=EPI_GELU,
                           y_aux=self.z, y_q=hq, y_amax_slot=mt["h"].amax_history[0:1])
            fp8_linear_fwd(None, self.w2, self.y, r, mt["h"], mt["w2"], self.saved2)
        else:
            fp8_linear_fwd(self.x, self.w1, self.h, r, mt["x"], mt["w1"], self.saved1, epilogue=EPI_GELU, y_aux=self.z)
            fp8_linear_fwd(self.h, self.w2, self.y, r, mt["h"], mt["w2"], self.saved2)

    def backward(self):
        r, mt = self.recipe, self.meta
        fp8_linear_bwd(self.dy, self.ffn, r, mt["dy"], self.saved2, self.dyq, self.dyq_t, dx=self.dh, dw=self.dw2)
        fp8_linear_bwd(self.dh, self.hidden, r, mt["dz"], self.saved1, self.dzq, self.dzq_t, dx=self.dx,
                       dw=self.dw1, gelu_z=self.z, dz_out=self.dz)

    def update(self):
        self.bank.update(self.recipe)

    def step(self, record=None):
        """One step; with a list as `record`, appends the step's per-tensor
        amax, scales and (when counting) saturated codes, taken before the
        update (see metrics())."""
        self.forward()
        self.backward()
        if record is not None:
            record.append(self.metrics())
        self.update()

    def count_saturation(self, enable=True):
        """Opt-in saturated-code counters for the block's six tensors."""
        self.bank.count_saturation(enable)

    def metrics(self, clear=True):
        """Host snapshot per tensor name: amax slot 0, scale, inverse scale and
        (when counting) saturated codes since the last snapshot."""
        return self.bank.snapshot(MLP_TENSORS, clear)

    def state_dict(self):
        """The block's training state: the delayed-scaling metas (its weights
        are the caller's and are not updated here)."""
        return {"bank": self.bank.state_dict()}

    def load_state_dict(self, state):
        self.bank.load_state_dict(state["bank"])


LAYER_TENSORS = ("x", "wqkv", "ctx", "wo", "y1", "w1", "h", "w2", "g_fc2", "g_fc1", "g_o", "g_qkv")
LAYER_GRADS = ("g_fc2", "g_fc1", "g_o", "g_qkv")
LAYER_WEIGHTS = ("wqkv", "wo", "w1", "w2")


class Fp8TransformerLayer:
    """One transformer layer's FP8 linears around its bf16 attention core,
    trained with fp32 masters.

    Wiring (no normalisation layers, which the pages do not name):
        QKV = X Wqkv^T
        ctx = attention(QKV)                  bf16 scaled dot-product attention,
                                              `heads` heads of width hidden/heads
                                              over `batch` sequences of m/batch tokens
        Y1  = X + ctx Wo^T
        H   = gelu(Y1 W1^T),  Z kept
        Y   = Y1 + H W2^T
    Loss <Y, G> * S, so dY = bf16(G * S).  Backward:
        dH, dW2          = bwd FC2(dY)
        dY1, dW1         = bwd FC1(dH; gelu'(Z)) + dY          (skip path)
        dctx, dWo        = bwd O(dY1)
        dqkv             = bwd attention(dctx)
        dX, dWqkv        = bwd QKV(dqkv) + dY1                 (skip path)
    With heads=None the attention core is stood in for by the caller's
    tensors: ctx is the O linear's input and the QKV linear's gradient is
    bf16(dqkv * S) (the QKV output is computed and left unused).
    Update, all on the device and in this order ([MP-KR] "Mixed-Precision
    Training Iteration" and its dynamic loss scaling; [PT-VI] training script
    for the per-step history update after backward):
        fp8_loss_scale_update from the four gradient amax slots (Inf/NaN ->
        found_inf, S halves), fp8_amax_scale_update of the twelve metas, then
        the SGD step on the masters (skipped on found_inf).  Under delayed
        scaling (fuse_sgd_cast, the default) each weight's SGD step also casts
        the updated master to E4M3 with the scale the update just set and
        merges its amax into the rolled history, i.e. the cast the next
        forward would make, done while the master is in registers
        (fp8_sgd_step_cast); that forward then takes W pre-cast.  Otherwise
        fp8_sgd_step runs on all masters at once and every forward casts W.

    The masters live in one fp32 buffer and their gradients in another.  x, g (and the stand-ins ctx,
    dqkv) are bf16 device tensors of the caller; forward(x_in) may take another
    input of x's shape (the spiked one).  Residual adds happen in the GEMM
    epilogues; with fuse_casts (delayed scaling only; off by default, see the
    module notes) Y1 and H are also cast to E4M3 there, straight into the next
    linear's saved operands, so FC1 and FC2 skip their input casts (keep_h=True
    still writes the bf16 H).
    """

    def __init__(self, x, ctx, g, dqkv, wqkv, wo, w1, w2, history_len=1024, lr=2.0 ** -10, loss_scale=2.0 ** 16,
                 growth_interval=5, fast_accum=False, keep_dz=False, keep_codes=False, fuse_casts=False,
                 keep_h=False, heads=None, batch=1, fuse_sgd_cast=True):
        m, hid = x.shape
        ffn = w1.shape[0]
        assert wqkv.shape == (3 * hid, hid) and wo.shape == (hid, hid) and w1.shape == (ffn, hid)
        assert w2.shape == (hid, ffn) and g.shape == (m, hid)
        if heads is None:
            assert ctx is not None and dqkv is not None and ctx.shape == (m, hid) and dqkv.shape == (m, 3 * hid)
        else:
            assert hid % heads == 0 and m % batch == 0 and x.dtype == torch.bfloat16
        dev = x.device
        self.m, self.hidden, self.ffn = m, hid, ffn
        self.x, self.ctx, self.g, self.dqkv_in = x, ctx, g, dqkv
        self.lr, self.growth_interval = lr, growth_interval
        shapes = {"wqkv": (3 * hid, hid), "wo": (hid, hid), "w1": (ffn, hid), "w2": (hid, ffn)}
        total = sum(a * b for a, b in shapes.values())
        self.master = torch.empty(total, dtype=torch.float32, device=dev)
        self.grad = torch.empty(total, dtype=torch.float32, device=dev)
        self.w, self.dw, off = {}, {}, 0
        for name, src in zip(LAYER_WEIGHTS, (wqkv, wo, w1, w2)):
            n = src.numel()
            self.w[name] = self.master[off:off + n].view(shapes[name])
            self.w[name].copy_(src)
            self.dw[name] = self.grad[off:off + n].view(shapes[name])
            off += n          # every size is a multiple of 256 elements: the views stay 16-byte aligned
        act = dict(dtype=x.dtype, device=dev)
        self.fuse_casts = fuse_casts and x.dtype == torch.bfloat16
        self.fuse_sgd_cast = fuse_sgd_cast
        self._w_cast = False        # the saved W codes hold the masters cast with the current W scales
        self.qkv = torch.empty(m, 3 * hid, **act)
        self.y1 = torch.empty(m, hid, **act)
        self.z = torch.empty(m, ffn, **act)
        self.h = torch.empty(m, ffn, **act) if (keep_h or not self.fuse_casts) else None
        self.y = torch.empty(m, hid, **act)
        self.dy = torch.empty(m, hid, **act)
        self.dh = torch.empty(m, ffn, **act)
        self.dz = torch.empty(m, ffn, **act) if keep_dz else None
        self.dy1 = torch.empty(m, hid, **act)
        self.dctx = torch.empty(m, hid, **act)
        self.dqkv = torch.empty(m, 3 * hid, **act)
        self.heads, self.batch = heads, batch
        if heads is not None:
            seq = m // batch
            # one workspace serves the forward (V^T) and the backward (row sums): the larger figure
            wsb = max(attention_workspace_bytes(batch, seq, heads, hid // heads, backward=bw) for bw in (False, True))
            if wsb < 0:
                raise ValueError(f"attention core: unsupported shape batch={batch} seq={seq} heads={heads} "
                                 f"head width {hid // heads}")
            self.ctx = torch.empty(m, hid, **act)
            self.lse = torch.empty(batch, heads, seq, dtype=torch.float32, device=dev)
            self.attn_ws = torch.empty(wsb, dtype=torch.uint8, device=dev)     # holds the forward's too
        self.dx = torch.empty(m, hid, **act)
        # gradient-code workspaces: one pair reused by the four backward calls in
        # turn, or (keep_codes, for inspection) one pair per linear
        u8 = dict(dtype=torch.uint8, device=dev)
        cols = {"fc2": hid, "fc1": ffn, "o": hid, "qkv": 3 * hid}
        if keep_codes:
            self.gws = {k: (torch.empty(m, c, **u8), torch.empty(c, m, **u8)) for k, c in cols.items()}
        else:
            wide = max(cols.values())
            gq, gqt = torch.empty(m * wide, **u8), torch.empty(m * wide, **u8)
            self.gws = {k: (gq[:m * c].view(m, c), gqt[:m * c].view(c, m)) for k, c in cols.items()}
        self.saved = {"qkv": Saved(m, 3 * hid, hid, device=dev), "o": Saved(m, hid, hid, device=dev),
                      "fc1": Saved(m, ffn, hid, device=dev), "fc2": Saved(m, hid, ffn, device=dev)}
        self.bank = MetaBank([E5M2 if t.startswith("g_") else E4M3 for t in LAYER_TENSORS], history_len, device=dev)
        self.meta = {name: self.bank.meta(i) for i, name in enumerate(LAYER_TENSORS)}
        self.recipe = Recipe(FORMAT_HYBRID, history_len, AMAX_MAX, 0, fast_accum)
        self.ls_state = torch.tensor([loss_scale, 0.0, 0.0, loss_scale], dtype=torch.float32, device=dev)
        g0 = LAYER_TENSORS.index(LAYER_GRADS[0])
        assert LAYER_TENSORS[g0:g0 + len(LAYER_GRADS)] == LAYER_GRADS
        self._grad_amaxes = self.bank.amax_history[g0:, 0]          # n=4 slots, history_len floats apart

    def forward(self, x=None):
        x = self.x if x is None else x
        r, mt, sv = self.recipe, self.meta, self.saved
        # W is passed as None where the last update already cast it (delayed scaling)
        pre = self._w_cast and not r.just_in_time
        w = {n: (None if pre else t) for n, t in self.w.items()}
        fp8_linear_fwd(x, w["wqkv"], self.qkv, r, mt["x"], mt["wqkv"], sv["qkv"])
        if self.heads is not None:
            bf16_attention_fwd(self.qkv, self.batch, self.heads, self.ctx, self.lse, self.attn_ws)
        if self.fuse_casts and not r.just_in_time:
            # Y1 and H leave their GEMMs already cast to E4M3 for the next linear
            y1q = QOut(mt["y1"].scale, sv["fc1"].xq, sv["fc1"].xq_t, E4M3)
            fp8_linear_fwd(self.ctx, w["wo"], self.y1, r, mt["ctx"], mt["wo"], sv["o"], residual=x, y_q=y1q,
                           y_amax_slot=mt["y1"].amax_history[0:1])
            hq = QOut(mt["h"].scale, sv["fc2"].xq, sv["fc2"].xq_t, E4M3)
            fp8_linear_fwd(None, w["w1"], self.h, r, mt["y1"], mt["w1"], sv["fc1"], epilogue=EPI_GELU, y_aux=self.z,
                           y_q=hq, y_amax_slot=mt["h"].amax_history[0:1])
            fp8_linear_fwd(None, w["w2"], self.y, r, mt["h"], mt["w2"], sv["fc2"], residual=self.y1)
        else:
            fp8_linear_fwd(self.ctx, w["wo"], self.y1, r, mt["ctx"], mt["wo"], sv["o"], residual=x)
            fp8_linear_fwd(self.y1, w["w1"], self.h, r, mt["y1"], mt["w1"], sv["fc1"], epilogue=EPI_GELU,
                           y_aux=self.z)
            fp8_linear_fwd(self.h, w["w2"], self.y, r, mt["h"], mt["w2"], sv["fc2"], residual=self.y1)

    def backward(self):
        r, mt, sv, dw = self.recipe, self.meta, self.saved, self.dw
        hid, ffn = self.hidden, self.ffn
        fp8_loss_scale_apply(self.g, self.ls_state, self.dy)
        ws = self.gws
        fp8_linear_bwd(self.dy, ffn, r, mt["g_fc2"], sv["fc2"], *ws["fc2"], dx=self.dh, dw=dw["w2"])
        fp8_linear_bwd(self.dh, hid, r, mt["g_fc1"], sv["fc1"], *ws["fc1"], dx=self.dy1, dw=dw["w1"],
                       gelu_z=self.z, dz_out=self.dz, dx_residual=self.dy)
        fp8_linear_bwd(self.dy1, hid, r, mt["g_o"], sv["o"], *ws["o"], dx=self.dctx, dw=dw["wo"])
        if self.heads is not None:
            bf16_attention_bwd(self.qkv, self.ctx, self.lse, self.dctx, self.batch, self.heads, self.dqkv,
                               self.attn_ws)
        else:
            fp8_loss_scale_apply(self.dqkv_in, self.ls_state, self.dqkv)
        fp8_linear_bwd(self.dqkv, hid, r, mt["g_qkv"], sv["qkv"], *ws["qkv"], dx=self.dx, dw=dw["wqkv"],
                       dx_residual=self.dy1)

    def update(self):
        fp8_loss_scale_update(self._grad_amaxes, self.ls_state, stride=self.bank.history_len, n=len(LAYER_GRADS),
                              growth_interval=self.growth_interval)
        self.bank.update(self.recipe)
        if self.fuse_sgd_cast and not self.recipe.just_in_time:
            mt, sv = self.meta, self.saved
            for name, lin in zip(LAYER_WEIGHTS, ("qkv", "o", "fc1", "fc2")):
                fp8_sgd_step_cast(self.w[name], self.dw[name], self.lr, self.ls_state, mt[name].scale, sv[lin].wq,
                                  sv[lin].wq_t, mt[name].amax_history[0:1])
            self._w_cast = True
        else:
            fp8_sgd_step(self.master, self.grad, self.lr, self.ls_state)
            self._w_cast = False

    def step(self, x=None, record=None):
        """One step; with a list as `record`, appends the step's per-tensor
        amax, scales and (when counting) saturated codes, taken before the
        update (see metrics())."""
        self.forward(x)
        self.backward()
        if record is not None:
            record.append(self.metrics())
        self.update()

    def count_saturation(self, enable=True):
        """Opt-in saturated-code counters for the layer's twelve tensors."""
        self.bank.count_saturation(enable)

    def metrics(self, clear=True):
        """Host snapshot per tensor name: amax slot 0 (between backward and
        update: the step's amax), scale and inverse scale (the ones the step's
        casts used), the loss scale S, and (when counting) saturated codes
        since the last snapshot."""
        m = self.bank.snapshot(LAYER_TENSORS, clear)
        m["loss_scale"] = self.ls_state[0].item()
        return m

    def state_dict(self):
        """Everything a training run carries from step to step: the fp32
        masters, the delayed-scaling metas of the twelve tensors and the
        loss-scale state (host copies; plain tensors, so torch.save /
        torch.load(weights_only=True) round-trip them)."""
        return {"master": self.master.cpu().clone(), "bank": self.bank.state_dict(),
                "ls_state": self.ls_state.cpu().clone()}

    def load_state_dict(self, state):
        """Restores a state_dict in place; the next step continues exactly as
        the saved run would have."""
        if state["master"].shape != self.master.shape:
            raise ValueError("Fp8TransformerLayer.load_state_dict: master size differs")
        self.master.copy_(state["master"])
        self.bank.load_state_dict(state["bank"])
        self.ls_state.copy_(state["ls_state"])
        self._w_cast = False        # the next forward casts W from the restored masters

    def flops_per_step(self):
        """Algorithmic flops of one step: the twelve FP8 GEMMs (2 m n k each)
        and, with the attention core, its forward products Q K^T and P V and
        backward products dP, dV, dQ, dK (2 S^2 D each per sequence and head;
        the backward's recomputation of S is not counted)."""
        m, hid, ffn = self.m, self.hidden, self.ffn
        linears = 6 * m * (3 * hid * hid + hid * hid + 2 * ffn * hid)
        if self.heads is None:
            return linears
        seq = m // self.batch
        return linears + 12 * self.batch * self.heads * seq * seq * (hid // self.heads)

    def attention_flops(self):
        if self.heads is None:
            return 0
        seq = self.m // self.batch
        return 12 * self.batch * self.heads * seq * seq * (self.hidden // self.heads)
