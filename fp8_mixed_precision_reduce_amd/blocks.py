"""Layer compositions over the C entry points (argument marshalling only).

Fp8MlpBlock: the FC1 -> GeLU -> FC2 block of a transformer layer with FP8
linears and per-tensor delayed scaling ([TE-KR] "Using FP8 with Transformer
Engine": Linear layers under an FP8 autocast with a DelayedScaling recipe;
HYBRID formats).  One step() is the forward pass, the backward pass and the
per-step history/scale update of all six FP8 tensors (X, W1, H, W2, dY, dZ),
every part of it in the library's kernels:

  fp8_linear_fwd(X, W1, GELU)  -> H = gelu(Z) (bf16), Z kept for backward
  fp8_linear_fwd(H, W2)        -> Y (bf16)
  fp8_linear_bwd(dY; W2)       -> dH (bf16), dW2 (fp32)
  fp8_linear_bwd(dH; W1, Z)    -> GeLU backward fused into the dZ cast, dX (bf16), dW1 (fp32)
  fp8_amax_scale_update(6 tensors)

Page tags: [TE-KR] "Transformer Engine으로 FP8 사용하기" (coniverse.tistory.com).
"""
import torch

from . import (AMAX_MAX, E4M3, E5M2, EPI_GELU, FORMAT_HYBRID, MetaBank, Recipe, Saved, fp8_linear_bwd,
               fp8_linear_fwd)

MLP_TENSORS = ("x", "w1", "h", "w2", "dy", "dz")


class Fp8MlpBlock:
    """Buffers, metas and one training step of the FP8 MLP block.

    x [m][hidden], w1 [ffn][hidden], w2 [hidden][ffn], dy [m][hidden]: bf16 (or
    fp32) device tensors owned by the caller.  keep_dz=True also writes the
    rounded GeLU-backward gradient dZ (for inspection)."""

    def __init__(self, x, w1, w2, dy, history_len=1024, fast_accum=False, keep_dz=False):
        m, hidden = x.shape
        ffn = w1.shape[0]
        assert w1.shape == (ffn, hidden) and w2.shape == (hidden, ffn) and dy.shape == (m, hidden)
        dev = x.device
        self.m, self.hidden, self.ffn = m, hidden, ffn
        self.x, self.w1, self.w2, self.dy = x, w1, w2, dy
        act = dict(dtype=x.dtype, device=dev)
        self.h = torch.empty(m, ffn, **act)
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
        fp8_linear_fwd(self.x, self.w1, self.h, r, mt["x"], mt["w1"], self.saved1, epilogue=EPI_GELU, y_aux=self.z)
        fp8_linear_fwd(self.h, self.w2, self.y, r, mt["h"], mt["w2"], self.saved2)

    def backward(self):
        r, mt = self.recipe, self.meta
        fp8_linear_bwd(self.dy, self.ffn, r, mt["dy"], self.saved2, self.dyq, self.dyq_t, dx=self.dh, dw=self.dw2)
        fp8_linear_bwd(self.dh, self.hidden, r, mt["dz"], self.saved1, self.dzq, self.dzq_t, dx=self.dx,
                       dw=self.dw1, gelu_z=self.z, dz_out=self.dz)

    def update(self):
        self.bank.update(self.recipe)

    def step(self):
        self.forward()
        self.backward()
        self.update()
