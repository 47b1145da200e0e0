"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds only input recipes -- shapes, value distributions and seeds --
and none of the FP8 method's arithmetic.  Random values come from splitmix64
used as a counter generator (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", 2014): draw i of a seed is the splitmix64
output of state seed + (i + 1) * 0x9E3779B97F4A7C15, computed with 64-bit
integer operations that give the same integers on the CPU and the GPU and in
any torch version.  A uniform value takes the top 24 bits (k / 2^24, exact in
fp32); a normal value takes two draws, 53 bits each, through the Box-Muller
transform in fp64 (sqrt(-2 ln u1) cos(2 pi u2), u1 in (0, 1]), is scaled in
fp64 and rounded to fp32, then to the element type (a last-bit difference
between two libraries' fp64 log or cos changes a value only where it straddles
an fp32 rounding boundary).  Small tensors are drawn on the CPU, large ones on
the GPU.  Both the HIP path and the oracle consume the
same tensors (the oracle after a copy to the host).

Seed of a tensor: 12345 + 1000 * config + 10 * iteration + tensor_id (12345 is
the seed of the pages' Linear(768, 768) example).

Workloads:
  linear768  X f32 1024x768 ~ U[0,1), W f32 768x768 and b f32 768 ~ U(-1/sqrt(768), 1/sqrt(768)),
             dY f32 1024x768 ~ N(0,1) * 2^-20 (fresh X and dY each iteration)
  mlp        tokens 8192, hidden 4096, FFN 14336; X bf16 N(0,1) with round(0.001*4096) = 4
             outlier channels scaled x50 (chosen by a seeded permutation); W1 bf16 14336x4096 and
             W2 bf16 4096x14336 ~ N(0, 0.02); dY bf16 8192x4096 ~ N(0,1)
  quant      bf16 16384x16384; row r has magnitude 2^u_r, u_r ~ U[-20, 10], times N(0,1) values
  layer      tokens 8192 (seq 4096 x batch 2), hidden 8192, FFN 28672; X bf16 N(0,1); fp32 master
             weights ~ N(0, 0.02): Wqkv 24576x8192, Wo 8192x8192, W1 28672x8192, W2 8192x28672;
             upstream gradient G bf16 ~ N(0,1) * 2^-20 (the loss is <Y, G> * S); 64 attention
             heads of width 128; the spiked input of iteration 10 is bf16(fl32(X) * 100).  For
             the layer run without its attention core: stand-ins ctx bf16 8192x8192 ~ N(0,1) and
             d(QKV) bf16 8192x24576 ~ N(0,1) * 2^-20
  attention  the bf16 attention core of the layer (64 heads of width 128 over seq 4096 x batch 2):
             its input qkv bf16 [batch*seq][3*heads*128] ~ N(0, std^2) and an incoming gradient
             dctx bf16 [batch*seq][heads*128] ~ N(0,1) (smaller shapes for the parity cases)
"""
import math

import torch

SEED0 = 12345


def seed_of(config, iteration, tensor_id):
    return SEED0 + 1000 * config + 10 * iteration + tensor_id


def _s64(v):
    """A 64-bit pattern as the signed int64 torch stores."""
    v &= (1 << 64) - 1
    return v - (1 << 64) if v >> 63 else v


_GAMMA, _M1, _M2 = _s64(0x9E3779B97F4A7C15), _s64(0xBF58476D1CE4E5B9), _s64(0x94D049BB133111EB)


def _srl(z, s):
    """Logical right shift of int64 patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def splitmix64(seed, n, device="cpu"):
    """Draws 0 .. n-1 of the seed as int64 bit patterns (multiplication wraps
    mod 2^64, as the generator's definition requires)."""
    z = torch.arange(1, n + 1, dtype=torch.int64, device=device) * _GAMMA + _s64(seed)
    z = (z ^ _srl(z, 30)) * _M1
    z = (z ^ _srl(z, 27)) * _M2
    return z ^ _srl(z, 31)


def _numel(shape):
    return math.prod(shape) if isinstance(shape, (tuple, list)) else int(shape)


def uniform(shape, lo, hi, seed, dtype=torch.float32, device="cpu"):
    u = _srl(splitmix64(seed, _numel(shape), device), 40).to(torch.float32) * 2.0 ** -24
    return (u * (hi - lo) + lo).reshape(shape).to(dtype)


def normal(shape, std, seed, dtype=torch.float32, device="cpu"):
    n = _numel(shape)
    z = splitmix64(seed, 2 * n, device).view(n, 2)
    u1 = (_srl(z[:, 0], 11).to(torch.float64) + 1.0) * 2.0 ** -53
    u2 = _srl(z[:, 1], 11).to(torch.float64) * 2.0 ** -53
    del z
    x = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
    del u1, u2
    return (x * std).to(torch.float32).reshape(shape).to(dtype)


def permutation(n, seed):
    """A seeded permutation of 0 .. n-1: the indices ordered by their draws."""
    return torch.argsort(splitmix64(seed, n), stable=True)


# ------------------------------------------------------------ linear768 ----

LINEAR768 = dict(m=1024, n=768, k=768, history_len=16)


def linear768_weights(device="cpu", m=1024, n=768, k=768):
    a = 1.0 / math.sqrt(k)
    w = uniform((n, k), -a, a, seed_of(1, 0, 1), device=device)
    b = uniform((n,), -a, a, seed_of(1, 0, 2), device=device)
    return w, b


def linear768_x(iteration, device="cpu", m=1024, k=768):
    return uniform((m, k), 0.0, 1.0, seed_of(2, iteration, 0), device=device)


def linear768_dy(iteration, device="cpu", m=1024, n=768):
    return normal((m, n), 2.0 ** -20, seed_of(2, iteration, 3), device=device)


# ------------------------------------------------------------------ mlp ----

MLP = dict(m=8192, hidden=4096, ffn=14336, history_len=1024)


def mlp_inputs(iteration=0, device="cpu", m=8192, hidden=4096, ffn=14336):
    """X (with outlier channels), W1, W2 and the upstream gradient dY, all bf16."""
    x = normal((m, hidden), 1.0, seed_of(3, iteration, 0), device=device)
    n_out = round(0.001 * hidden)
    cols = permutation(hidden, seed_of(3, 0, 9))[:n_out].to(device)
    x[:, cols] *= 50.0
    x = x.to(torch.bfloat16)
    w1 = normal((ffn, hidden), 0.02, seed_of(3, 0, 1), torch.bfloat16, device)
    w2 = normal((hidden, ffn), 0.02, seed_of(3, 0, 2), torch.bfloat16, device)
    dy = normal((m, hidden), 1.0, seed_of(3, iteration, 3), torch.bfloat16, device)
    return x, w1, w2, dy


def mlp_outlier_channels(hidden=4096):
    n_out = round(0.001 * hidden)
    return permutation(hidden, seed_of(3, 0, 9))[:n_out]


# ---------------------------------------------------------------- quant ----

QUANT = dict(rows=16384, cols=16384, history_len=1024)


def quant_tensor(device="cpu", rows=16384, cols=16384):
    u = uniform((rows, 1), -20.0, 10.0, seed_of(4, 0, 1), device=device)
    x = normal((rows, cols), 1.0, seed_of(4, 0, 0), device=device)
    return (x * torch.exp2(u)).to(torch.bfloat16)


# ---------------------------------------------------------------- layer ----

LAYER = dict(m=8192, hidden=8192, ffn=28672, history_len=1024, iterations=20, spike_iteration=10,
             spike_factor=100.0, heads=64, batch=2)


def layer_inputs(device="cpu", m=8192, hidden=8192, ffn=28672):
    """dict of X, ctx, G, dqkv (bf16) and the fp32 masters wqkv, wo, w1, w2.

    The same X, G and stand-ins are used at every iteration; only the master
    weights (updated by SGD) and the scales change from step to step."""
    bf = torch.bfloat16
    return dict(
        x=normal((m, hidden), 1.0, seed_of(5, 0, 0), bf, device),
        wqkv=normal((3 * hidden, hidden), 0.02, seed_of(5, 0, 1), device=device),
        wo=normal((hidden, hidden), 0.02, seed_of(5, 0, 2), device=device),
        w1=normal((ffn, hidden), 0.02, seed_of(5, 0, 3), device=device),
        w2=normal((hidden, ffn), 0.02, seed_of(5, 0, 4), device=device),
        g=normal((m, hidden), 2.0 ** -20, seed_of(5, 0, 5), bf, device),
        ctx=normal((m, hidden), 1.0, seed_of(5, 0, 6), bf, device),
        dqkv=normal((m, 3 * hidden), 2.0 ** -20, seed_of(5, 0, 7), bf, device),
    )


def layer_spike(x, factor=100.0):
    """The spiked layer input: bf16(fl32(x) * factor)."""
    return (x.float() * factor).to(torch.bfloat16)


def attention_inputs(batch, seq, heads, std=1.0, seed=None, device="cpu", head_dim=128):
    """qkv [batch*seq][3*heads*head_dim] bf16 ~ N(0, std^2) and dctx
    [batch*seq][heads*head_dim] bf16 ~ N(0,1)."""
    seed = seed_of(5, 0, 20) if seed is None else seed
    m, hd = batch * seq, heads * head_dim
    qkv = normal((m, 3 * hd), std, seed, dtype=torch.bfloat16, device=device)
    dctx = normal((m, hd), 1.0, seed + 1, dtype=torch.bfloat16, device=device)
    return qkv, dctx
