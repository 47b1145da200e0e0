"""GPU parity past 2^31 elements: the 64-bit indexing of the amax, cast,
cast-transpose and dequant kernels.

The bf16 tensors (just over 2^31 elements, with a ragged tail) are drawn on the
GPU from a seeded generator.  The cast and the dequant are elementwise, so the
oracle checks a sample of elements exactly: random positions, the elements on
both sides of index 2^31 and the whole tail.  The amax is pinned by a planted
maximum (every other value is a standard normal draw, far below it) placed past
index 2^31.
"""
import numpy as np
import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
from helpers import assert_bits_equal, np_of

pytestmark = pytest.mark.gpu

BIG = 1 << 31


def _scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def _normal_bf16(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)


def test_amax_cast_dequant_past_2_31_elements(oracle):
    n = BIG + 4096 + 40                                  # not a multiple of the 8-element vectors
    x = _normal_bf16((n,), 31)
    x[BIG + 1234] = 300.0
    x[n - 1] = -320.0                                    # the maximum |x| sits in the scalar tail
    scale = np.float32(1.25)
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    slot = torch.zeros(1, dtype=torch.float32, device="cuda")
    F.fp8_cast(x, F.E4M3, _scalar(float(scale)), q, slot)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    F.fp8_amax(x, amax)
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    F.fp8_dequant(q, F.E4M3, _scalar(float(np.float32(1) / scale)), out)
    torch.cuda.synchronize()
    assert_bits_equal(np_of(slot)[0], np.float32(320.0), "amax fused into the cast")
    assert_bits_equal(np_of(amax)[0], np.float32(320.0), "standalone amax")

    rng = np.random.default_rng(31)
    idx = np.unique(np.concatenate([rng.integers(0, n, 8192), np.arange(BIG - 96, BIG + 96),
                                    np.arange(n - 200, n), [BIG + 1234]]))
    ti = torch.from_numpy(idx).cuda()
    xs, qs, outs = np_of(x[ti]), np_of(q[ti]), np_of(out[ti])
    assert_bits_equal(qs, oracle.cast(xs, 0, scale), "codes at sampled positions")
    assert_bits_equal(outs, oracle.dequant(qs, 0, np.float32(1) / scale, oracle.BF16), "dequant at sampled positions")


def test_cast_transpose_past_2_31_elements(oracle):
    rows, cols = (1 << 16) + 16, 1 << 15                 # 2^31 + 2^19 elements; 128-tile rows ragged
    x = _normal_bf16((rows, cols), 32)
    x[rows - 1, cols - 5] = 400.0
    scale = np.float32(256.0)                            # 400 * 256 saturates to the E5M2 maximum, 57344
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    qt = torch.empty(cols, rows, dtype=torch.uint8, device="cuda")
    slot = torch.zeros(1, dtype=torch.float32, device="cuda")
    F.fp8_cast_transpose(x, F.E5M2, _scalar(float(scale)), q, qt, slot)
    torch.cuda.synchronize()
    assert_bits_equal(np_of(slot)[0], np.float32(400.0), "amax")

    rng = np.random.default_rng(32)
    r = np.unique(np.concatenate([rng.integers(0, rows, 96), np.arange(rows - 16, rows), [0, 1 << 15, 1 << 16]]))
    c = np.unique(np.concatenate([rng.integers(0, cols, 96), np.arange(cols - 16, cols), [0]]))
    tr, tc = torch.from_numpy(r).cuda(), torch.from_numpy(c).cuda()
    xs = np_of(x.index_select(0, tr).index_select(1, tc))
    want = oracle.cast(xs, 1, scale)
    assert_bits_equal(np_of(q.index_select(0, tr).index_select(1, tc)), want, "row-major codes")
    assert_bits_equal(np_of(qt.index_select(0, tc).index_select(1, tr)), want.T, "transposed codes")
