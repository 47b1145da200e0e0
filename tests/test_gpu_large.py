"""GPU parity past 2^31 elements: the 64-bit indexing of the amax, cast,
cast-transpose and dequant kernels; and the cast-transpose at the largest
dimensions its entry points admit (its tiles use 32-bit offsets).

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
import synth
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


def test_cast_transpose_largest_admitted_dims(oracle):
    """The cast-transpose kernels address a tile with 32-bit offsets; the
    entry points admit cols < 2^22 and rows < 2^24.  At the largest admitted
    width (16 x (2^22 - 16), fp32) and height ((2^24 - 16) x 16, bf16, the
    dual-format kernel) every code, both layouts, and the amax equal the
    oracle's."""
    u8 = dict(dtype=torch.uint8, device="cuda")
    # widest: fp32, one row of tiles, the last tile ragged (2^22 - 16 = 32767 * 128 + 112)
    rows, cols = 16, (1 << 22) - 16
    x = synth.normal((rows, cols), 3.0, synth.seed_of(7, 0, 0), device="cuda")
    x[rows - 1, cols - 1] = -500.0                       # the maximum, in the last (ragged) tile
    s = np.float32(448.0 / 4.0)
    q, qt = torch.empty(rows, cols, **u8), torch.empty(cols, rows, **u8)
    slot = torch.zeros(1, device="cuda")
    F.fp8_cast_transpose(x, F.E4M3, _scalar(float(s)), q, qt, slot)
    torch.cuda.synchronize()
    xh = np_of(x)
    want_q, want_qt = oracle.cast_transpose(xh, 0, s)
    assert_bits_equal(np_of(q), want_q, "q, widest")
    assert_bits_equal(np_of(qt), want_qt, "q_t, widest")
    assert_bits_equal(np_of(slot)[0], np.float32(500.0), "amax, widest")
    del x, q, qt, xh, want_q, want_qt
    # tallest: bf16, one column of tiles, dual format (both layouts of both formats)
    rows, cols = (1 << 24) - 16, 16
    x = synth.normal((rows, cols), 1.0, synth.seed_of(7, 0, 1), torch.bfloat16, "cuda")
    x[rows - 1, 0] = 200.0
    s4, s5 = np.float32(448.0 / 8.0), np.float32(57344.0 / 8.0)
    outs = [torch.empty(rows, cols, **u8), torch.empty(cols, rows, **u8), torch.empty(rows, cols, **u8),
            torch.empty(cols, rows, **u8)]
    slots = torch.zeros(2, device="cuda")
    F.fp8_cast_transpose_dual(x, _scalar(float(s4)), _scalar(float(s5)), *outs, slots[0:1], slots[1:2])
    torch.cuda.synchronize()
    xh = np_of(x)
    for k, (fmt, sc) in enumerate(((0, s4), (1, s5))):
        want_q, want_qt = oracle.cast_transpose(xh, fmt, sc)
        assert_bits_equal(np_of(outs[2 * k]), want_q, f"q, tallest, format {fmt}")
        assert_bits_equal(np_of(outs[2 * k + 1]), want_qt, f"q_t, tallest, format {fmt}")
    assert_bits_equal(np_of(slots), np.array([200.0, 200.0], dtype=np.float32), "amax, tallest")
