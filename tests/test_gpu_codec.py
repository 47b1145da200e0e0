"""GPU parity: the FP8 cast and decode against the oracle, bit for bit.

Includes the exhaustive check of all 2^32 fp32 bit patterns at scale 1 for
both formats, every bf16 pattern at several scales, and ragged lengths.
"""
import numpy as np
import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
from helpers import assert_bits_equal, dev, np_of

pytestmark = pytest.mark.gpu
FMTS = [(F.E4M3, 0), (F.E5M2, 1)]


def _scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("lf,of", FMTS, ids=["e4m3", "e5m2"])
def test_cast_every_fp32_bit_pattern(oracle, lf, of):
    one = _scalar(1.0)
    chunk = 1 << 28
    q = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    for start in range(0, 1 << 32, chunk):
        s = start if start < (1 << 31) else start - (1 << 32)
        x = torch.arange(s, s + chunk, dtype=torch.int32, device="cuda").view(torch.float32)
        F.fp8_cast(x, lf, one, q)
        got = q.cpu().numpy()
        want = oracle.encode_bits_range(start, chunk, of)
        assert_bits_equal(got, want, f"fp32 patterns [{start:#x}, +2^28)")
        del x


@pytest.mark.parametrize("lf,of", FMTS, ids=["e4m3", "e5m2"])
def test_cast_every_bf16_pattern_at_several_scales(oracle, lf, of):
    bits = np.arange(1 << 16, dtype=np.uint16)
    x = dev(bits)
    q = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    for s in (1.0, 3.3, 2.0 ** -20, 1.0 / 3.0, 448.0 / 7.5, 57344.0, 1.5e-38, 3.0e38):
        F.fp8_cast(x, lf, _scalar(s), q)
        assert_bits_equal(np_of(q), oracle.cast(bits, of, np.float32(s)), f"bf16 patterns x {s}")


@pytest.mark.parametrize("lf,of", FMTS, ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 4096 + 3, 1000003])
def test_cast_random_scaled_and_ragged(oracle, lf, of, n):
    rng = np.random.default_rng(n + 17 * lf)
    x = (rng.standard_normal(n) * np.exp2(rng.uniform(-30, 30, n))).astype(np.float32)
    if n > 8:
        x[:8] = [np.nan, -np.inf, np.inf, -0.0, 0.0, 1e-45, -3e-44, 3.4e38]
    for s in (np.float32(1.0), np.float32(0.37), np.float32(2.0 ** 17 / 3)):
        q = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")[:n]
        slot = torch.zeros(1, dtype=torch.float32, device="cuda")
        F.fp8_cast(dev(x), lf, _scalar(float(s)), q, slot)
        assert_bits_equal(np_of(q), oracle.cast(x, of, s), f"n={n} s={s}")
        assert_bits_equal(np_of(slot)[0], oracle.amax(x), "fused amax")


@pytest.mark.parametrize("lf,of", FMTS, ids=["e4m3", "e5m2"])
def test_decode_every_code(oracle, lf, of):
    codes = np.arange(256, dtype=np.uint8)
    for sinv in (1.0, 0.125, 3.7e-5, 1.0 / 3.0):
        out = torch.empty(256, dtype=torch.float32, device="cuda")
        F.fp8_dequant(dev(codes), lf, _scalar(sinv), out)
        assert_bits_equal(np_of(out), oracle.dequant(codes, of, np.float32(sinv), 0), f"f32 sinv={sinv}")
        outb = torch.empty(256, dtype=torch.bfloat16, device="cuda")
        F.fp8_dequant(dev(codes), lf, _scalar(sinv), outb)
        want = oracle.dequant(codes, of, np.float32(sinv), 1)
        got = np_of(outb)
        nan = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
        assert_bits_equal(got[~nan], want[~nan], f"bf16 sinv={sinv}")
        assert np.all(((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0))


@pytest.mark.parametrize("lf,of", FMTS, ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("n", [0, 5, 16, 4099, 1 << 20])
def test_dequant_ragged(oracle, lf, of, n):
    rng = np.random.default_rng(n)
    codes = rng.integers(0, 256, n, dtype=np.uint8)
    out = torch.empty(max(n, 1), dtype=torch.float32, device="cuda")[:n]
    F.fp8_dequant(dev(codes), lf, _scalar(0.75), out)
    assert_bits_equal(np_of(out), oracle.dequant(codes, of, np.float32(0.75), 0), f"n={n}")
