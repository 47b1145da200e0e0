"""GPU: the opt-in saturated-code counters (fp8lin_count_saturation).

Every cast entry point that takes an amax slot adds, for a registered slot,
the number of elements whose fp32 product with the scale exceeds the format's
largest finite magnitude; the counts are compared with the oracle's count over
the same inputs and scales.  Inputs carry planted boundary values (a product of
exactly the maximum, one step above it, +-Inf, NaN) and a ragged tail, so the
vector, tail and transposed paths all count.  Registrations are removed before
their buffers are freed (a stale one would add into reused memory)."""
import contextlib

import numpy as np
import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
from helpers import dev, np_of

pytestmark = pytest.mark.gpu
FMTS = [(F.E4M3, 0, 448.0), (F.E5M2, 1, 57344.0)]
SCALE = np.float32(128.0)           # a power of two: the planted products are exact


def _scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


@contextlib.contextmanager
def _counting(*slots):
    """Registers one fresh int32 counter per slot; yields the counters."""
    ctrs = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in slots]
    try:
        for s, c in zip(slots, ctrs):
            F.count_saturation(s, c)
        yield ctrs
    finally:
        for s in slots:
            F.count_saturation(s, None)


def _values(oracle, rng, n, mx, dtype):
    """n values around the saturation threshold mx / SCALE, with planted
    boundary values at random places (as bf16 bits or fp32)."""
    t = np.float32(mx) / SCALE
    x = (rng.standard_normal(n) * t * 0.8).astype(np.float32)
    step = np.float32(2.0 ** (np.floor(np.log2(t)) - 7))          # one bf16 step at t
    plants = np.array([t, -t, t + step, -(t + step), np.inf, -np.inf, np.nan, 0.0], dtype=np.float32)
    idx = rng.choice(n, size=min(n, 4 * plants.size), replace=False)
    x[idx] = np.resize(plants, idx.size)
    return oracle.bf16_from_f32(x) if dtype == "bf16" else x


@pytest.mark.parametrize("lf,of,mx", FMTS, ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [100003, 64])
def test_cast_counts(oracle, lf, of, mx, dtype, n):
    rng = np.random.default_rng(n + 7 * of + (dtype == "bf16"))
    x = _values(oracle, rng, n, mx, dtype)
    want = oracle.count_saturated(x, of, SCALE)
    assert n < 100 or want > 100
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    slot, other = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    with _counting(slot) as (c,):
        F.fp8_cast(dev(x), lf, _scalar(float(SCALE)), q, slot)
        F.fp8_cast(dev(x), lf, _scalar(float(SCALE)), q, other)      # another slot: not counted
        F.fp8_cast(dev(x), lf, _scalar(float(SCALE)), q, None)
        torch.cuda.synchronize()
        assert int(c.item()) == want
        F.fp8_cast(dev(x), lf, _scalar(float(SCALE)), q, slot)      # counts accumulate
        torch.cuda.synchronize()
        assert int(c.item()) == 2 * want
    F.fp8_cast(dev(x), lf, _scalar(float(SCALE)), q, slot)          # unregistered: untouched
    torch.cuda.synchronize()
    assert int(c.item()) == 2 * want


@pytest.mark.parametrize("lf,of,mx", FMTS, ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dbias", [False, True], ids=["plain", "dbias"])
def test_cast_transpose_counts(oracle, lf, of, mx, dtype, dbias):
    rows, cols = 272, 400
    rng = np.random.default_rng(rows + of + 2 * dbias)
    x = _values(oracle, rng, rows * cols, mx, dtype).reshape(rows, cols)
    want = oracle.count_saturated(x, of, SCALE)
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    qt = torch.empty(cols, rows, dtype=torch.uint8, device="cuda")
    db = torch.empty(cols, device="cuda") if dbias else None
    ws = torch.empty(F.dbias_workspace_bytes(rows, cols) // 4, device="cuda") if dbias else None
    slot = torch.zeros(1, device="cuda")
    with _counting(slot) as (c,):
        F.fp8_cast_transpose(dev(x), lf, _scalar(float(SCALE)), q, qt, slot, db, ws)
        torch.cuda.synchronize()
        assert int(c.item()) == want
        if dbias:
            c.zero_()
            F.fp8_cast_transpose_dbias_noalloc(dev(x), lf, _scalar(float(SCALE)), q, qt, db, slot)
            torch.cuda.synchronize()
            assert int(c.item()) == want


def test_cast_transpose_dgelu_counts(oracle):
    """The GeLU-backward cast counts over dZ = round(dH * gelu'(Z)); the
    kernel's dZ may differ from the oracle's by one bf16 step, so the count is
    bracketed by the oracle's counts with dZ moved one step toward and away
    from zero."""
    rows, cols = 272, 400
    rng = np.random.default_rng(5)
    dh = oracle.bf16_from_f32((rng.standard_normal((rows, cols)) * 6.0).astype(np.float32))
    z = oracle.bf16_from_f32((rng.standard_normal((rows, cols)) * 2.0).astype(np.float32))
    dz = oracle.gelu_bwd(dh, z)                    # bf16 bits
    s = np.float32(448.0 / 5.0)
    mag = dz & 0x7FFF
    down = np.where(mag > 0, dz - 1, dz).astype(np.uint16)                    # one step toward zero
    up = np.where(mag < 0x7F80, dz + 1, dz).astype(np.uint16)                 # one step away from zero
    lo, hi = oracle.count_saturated(down, 0, s), oracle.count_saturated(up, 0, s)
    assert lo > 100
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    qt = torch.empty(cols, rows, dtype=torch.uint8, device="cuda")
    slot = torch.zeros(1, device="cuda")
    with _counting(slot) as (c,):
        F.fp8_cast_transpose_dgelu(dev(dh), dev(z), F.E4M3, _scalar(float(s)), q, qt, slot)
        torch.cuda.synchronize()
        got = int(c.item())
    assert lo <= got <= hi, (lo, got, hi)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dual_cast_counts(oracle, dtype):
    """Both formats of the dual cast, each into its own slot's counter, with
    the plain launch and with the scale update fused (two metas in a bank)."""
    rows, cols = 272, 400
    rng = np.random.default_rng(11)
    x = _values(oracle, rng, rows * cols, 448.0, dtype).reshape(rows, cols)
    s4, s5 = SCALE, np.float32(0.5)                # E5M2 saturates above 114688 before the scale
    x[::7, ::5] = (oracle.bf16_from_f32(np.float32(2.0e5)) if dtype == "bf16" else np.float32(2.0e5))
    want4, want5 = oracle.count_saturated(x, 0, s4), oracle.count_saturated(x, 1, s5)
    assert want4 > 100 and want5 > 100
    u8 = dict(dtype=torch.uint8, device="cuda")
    outs = [torch.empty(rows, cols, **u8), torch.empty(cols, rows, **u8), torch.empty(rows, cols, **u8),
            torch.empty(cols, rows, **u8)]
    slots = torch.zeros(2, device="cuda")
    with _counting(slots[0:1], slots[1:2]) as (c4, c5):
        F.fp8_cast_transpose_dual(dev(x), _scalar(float(s4)), _scalar(float(s5)), *outs, slots[0:1], slots[1:2])
        torch.cuda.synchronize()
        assert (int(c4.item()), int(c5.item())) == (want4, want5)
    L = 16
    bank = F.MetaBank([F.E4M3, F.E5M2], L)
    bank.scale.copy_(torch.tensor([float(s4), float(s5)], device="cuda"))
    recipe = F.Recipe(F.FORMAT_HYBRID, L, F.AMAX_MAX, 0)
    ticket = torch.zeros(1, dtype=torch.int32, device="cuda")
    with _counting(bank.amax_history[0], bank.amax_history[1]) as (c4, c5):
        F.fp8_cast_transpose_dual_update(dev(x), bank, recipe, ticket, *outs)
        torch.cuda.synchronize()
        assert (int(c4.item()), int(c5.item())) == (want4, want5)
    assert int(ticket.item()) == 0


def test_metabank_counters_and_snapshot(oracle):
    """MetaBank.count_saturation registers one counter per tensor; snapshot()
    reads amax slot 0, the scales and the counts, and clears the counts."""
    bank = F.MetaBank([F.E4M3, F.E5M2], 8)
    bank.scale.fill_(float(SCALE))
    x = _values(oracle, np.random.default_rng(3), 4096, 448.0, "f32")
    x[np.isnan(x)] = 0.0               # (a NaN would be the amax: the statistic compares bit patterns)
    bank.count_saturation()
    try:
        for i, fmt in enumerate((F.E4M3, F.E5M2)):
            q = torch.empty(4096, dtype=torch.uint8, device="cuda")
            F.fp8_cast(dev(x), fmt, bank.scale[i:i + 1], q, bank.amax_history[i])
        snap = bank.snapshot(["a", "b"])
        assert snap["a"]["saturated"] == oracle.count_saturated(x, 0, SCALE) > 100
        assert snap["b"]["saturated"] == oracle.count_saturated(x, 1, SCALE)
        assert snap["a"]["amax"] == snap["b"]["amax"] == float(oracle.amax(x))
        assert snap["a"]["scale"] == float(SCALE) and snap["b"]["scale_inv"] == 1.0
        assert all(v["saturated"] == 0 for v in bank.snapshot(["a", "b"]).values())      # cleared
    finally:
        bank.count_saturation(False)
