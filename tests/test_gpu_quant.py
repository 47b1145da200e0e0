"""GPU parity of standalone quantisation at full size: a 2^28-element bf16
tensor (16384 x 16384, row magnitudes 2^u with u ~ U[-20, 10]) cast and
transposed to E4M3 and E5M2 with fused amax, dequantised back to bf16, and the
two metas (history 1024) updated between repetitions.  Every code, transposed
code, dequantised value, amax, history entry and scale is compared bit for bit
with the oracle over all 2^28 elements."""
import numpy as np
import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
import synth
from helpers import assert_bits_equal, dev, np_of

pytestmark = pytest.mark.gpu


def test_quant_tensor_full_size(oracle):
    rows = cols = 16384
    L = 1024
    x = synth.quant_tensor(device="cuda")
    X = np_of(x)
    bank = F.MetaBank([F.E4M3, F.E5M2], L)
    om = [oracle.Meta(L, 0), oracle.Meta(L, 1)]
    recipe = F.Recipe(F.FORMAT_HYBRID, L, F.AMAX_MAX, 0)
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    qt = torch.empty(cols, rows, dtype=torch.uint8, device="cuda")
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda")
    for rep in range(2):
        for i, (lf, of) in enumerate(((F.E4M3, 0), (F.E5M2, 1))):
            F.fp8_cast_transpose(x, lf, bank.scale[i:i + 1], q, qt, bank.amax_history[i, 0:1])
            F.fp8_dequant(q, lf, bank.scale_inv[i:i + 1], out)
            wq, wqt = oracle.cast_transpose(X, of, om[i].scale)
            tag = f"rep {rep} fmt {of}"
            assert_bits_equal(np_of(q), wq, tag + " q")
            assert_bits_equal(np_of(qt), wqt, tag + " q^T")
            assert_bits_equal(np_of(out), oracle.dequant(wq, of, om[i].scale_inv, 1), tag + " dequant")
            del wq, wqt
            om[i].record(X)
            assert_bits_equal(np_of(bank.amax_history[i, 0]), om[i].hist[0], tag + " amax")
        bank.update(recipe)
        oracle.update_metas(om)
        for i in range(2):
            assert_bits_equal(np_of(bank.amax_history[i]), om[i].hist, f"rep {rep} history {i}")
            assert_bits_equal(np_of(bank.scale[i]), om[i].scale, f"rep {rep} scale {i}")
            assert_bits_equal(np_of(bank.scale_inv[i]), om[i].scale_inv, f"rep {rep} scale_inv {i}")
    # after the first update both formats use their full range: nothing saturates
    # except the tensor's own maximum, nothing is NaN
    codes = np_of(q)
    assert not np.any((codes & 0x7F) == 0x7F)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_cast_transpose_dual_small_ragged(oracle, dtype):
    """One read, both formats, both layouts: every output equals the
    single-format oracle cast with that format's scale; the outputs the
    caller leaves NULL are not written; both amax slots get amax(x)."""
    rows, cols = 272, 400
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(rows, cols, generator=g) * torch.exp2(torch.randint(-12, 12, (rows, 1), generator=g))).to(dtype)
    X = np_of(x)
    s4, s5 = np.float32(3.5), np.float32(1.0 / 3.0)
    xd = x.cuda()
    sd4, sd5 = dev(np.array([s4])), dev(np.array([s5]))
    outs = [torch.full((rows, cols), 0xA5, dtype=torch.uint8, device="cuda"),
            torch.full((cols, rows), 0xA5, dtype=torch.uint8, device="cuda"),
            torch.full((rows, cols), 0xA5, dtype=torch.uint8, device="cuda"),
            torch.full((cols, rows), 0xA5, dtype=torch.uint8, device="cuda")]
    slots = torch.zeros(2, dtype=torch.float32, device="cuda")
    w4, w4t = oracle.cast_transpose(X, 0, s4)
    w5, w5t = oracle.cast_transpose(X, 1, s5)
    want = [w4, w4t, w5, w5t]
    for mask in (0b1111, 0b0101, 0b1010, 0b0001, 0b1000):
        for o in outs:
            o.fill_(0xA5)
        slots.zero_()
        use = [o if mask >> i & 1 else None for i, o in enumerate(outs)]
        F.fp8_cast_transpose_dual(xd, sd4, sd5, *use, amax_slot_e4m3=slots[0:1], amax_slot_e5m2=slots[1:2])
        for i in range(4):
            got = np_of(outs[i])
            if mask >> i & 1:
                assert_bits_equal(got, want[i], f"mask {mask:04b} output {i}")
            else:
                assert np.all(got == 0xA5), f"mask {mask:04b}: output {i} written"
        a = oracle.amax(X)
        assert_bits_equal(np_of(slots), np.array([a, a], dtype=np.float32), f"mask {mask:04b} amax")


def test_cast_transpose_dual_full_size(oracle):
    """The 2^28-element tensor through the dual-format kernel with the scales a
    first update of its two metas gives; all four outputs bit-exact."""
    rows = cols = 16384
    L = 1024
    x = synth.quant_tensor(device="cuda")
    X = np_of(x)
    bank = F.MetaBank([F.E4M3, F.E5M2], L)
    recipe = F.Recipe(F.FORMAT_HYBRID, L, F.AMAX_MAX, 0)
    F.fp8_amax(x, bank.amax_history[0, 0:1])
    F.fp8_amax(x, bank.amax_history[1, 0:1])
    bank.update(recipe)
    om = [oracle.Meta(L, 0), oracle.Meta(L, 1)]
    for m in om:
        m.record(X)
    oracle.update_metas(om)
    assert_bits_equal(np_of(bank.scale), np.array([om[0].scale, om[1].scale]), "scales")
    u8 = dict(dtype=torch.uint8, device="cuda")
    q4, q4t, q5, q5t = (torch.empty(rows, cols, **u8), torch.empty(cols, rows, **u8), torch.empty(rows, cols, **u8),
                        torch.empty(cols, rows, **u8))
    F.fp8_cast_transpose_dual(x, bank.scale[0:1], bank.scale[1:2], q4, q4t, q5, q5t, bank.amax_history[0, 0:1],
                              bank.amax_history[1, 0:1])
    for fmt, q, qt in ((0, q4, q4t), (1, q5, q5t)):
        wq, wqt = oracle.cast_transpose(X, fmt, om[fmt].scale)
        assert_bits_equal(np_of(q), wq, f"fmt {fmt} q")
        del wq
        assert_bits_equal(np_of(qt), wqt, f"fmt {fmt} q^T")
        del wqt
    a = oracle.amax(X)
    assert_bits_equal(np_of(bank.amax_history[:, 0]), np.array([a, a], dtype=np.float32), "amax slots")


@pytest.mark.parametrize("shape", [(272, 400), (16384, 16384)], ids=["272x400", "16384x16384"])
def test_cast_transpose_dual_update_matches_oracle(oracle, shape):
    """The dual-format cast-transpose with the two metas' scale update in its
    last workgroup: over 4 consecutive calls (histories of 1024 and 16, margin
    0 and 2, the ticket reused), every code, history entry, scale and inverse
    scale equals the oracle's cast-transpose of both formats followed by its
    update, bit for bit; the ticket is left at zero."""
    rows, cols = shape
    big = rows * cols > 1 << 20
    x = synth.quant_tensor(device="cuda", rows=rows, cols=cols)
    X = np_of(x)
    ticket = torch.zeros(1, dtype=torch.int32, device="cuda")
    u8 = dict(dtype=torch.uint8, device="cuda")
    outs = [torch.empty(rows, cols, **u8), torch.empty(cols, rows, **u8), torch.empty(rows, cols, **u8),
            torch.empty(cols, rows, **u8)]
    for L, margin in ((1024, 0), (16, 2)):
        bank = F.MetaBank([F.E4M3, F.E5M2], L)
        recipe = F.Recipe(F.FORMAT_HYBRID, L, F.AMAX_MAX, margin)
        om = [oracle.Meta(L, 0), oracle.Meta(L, 1)]
        for call in range(4 if not big else 2):
            xin = x if call % 2 == 0 else x * 3      # the amax changes between calls
            Xin = X if call % 2 == 0 else np_of(xin)
            F.fp8_cast_transpose_dual_update(xin, bank, recipe, ticket, *outs)
            torch.cuda.synchronize()
            tag = f"L {L} margin {margin} call {call}"
            for i, fmt in enumerate((0, 1)):
                wq, wqt = oracle.cast_transpose(Xin, fmt, om[fmt].scale)
                assert_bits_equal(np_of(outs[2 * i]), wq, f"{tag} fmt {fmt} q")
                del wq
                assert_bits_equal(np_of(outs[2 * i + 1]), wqt, f"{tag} fmt {fmt} q^T")
                del wqt
                om[fmt].record(Xin)
            oracle.update_metas(om, margin=margin)
            for i in range(2):
                assert_bits_equal(np_of(bank.amax_history[i]), om[i].hist, f"{tag} history {i}")
                assert_bits_equal(np_of(bank.scale[i]), om[i].scale, f"{tag} scale {i}")
                assert_bits_equal(np_of(bank.scale_inv[i]), om[i].scale_inv, f"{tag} scale_inv {i}")
            assert int(ticket.item()) == 0, "ticket not left at zero"
