"""GPU parity: the FP8 GEMM and its epilogues against the oracle's fp64 GEMM.

Shapes cover all three tile configurations (64, 128 and 256 square tiles),
ragged M/N/K tails (multiples of 16 that are not multiples of the tile), K=0,
both operand-format pairs of the layer (E4M3 x E4M3, E5M2 x E4M3) and the two
the layer does not use.
"""
import numpy as np
import pytest
import torch

import fp8_mixed_precision_reduce_amd as F
from helpers import (GELU_LIPSCHITZ, assert_bits_equal, assert_fast_bf16, assert_fast_f32, assert_gemm_bf16,
                     assert_gemm_f32, dev, fast_accum_bound, np_of)

pytestmark = pytest.mark.gpu
PAIRS = [((F.E4M3, 0), (F.E4M3, 0)), ((F.E5M2, 1), (F.E4M3, 0)), ((F.E4M3, 0), (F.E5M2, 1)),
         ((F.E5M2, 1), (F.E5M2, 1))]


def _scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def _codes(oracle, rng, shape, fmt, spread=4.0):
    x = (rng.standard_normal(shape) * np.exp2(rng.uniform(-spread, spread, shape))).astype(np.float32)
    return oracle.cast(x, fmt, 1.0)


def _torch_codes(x, fmt):
    """FP8 codes of x (in range) from PyTorch's float8 conversion, as uint8."""
    return x.to(torch.float8_e4m3fn if fmt == F.E4M3 else torch.float8_e5m2).view(torch.uint8)


def _run(a, af, b, bf, sa, sb, out_dtype=torch.float32, bias=None, epilogue=0, aux=False, d0=None):
    m, n = a.shape[0], b.shape[0]
    d = d0.clone() if d0 is not None else torch.empty(m, n, dtype=out_dtype, device="cuda")
    ax = torch.empty(m, n, dtype=out_dtype, device="cuda") if aux else None
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    F.fp8_gemm(dev(a), af, dev(b), bf, _scalar(sa), _scalar(sb), d, bias=bias, epilogue=epilogue, aux=ax,
               amax_d=amax)
    return d, ax, amax


SHAPES = [(16, 16, 16), (64, 64, 128), (80, 48, 400), (272, 528, 400), (1024, 768, 768), (1040, 1536, 1168),
          (4096, 4096, 256)]


@pytest.mark.parametrize("pair", PAIRS, ids=["e4m3xe4m3", "e5m2xe4m3", "e4m3xe5m2", "e5m2xe5m2"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_f32_matches_oracle(oracle, pair, shape):
    (af, oaf), (bf, obf) = pair
    m, n, k = shape
    rng = np.random.default_rng(m + 3 * n + 7 * k + af)
    a = _codes(oracle, rng, (m, k), oaf)
    b = _codes(oracle, rng, (n, k), obf)
    sa, sb = np.float32(0.0371), np.float32(1.73)
    d, _, amax = _run(a, af, b, bf, float(sa), float(sb))
    rows = np.unique(np.concatenate([np.arange(min(m, 64)), rng.integers(0, m, 64), [m - 1]]))
    want = oracle.gemm(a, oaf, b, obf, sa, sb, rows=rows)
    got = np_of(d)
    assert_gemm_f32(got[rows], want, f"{shape}")
    assert_bits_equal(np_of(amax)[0], np.float32(np.max(np.abs(got))), "output amax")


@pytest.mark.parametrize("shape", [(272, 528, 400), (2048, 2048, 512)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_bias_gelu_aux_bf16(oracle, shape):
    m, n, k = shape
    rng = np.random.default_rng(k)
    a = _codes(oracle, rng, (m, k), 0)
    b = _codes(oracle, rng, (n, k), 0)
    bias = rng.standard_normal(n).astype(np.float32)
    sa, sb = np.float32(0.02), np.float32(0.05)
    d, aux, amax = _run(a, F.E4M3, b, F.E4M3, float(sa), float(sb), torch.bfloat16, bias=dev(bias),
                        epilogue=F.EPI_GELU, aux=True)
    rows = np.unique(np.concatenate([np.arange(32), rng.integers(0, m, 48), [m - 1]]))
    y, pre = oracle.gemm(a, 0, b, 0, sa, sb, bias.astype(np.float64), gelu=True, rows=rows, want_pre=True)
    assert_gemm_bf16(np_of(d)[rows], y, oracle, "gelu(y)")
    assert_gemm_bf16(np_of(aux)[rows], pre, oracle, "pre-gelu aux")
    got = np_of(d)
    assert_bits_equal(np_of(amax)[0], np.float32(np.max(np.abs(oracle.bf16_to_f64(got)))), "amax of bf16 out")


def test_gemm_bf16_bias_and_accumulate(oracle):
    m, n, k = 320, 256, 272
    rng = np.random.default_rng(1)
    a = _codes(oracle, rng, (m, k), 1)
    b = _codes(oracle, rng, (n, k), 0)
    bias16 = oracle.bf16_from_f32(rng.standard_normal(n).astype(np.float32))
    d, _, _ = _run(a, F.E5M2, b, F.E4M3, 0.5, 0.25, torch.float32, bias=dev(bias16))
    want = oracle.gemm(a, 1, b, 0, 0.5, 0.25, oracle.bf16_to_f64(bias16))
    assert_gemm_f32(np_of(d), want, "bf16 bias")
    d0 = torch.from_numpy(rng.standard_normal((m, n)).astype(np.float32)).cuda()
    d, _, _ = _run(a, F.E5M2, b, F.E4M3, 0.5, 0.25, d0=d0, epilogue=F.EPI_ACCUMULATE)
    want = oracle.gemm(a, 1, b, 0, 0.5, 0.25) + np_of(d0).astype(np.float64)
    assert_gemm_f32(np_of(d), want, "accumulate")


def test_gemm_empty_k_writes_bias(oracle):
    m, n = 48, 64
    bias = np.arange(n, dtype=np.float32)
    d = torch.full((m, n), 7.0, device="cuda")
    a = torch.empty(m, 0, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, 0, dtype=torch.uint8, device="cuda")
    F.fp8_gemm(a, F.E4M3, b, F.E4M3, _scalar(1.0), _scalar(1.0), d, bias=dev(bias))
    assert np.array_equal(np_of(d), np.tile(bias, (m, 1)))


def test_gemm_deterministic(oracle):
    rng = np.random.default_rng(2)
    a = _codes(oracle, rng, (1024, 2048), 0)
    b = _codes(oracle, rng, (1536, 2048), 0)
    d1, _, m1 = _run(a, F.E4M3, b, F.E4M3, 1.0, 1.0)
    d2, _, m2 = _run(a, F.E4M3, b, F.E4M3, 1.0, 1.0)
    assert torch.equal(d1.view(torch.int32), d2.view(torch.int32)) and torch.equal(m1, m2)


@pytest.mark.parametrize("which", ["fc1", "fc2_dgrad", "fc1_wgrad", "fc2_wgrad"])
def test_gemm_full_size_mlp_shapes_sampled(oracle, which):
    """The MLP block's GEMM shapes at full size, in the launch configuration the
    benchmark times; the oracle recomputes 24 sampled rows."""
    m, n, k, af, oaf = {"fc1": (8192, 14336, 4096, F.E4M3, 0),
                        "fc2_dgrad": (8192, 14336, 4096, F.E5M2, 1),
                        "fc1_wgrad": (14336, 4096, 8192, F.E5M2, 1),
                        "fc2_wgrad": (4096, 14336, 8192, F.E5M2, 1)}[which]
    g = torch.Generator(device="cuda")
    g.manual_seed(m + n + k)
    # operand codes from PyTorch's own float8 conversions (not this library's cast)
    a = _torch_codes(torch.randn(m, k, device="cuda", generator=g) * 8.0, af)
    b = _torch_codes(torch.randn(n, k, device="cuda", generator=g) * 40.0, F.E4M3)
    d = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    F.fp8_gemm(a, af, b, F.E4M3, _scalar(0.125), _scalar(1 / 2000.0), d)
    rows = np.random.default_rng(0).choice(m, 24, replace=False)
    a_np = np_of(a)
    want = oracle.gemm(a_np, oaf, np_of(b), 0, np.float32(0.125), np.float32(1 / 2000.0), rows=rows)
    assert_gemm_bf16(np_of(d)[rows], want, oracle, which)
    # the same GEMM with fp32 output meets the normwise 1e-5 bound before rounding
    d32 = torch.empty(m, n, dtype=torch.float32, device="cuda")
    F.fp8_gemm(a, af, b, F.E4M3, _scalar(0.125), _scalar(1 / 2000.0), d32)
    assert_gemm_f32(np_of(d32)[rows], want, which + " f32")


def test_gemm_identity_over_every_code(oracle):
    """A row holding every finite code times an identity returns each decoded
    value exactly; a NaN or Inf operand makes its whole output row NaN."""
    for af, of in ((F.E4M3, 0), (F.E5M2, 1)):
        k = 256
        vals = np.array([oracle.decode(c, of) for c in range(256)])
        codes = np.where(np.isfinite(vals), np.arange(256), 0).astype(np.uint8)
        a = np.tile(codes, (16, 1))
        a[15, 7] = 0x7F                                              # NaN in both formats
        ident = np.zeros((k, k), np.uint8)
        ident[np.arange(k), np.arange(k)] = 0x38                    # E4M3 1.0
        d, _, _ = _run(a, af, ident, F.E4M3, 1.0, 1.0)
        got = np_of(d).astype(np.float64)
        want = np.where(np.isfinite(vals), vals, 0.0)
        assert np.array_equal(got[:15], np.tile(want, (15, 1)))
        assert np.all(np.isnan(got[15]))


# --------------------------------------------------------------------------
# The fast inner product (FP8LIN_EPI_FAST_ACCUM, native FP8 MFMA): checked
# against the measured group-truncation bound (tests/helpers.py) instead of the
# fp32 normwise bound, in every tile configuration and launch split the
# library uses and with every epilogue.

FAST_SHAPES = [(64, 64, 128), (272, 528, 400), (1024, 1024, 1024),   # 64 x 64 tiles
               (2048, 2048, 512), (2064, 1552, 656),                  # 128 x 128 tiles (ragged)
               (4096, 4096, 1024), (4112, 4368, 528)]                 # 256 x 256 tiles (ragged)


def _dec(oracle, codes, ofmt):
    return oracle.decode_table(ofmt)[codes]


@pytest.mark.parametrize("pair", PAIRS, ids=["e4m3xe4m3", "e5m2xe4m3", "e4m3xe5m2", "e5m2xe5m2"])
@pytest.mark.parametrize("shape", FAST_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_fast_accum_within_group_truncation_bound(oracle, pair, shape):
    (af, oaf), (bf, obf) = pair
    m, n, k = shape
    rng = np.random.default_rng(m + n + k + 11 * af + 13 * bf)
    a = _codes(oracle, rng, (m, k), oaf)
    b = _codes(oracle, rng, (n, k), obf)
    sa, sb = np.float32(0.5), np.float32(0.25)
    d, _, amax = _run(a, af, b, bf, float(sa), float(sb), epilogue=F.EPI_FAST_ACCUM)
    rows = np.unique(np.concatenate([rng.choice(m, min(m, 24), replace=False), [0, m - 1]]))
    want = oracle.gemm(a, oaf, b, obf, sa, sb, rows=rows)
    bound = fast_accum_bound(_dec(oracle, a[rows], oaf), _dec(oracle, b, obf), sa, sb)
    got = np_of(d)
    assert_fast_f32(got[rows], want, bound, f"fast {shape}")
    assert_bits_equal(np_of(amax)[0], np.float32(np.max(np.abs(got))), "output amax")


@pytest.mark.parametrize("shape", [(272, 528, 400), (2064, 1552, 656), (4112, 4368, 528)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_fast_accum_bf16_epilogues(oracle, shape):
    """bf16 output on the fast inner product with bias, GeLU, the pre-GeLU
    copy and a residual, then the FP8 copy of the output (codes and transposed
    codes exactly those of a cast of the output as written), in the 64-, 128-
    and 256-tile configurations."""
    m, n, k = shape
    rng = np.random.default_rng(m * 3 + n + k)
    a = _codes(oracle, rng, (m, k), 0)
    b = _codes(oracle, rng, (n, k), 0)
    sa, sb = np.float32(0.02), np.float32(0.05)
    bias = rng.standard_normal(n).astype(np.float32)
    r = oracle.bf16_from_f32(rng.standard_normal((m, n)).astype(np.float32))
    d = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    ax = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    F.fp8_gemm(dev(a), F.E4M3, dev(b), F.E4M3, _scalar(float(sa)), _scalar(float(sb)), d, bias=dev(bias),
               epilogue=F.EPI_GELU | F.EPI_FAST_ACCUM, aux=ax, residual=dev(r), amax_d=amax)
    rows = np.unique(np.concatenate([np.arange(8), rng.integers(0, m, 24), [m - 1]]))
    y, pre = oracle.gemm(a, 0, b, 0, sa, sb, bias.astype(np.float64), gelu=True, rows=rows, want_pre=True)
    bound = fast_accum_bound(_dec(oracle, a[rows], 0), _dec(oracle, b, 0), sa, sb)
    r64 = oracle.bf16_to_f64(r[rows])
    got = np_of(d)
    assert_fast_bf16(np_of(ax)[rows], pre, bound, f"{shape} pre-GeLU copy")
    assert_fast_bf16(got[rows], y + r64, bound, f"{shape} gelu(y) + residual", lipschitz=GELU_LIPSCHITZ,
                     extra=r64)
    assert_bits_equal(np_of(amax)[0], np.float32(np.max(np.abs(oracle.bf16_to_f64(got)))), "amax of d as written")
    # the FP8 copy of the output from the epilogue
    qs = np.float32(37.5)
    d2 = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    q = torch.full((m, n), 0xA5, dtype=torch.uint8, device="cuda")
    qt = torch.full((n, m), 0xA5, dtype=torch.uint8, device="cuda")
    F.fp8_gemm(dev(a), F.E4M3, dev(b), F.E4M3, _scalar(float(sa)), _scalar(float(sb)), d2, bias=dev(bias),
               epilogue=F.EPI_GELU | F.EPI_FAST_ACCUM, residual=dev(r),
               q_out=F.QOut(_scalar(float(qs)), q, qt, F.E4M3))
    D2 = np_of(d2)
    assert_bits_equal(D2, got, "same output with the FP8 copy")
    wq, wqt = oracle.cast_transpose(D2, 0, qs)
    assert_bits_equal(np_of(q), wq, "codes of the output")
    assert_bits_equal(np_of(qt), wqt, "transposed codes of the output")


@pytest.mark.parametrize("mode", ["f32_accumulate", "bf16_gelu_aux"])
@pytest.mark.parametrize("orient", ["tall", "wide"])
def test_gemm_fast_accum_partial_last_round_split(oracle, mode, orient):
    """The two-launch splits (256 x 256 tiles, then 128 x 128 tiles for the
    last rows or columns) on the fast inner product: outputs on both sides of
    the split, the output amax over the whole output, bias and epilogues."""
    m, n, k = (14336, 4096, 256) if orient == "tall" else (4096, 14336, 256)
    rng = np.random.default_rng(m + 2 * n + 5)
    a = _codes(oracle, rng, (m, k), 1)
    b = _codes(oracle, rng, (n, k), 0)
    sa, sb = np.float32(0.5), np.float32(0.25)
    rows = np.unique(np.concatenate([rng.integers(0, min(m, 12288), 8), rng.integers(min(m, 12288) - 256, m, 8),
                                     [0, m - 1] + ([12287, 12288] if m > 12288 else [])]))
    bias = rng.standard_normal(n).astype(np.float32)
    bound = fast_accum_bound(_dec(oracle, a[rows], 1), _dec(oracle, b, 0), sa, sb)
    if mode == "f32_accumulate":
        d0 = torch.from_numpy(rng.standard_normal((m, n)).astype(np.float32)).cuda()
        d, _, amax = _run(a, F.E5M2, b, F.E4M3, float(sa), float(sb), d0=d0, bias=dev(bias),
                          epilogue=F.EPI_ACCUMULATE | F.EPI_FAST_ACCUM)
        want = oracle.gemm(a, 1, b, 0, sa, sb, bias.astype(np.float64), rows=rows) + np_of(d0)[rows].astype(np.float64)
        got = np_of(d)
        assert_fast_f32(got[rows], want, bound, f"fast split ({orient}) f32 accumulate")
    else:
        d, ax, amax = _run(a, F.E5M2, b, F.E4M3, float(sa), float(sb), out_dtype=torch.bfloat16, bias=dev(bias),
                           epilogue=F.EPI_GELU | F.EPI_FAST_ACCUM, aux=True)
        want, pre = oracle.gemm(a, 1, b, 0, sa, sb, bias.astype(np.float64), gelu=True, rows=rows, want_pre=True)
        assert_fast_bf16(np_of(d)[rows], want, bound, f"fast split ({orient}) bf16 gelu", lipschitz=GELU_LIPSCHITZ)
        assert_fast_bf16(np_of(ax)[rows], pre, bound, f"fast split ({orient}) pre-GeLU copy")
        got = oracle.bf16_to_f64(np_of(d))
    assert_bits_equal(np_of(amax)[0], np.float32(np.max(np.abs(got))), "output amax over both launches")


MLP_GEMMS = {   # m, n, k, A format, output, epilogue of the MLP block's six GEMMs (8192 tokens, 4096, 14336)
    "fc1": (8192, 14336, 4096, F.E4M3, torch.bfloat16, F.EPI_GELU),
    "fc2": (8192, 4096, 14336, F.E4M3, torch.bfloat16, 0),
    "fc2_dgrad": (8192, 14336, 4096, F.E5M2, torch.bfloat16, 0),
    "fc1_dgrad": (8192, 4096, 14336, F.E5M2, torch.bfloat16, 0),
    "fc1_wgrad": (14336, 4096, 8192, F.E5M2, torch.float32, 0),
    "fc2_wgrad": (4096, 14336, 8192, F.E5M2, torch.float32, 0),
}


def _full_size_operands(m, n, k, af, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    # operand codes from PyTorch's own float8 conversions (not this library's cast)
    a = _torch_codes(torch.randn(m, k, device="cuda", generator=g) * 8.0, af)
    b = _torch_codes(torch.randn(n, k, device="cuda", generator=g) * 40.0, F.E4M3)
    return a, b


@pytest.mark.parametrize("which", list(MLP_GEMMS))
def test_gemm_fast_accum_full_size_mlp_shapes_sampled(oracle, which):
    """The MLP block's six GEMMs at full size on the fast inner product, in
    the launch configuration the benchmark's fast figure times (splits
    included); 8 sampled rows against the truncation bound."""
    m, n, k, af, odt, epi = MLP_GEMMS[which]
    oaf = 0 if af == F.E4M3 else 1
    a, b = _full_size_operands(m, n, k, af, m + n + k + 1)
    sa, sb = np.float32(0.125), np.float32(1 / 2000.0)
    d = torch.empty(m, n, dtype=odt, device="cuda")
    ax = torch.empty(m, n, dtype=odt, device="cuda") if epi else None
    F.fp8_gemm(a, af, b, F.E4M3, _scalar(float(sa)), _scalar(float(sb)), d, epilogue=epi | F.EPI_FAST_ACCUM, aux=ax)
    rows = np.sort(np.random.default_rng(1).choice(m, 8, replace=False))
    a_np, b_np = np_of(a), np_of(b)
    y, pre = oracle.gemm(a_np, oaf, b_np, 0, sa, sb, gelu=bool(epi), rows=rows, want_pre=True)
    bound = fast_accum_bound(_dec(oracle, a_np[rows], oaf), _dec(oracle, b_np, 0), sa, sb)
    if odt == torch.float32:
        assert_fast_f32(np_of(d)[rows], y, bound, which)
    else:
        assert_fast_bf16(np_of(d)[rows], y, bound, which, lipschitz=GELU_LIPSCHITZ if epi else 1.0)
        if epi:
            assert_fast_bf16(np_of(ax)[rows], pre, bound, which + " pre-GeLU copy")


@pytest.mark.parametrize("shape", [(8192, 4096, 14336), (8192, 8192, 28672)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_f32_long_reduction_sampled(oracle, shape):
    """The exact inner product meets the fp32 normwise 1e-5 bound at the
    longest reductions of the workloads: K = 14336 (the MLP block's FC2 and
    FC1 dgrad) and K = 28672 (the transformer layer's FC2 and FC1 dgrad), in
    both format pairs, fp32 output, 16 sampled rows."""
    m, n, k = shape
    rows = np.sort(np.random.default_rng(2).choice(m, 16, replace=False))
    for af, oaf in ((F.E4M3, 0), (F.E5M2, 1)):
        a, b = _full_size_operands(m, n, k, af, m + n + k + af)
        sa, sb = np.float32(0.125), np.float32(1 / 2000.0)
        d = torch.empty(m, n, dtype=torch.float32, device="cuda")
        F.fp8_gemm(a, af, b, F.E4M3, _scalar(float(sa)), _scalar(float(sb)), d)
        want = oracle.gemm(np_of(a), oaf, np_of(b), 0, sa, sb, rows=rows)
        assert_gemm_f32(np_of(d)[rows], want, f"{shape} A format {af}")
        del a, b, d
        torch.cuda.empty_cache()


@pytest.mark.parametrize("in_place", [False, True], ids=["separate", "in_place"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", [(272, 528, 400), (2048, 1536, 512)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_residual(oracle, shape, out_dtype, in_place):
    """d = gelu(y) + residual (and y + residual), added in fp32 before the one
    rounding to the output type; residual may be d itself (in-place add).
    Covers a 128- and a 256-tile configuration with ragged tails."""
    m, n, k = shape
    rng = np.random.default_rng(m + n + k + (1 if in_place else 0))
    a = _codes(oracle, rng, (m, k), 0)
    b = _codes(oracle, rng, (n, k), 0)
    sa, sb = np.float32(0.05), np.float32(0.7)
    r = rng.standard_normal((m, n)).astype(np.float32)
    r_store = r if out_dtype == torch.float32 else oracle.bf16_from_f32(r)
    for gelu in (False, True):
        res = dev(r_store)
        d = res if in_place else torch.empty(m, n, dtype=out_dtype, device="cuda")
        ax = torch.empty(m, n, dtype=out_dtype, device="cuda") if gelu else None
        amax = torch.zeros(1, dtype=torch.float32, device="cuda")
        F.fp8_gemm(dev(a), F.E4M3, dev(b), F.E4M3, _scalar(float(sa)), _scalar(float(sb)), d,
                   epilogue=F.EPI_GELU if gelu else 0, aux=ax, residual=res, amax_d=amax)
        rows = np.unique(np.concatenate([np.arange(32), rng.integers(0, m, 64), [m - 1]]))
        y, pre = oracle.gemm(a, 0, b, 0, sa, sb, gelu=gelu, rows=rows, want_pre=True)
        want = oracle.add_residual(y, r_store[rows])
        got = np_of(d)
        tag = f"{shape} gelu={gelu} in_place={in_place}"
        if out_dtype == torch.float32:
            assert_gemm_f32(got[rows], want, tag)
        else:
            assert_gemm_bf16(got[rows], want, oracle, tag)
            if gelu:
                assert_gemm_bf16(np_of(ax)[rows], pre, oracle, tag + " aux")
        full = got.astype(np.float64) if out_dtype == torch.float32 else oracle.bf16_to_f64(got)
        assert_bits_equal(np_of(amax)[0], np.float32(np.max(np.abs(full))), tag + " amax of d as written")


@pytest.mark.parametrize("fmt", [(F.E4M3, 0), (F.E5M2, 1)], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", [(80, 48, 400), (272, 528, 400), (2048, 1536, 512), (1040, 4096, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_fp8_output(oracle, shape, fmt):
    """The epilogue's FP8 copy of a bf16 output (GeLU and residual on): the
    codes and transposed codes equal the oracle's cast-transpose of the bf16
    output as written, with the given scale; without d the same codes come
    out and the amax is unchanged.  Covers the 64, 128 and 256 tile
    configurations with ragged tails."""
    lf, of = fmt
    m, n, k = shape
    rng = np.random.default_rng(m + 5 * n + k + lf)
    a = _codes(oracle, rng, (m, k), 0)
    b = _codes(oracle, rng, (n, k), 0)
    sa, sb = np.float32(0.05), np.float32(0.7)
    r = oracle.bf16_from_f32(rng.standard_normal((m, n)).astype(np.float32))
    qs = np.float32(37.5 if lf == F.E4M3 else 3000.0)
    outs = []
    for with_d in (True, False):
        d = torch.empty(m, n, dtype=torch.bfloat16, device="cuda") if with_d else None
        ax = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
        q = torch.full((m, n), 0xA5, dtype=torch.uint8, device="cuda")
        qt = torch.full((n, m), 0xA5, dtype=torch.uint8, device="cuda")
        amax = torch.zeros(1, dtype=torch.float32, device="cuda")
        F.fp8_gemm(dev(a), F.E4M3, dev(b), F.E4M3, _scalar(float(sa)), _scalar(float(sb)), d, epilogue=F.EPI_GELU,
                   aux=ax, residual=dev(r), amax_d=amax, q_out=F.QOut(_scalar(float(qs)), q, qt, lf))
        outs.append((np_of(d) if with_d else None, np_of(q), np_of(qt), np_of(amax)[0]))
    D, q1, qt1, a1 = outs[0]
    wq, wqt = oracle.cast_transpose(D, of, qs)
    assert_bits_equal(q1, wq, "codes")
    assert_bits_equal(qt1, wqt, "transposed codes")
    assert_bits_equal(a1, oracle.amax(D), "amax of d as written")
    _, q2, qt2, a2 = outs[1]
    assert_bits_equal(q2, q1, "codes without d")
    assert_bits_equal(qt2, qt1, "transposed codes without d")
    assert_bits_equal(a2, a1, "amax without d")
    rows = np.unique(np.concatenate([np.arange(16), rng.integers(0, m, 32), [m - 1]]))
    y = oracle.gemm(a, 0, b, 0, sa, sb, gelu=True, rows=rows)
    assert_gemm_bf16(D[rows], oracle.add_residual(y, r[rows]), oracle, "d")


@pytest.mark.parametrize("shape", [(272, 8192, 128), (1040, 8192, 256), (2064, 16384, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_f32_row_stride_of_32k_multiple(oracle, shape):
    """fp32 outputs whose rows are a multiple of 32 KiB apart (8192 or 16384
    columns) take the LDS-staged epilogue; the three shapes run it on 64-,
    128- and 256-tile configurations with a ragged M.  Bias, residual and
    accumulate are applied in the register path's order, so the results are
    checked against the oracle and the amax against the output as written;
    a GeLU epilogue on the same shape (register path) is checked too."""
    m, n, k = shape
    rng = np.random.default_rng(m + n + k)
    a = _codes(oracle, rng, (m, k), 1)
    b = _codes(oracle, rng, (n, k), 0)
    sa, sb = np.float32(0.125), np.float32(0.75)
    bias = rng.standard_normal(n).astype(np.float32)
    r = rng.standard_normal((m, n)).astype(np.float32)
    d0 = rng.standard_normal((m, n)).astype(np.float32)
    rows = np.unique(np.concatenate([np.arange(8), rng.integers(0, m, 40), [m - 1]]))
    # bias + residual
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    d = torch.empty(m, n, dtype=torch.float32, device="cuda")
    F.fp8_gemm(dev(a), F.E5M2, dev(b), F.E4M3, _scalar(float(sa)), _scalar(float(sb)), d, bias=dev(bias),
               residual=dev(r), amax_d=amax)
    y = oracle.gemm(a, 1, b, 0, sa, sb, bias.astype(np.float64), rows=rows)
    got = np_of(d)
    assert_gemm_f32(got[rows], oracle.add_residual(y, r[rows]), f"{shape} bias+residual")
    assert_bits_equal(np_of(amax)[0], np.float32(np.max(np.abs(got))), f"{shape} amax")
    # accumulate into d
    dacc = dev(d0)
    F.fp8_gemm(dev(a), F.E5M2, dev(b), F.E4M3, _scalar(float(sa)), _scalar(float(sb)), dacc,
               epilogue=F.EPI_ACCUMULATE)
    want = oracle.gemm(a, 1, b, 0, sa, sb, rows=rows) + d0[rows].astype(np.float64)
    assert_gemm_f32(np_of(dacc)[rows], want, f"{shape} accumulate")
    # GeLU with its fp32 pre-GeLU copy
    dg = torch.empty(m, n, dtype=torch.float32, device="cuda")
    ax = torch.empty(m, n, dtype=torch.float32, device="cuda")
    F.fp8_gemm(dev(a), F.E5M2, dev(b), F.E4M3, _scalar(float(sa)), _scalar(float(sb)), dg, bias=dev(bias),
               epilogue=F.EPI_GELU, aux=ax)
    yg, pre = oracle.gemm(a, 1, b, 0, sa, sb, bias.astype(np.float64), gelu=True, rows=rows, want_pre=True)
    assert_gemm_f32(np_of(dg)[rows], yg, f"{shape} gelu")
    assert_gemm_f32(np_of(ax)[rows], pre, f"{shape} pre-gelu copy")


@pytest.mark.parametrize("mode", ["f32_accumulate", "bf16_gelu_aux"])
@pytest.mark.parametrize("orient", ["tall", "wide"])
def test_gemm_partial_last_round_split(oracle, mode, orient):
    """14336 x 4096 and 4096 x 14336 outputs: 896 tiles of 256 x 256 on a
    256-workgroup grid leave a half-empty last round, so the library runs the
    first 12288 rows (tall) or columns (wide) on 256 x 256 tiles and the rest
    on 128 x 128 tiles (two launches; the wide case writes through the output's
    row stride).  Outputs on both sides of the split, the output amax over the
    whole output, the bias, and the accumulate / GeLU / pre-GeLU-copy
    epilogues are checked."""
    m, n, k = (14336, 4096, 256) if orient == "tall" else (4096, 14336, 256)
    rng = np.random.default_rng(m + 2 * n)
    a = _codes(oracle, rng, (m, k), 1)
    b = _codes(oracle, rng, (n, k), 0)
    sa, sb = np.float32(0.5), np.float32(0.25)
    rows = np.unique(np.concatenate([rng.integers(0, min(m, 12288), 24), rng.integers(min(m, 12288) - 256, m, 24),
                                     [0, m - 1] + ([12287, 12288] if m > 12288 else [])]))
    bias = rng.standard_normal(n).astype(np.float32)
    if mode == "f32_accumulate":
        d0 = torch.from_numpy(rng.standard_normal((m, n)).astype(np.float32)).cuda()
        d, _, amax = _run(a, F.E5M2, b, F.E4M3, float(sa), float(sb), d0=d0, bias=dev(bias),
                          epilogue=F.EPI_ACCUMULATE)
        want = oracle.gemm(a, 1, b, 0, sa, sb, bias.astype(np.float64), rows=rows) + np_of(d0)[rows].astype(np.float64)
        got = np_of(d)
        assert_gemm_f32(got[rows], want, f"split ({orient}) f32 accumulate")
    else:
        d, ax, amax = _run(a, F.E5M2, b, F.E4M3, float(sa), float(sb), out_dtype=torch.bfloat16, bias=dev(bias),
                           epilogue=F.EPI_GELU, aux=True)
        want, pre = oracle.gemm(a, 1, b, 0, sa, sb, bias.astype(np.float64), gelu=True, rows=rows, want_pre=True)
        assert_gemm_bf16(np_of(d)[rows], want, oracle, f"split ({orient}) bf16 gelu")
        assert_gemm_bf16(np_of(ax)[rows], pre, oracle, f"split ({orient}) pre-GeLU copy")
        got = oracle.bf16_to_f64(np_of(d))
    assert_bits_equal(np_of(amax)[0], np.float32(np.max(np.abs(got))), "output amax over both launches")
