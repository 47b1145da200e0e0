"""Pins for the oracle's FP8 GEMM, GeLU and layer composition (CPU only).

GEMM: exact 128-bit integer sums, closed forms (identity, all-ones), numpy's
fp64 matmul on the decoded operands, and the transposition identities the
backward pass relies on.  GeLU: scipy's normal CDF, symmetry and limits.
"""
import math

import numpy as np
import pytest
import scipy.special

E4M3, E5M2 = 0, 1


def _rand_codes(rng, shape, fmt):
    """Random finite codes of a format (no NaN / Inf)."""
    maxc = 0x7E if fmt == E4M3 else 0x7B
    mag = rng.integers(0, maxc + 1, size=shape)
    sign = rng.integers(0, 2, size=shape) << 7
    return (mag | sign).astype(np.uint8)


def _rand_normal_codes(oracle, rng, shape, fmt, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return oracle.cast(x, fmt, 1.0)


@pytest.mark.parametrize("afmt,bfmt", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)])
def test_gemm_fp64_matches_exact_integer_sum(oracle, afmt, bfmt):
    rng = np.random.default_rng(10 + afmt * 2 + bfmt)
    for (m, n, k) in ((3, 5, 16), (4, 4, 48), (2, 3, 160)):
        a = _rand_codes(rng, (m, k), afmt)
        b = _rand_codes(rng, (n, k), bfmt)
        ints, e = oracle.gemm_exact(a, afmt, b, bfmt)
        y = oracle.gemm(a, afmt, b, bfmt)
        exact = np.array([[math.ldexp(float(v), e) for v in row] for row in ints])
        # the fp64 sum of at most 160 products of <= 7-bit values stays within 2^-50
        num = np.linalg.norm(y - exact)
        den = max(np.linalg.norm(exact), 1e-300)
        assert num <= 2.0 ** -50 * den
        # rebuild the exact value independently of the fp64 path: Python big ints
        ta = [oracle.decode(c, afmt) for c in range(256)]
        tb = [oracle.decode(c, bfmt) for c in range(256)]
        fa = 9 if afmt == E4M3 else 16
        fb = 9 if bfmt == E4M3 else 16
        for i in range(m):
            for j in range(n):
                s = sum(int(ta[a[i, kk]] * 2 ** fa) * int(tb[b[j, kk]] * 2 ** fb) for kk in range(k))
                assert s == ints[i][j] and e == -(fa + fb)


def test_gemm_matches_numpy_matmul_on_decoded(oracle):
    rng = np.random.default_rng(77)
    for afmt, bfmt in ((E4M3, E4M3), (E5M2, E4M3)):
        a = _rand_normal_codes(oracle, rng, (37, 96), afmt, 3.0)
        b = _rand_normal_codes(oracle, rng, (29, 96), bfmt, 3.0)
        ta, tb = oracle.decode_table(afmt), oracle.decode_table(bfmt)
        sa, sb = np.float32(0.37), np.float32(1.9)
        bias = rng.standard_normal(29)
        ref = (ta[a] @ tb[b].T) * np.float64(sa) * np.float64(sb) + bias
        y = oracle.gemm(a, afmt, b, bfmt, sa, sb, bias)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
        rows = np.array([5, 0, 36, 5])
        yr = oracle.gemm(a, afmt, b, bfmt, sa, sb, bias, rows=rows)
        assert np.array_equal(yr, y[rows])


def test_gemm_identity_and_ones(oracle):
    rng = np.random.default_rng(8)
    k = 64
    x = _rand_normal_codes(oracle, rng, (24, k), E4M3, 2.0)
    ident = np.zeros((k, k), np.uint8)
    ident[np.arange(k), np.arange(k)] = 0x38                      # E4M3 1.0
    assert oracle.decode(0x38, E4M3) == 1.0
    sinv = np.float32(0.125)
    y = oracle.gemm(x, E4M3, ident, E4M3, sinv, 1.0)
    assert np.array_equal(y, oracle.decode_table(E4M3)[x] * 0.125)
    ones_a = np.full((5, k), 0x38, np.uint8)
    ones_b = np.full((7, k), 0x3C, np.uint8)                      # E5M2 1.0
    assert oracle.decode(0x3C, E5M2) == 1.0
    y = oracle.gemm(ones_a, E4M3, ones_b, E5M2, 0.5, 3.0)
    assert np.all(y == k * 0.5 * np.float64(np.float32(3.0)))


def test_gemm_minimal_shape_and_empty_k(oracle):
    a = np.full((16, 16), 0x38, np.uint8)
    assert np.all(oracle.gemm(a, E4M3, a, E4M3) == 16.0)
    z = np.zeros((3, 0), np.uint8)
    y = oracle.gemm(z, E4M3, np.zeros((4, 0), np.uint8), E4M3, 1.0, 1.0, np.arange(4.0))
    assert np.array_equal(y, np.tile(np.arange(4.0), (3, 1)))


def test_backward_transposition_identities(oracle):
    """dgrad from (dYq, Wq^T) and wgrad from (dYq^T, Xq^T) equal the direct sums
    over the un-transposed codes."""
    rng = np.random.default_rng(12)
    m, n, k = 40, 24, 32
    g = _rand_normal_codes(oracle, rng, (m, n), E5M2)
    w = _rand_normal_codes(oracle, rng, (n, k), E4M3)
    x = _rand_normal_codes(oracle, rng, (m, k), E4M3)
    G, W, X = oracle.decode_table(E5M2)[g], oracle.decode_table(E4M3)[w], oracle.decode_table(E4M3)[x]
    dx = oracle.gemm(g, E5M2, oracle.transpose_u8(w), E4M3)
    dw = oracle.gemm(oracle.transpose_u8(g), E5M2, oracle.transpose_u8(x), E4M3)
    direct_dx = np.array([[sum(G[i, j] * W[j, kk] for j in range(n)) for kk in range(k)] for i in range(m)])
    direct_dw = np.array([[sum(G[i, j] * X[i, kk] for i in range(m)) for kk in range(k)] for j in range(n)])
    assert np.allclose(dx, direct_dx, rtol=1e-13, atol=0)
    assert np.allclose(dw, direct_dw, rtol=1e-13, atol=0)


# ------------------------------------------------------------------ GeLU ----

def test_gelu_against_normal_cdf(oracle):
    z = np.linspace(-12, 12, 2001)
    ref = z * scipy.special.ndtr(z)
    got = np.array([oracle.gelu(v) for v in z])
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)
    # odd-part identity gelu(z) - gelu(-z) = z, limits, and the derivative
    for v in (0.3, 1.7, 5.0):
        assert math.isclose(oracle.gelu(v) - oracle.gelu(-v), v, rel_tol=1e-14)
    assert oracle.gelu(0.0) == 0.0 and oracle.gelu(40.0) == 40.0 and oracle.gelu(-40.0) == -0.0
    assert oracle.gelu_grad(0.0) == 0.5
    for v in np.linspace(-6, 6, 61):
        h = 1e-6
        fd = (oracle.gelu(v + h) - oracle.gelu(v - h)) / (2 * h)
        assert math.isclose(oracle.gelu_grad(v), fd, rel_tol=1e-6, abs_tol=1e-9)


def test_gelu_bwd_rounding(oracle):
    rng = np.random.default_rng(6)
    dh = rng.standard_normal(1000).astype(np.float32)
    z = rng.standard_normal(1000).astype(np.float32)
    got = oracle.gelu_bwd(dh, z)
    z64 = z.astype(np.float64)
    ref = dh.astype(np.float64) * (scipy.special.ndtr(z64) + z64 * np.exp(-0.5 * z64 ** 2)
                                   / math.sqrt(2 * math.pi))
    assert np.allclose(got, ref, rtol=2 ** -23, atol=1e-30)


# ------------------------------------------------------ layer composition ----

def test_layer_steps_constant_input_gives_constant_scale(oracle):
    """Same inputs every step: after the first update the scales stop moving."""
    rng = np.random.default_rng(12345)
    x = rng.uniform(0, 1, (64, 48)).astype(np.float32)
    w = rng.uniform(-1 / math.sqrt(48), 1 / math.sqrt(48), (32, 48)).astype(np.float32)
    mx, mw = oracle.Meta(16, E4M3), oracle.Meta(16, E4M3)
    scales = []
    for _ in range(4):
        oracle.linear_fwd(x, w, mx, mw)
        oracle.update_metas([mx, mw])
        scales.append((mx.scale, mw.scale))
    assert scales[0] == scales[1] == scales[2] == scales[3]
    assert mx.scale == np.float32(448.0 / np.float64(x.max()))


def test_e5m2_underflow_before_first_update(oracle):
    """N(0,1)*2^-20 gradients cast at the initial scale 1 underflow to zero in
    E5M2 (amax ~ 5*2^-20 is below half the smallest subnormal 2^-17); after the
    first update the scale lifts them into range."""
    rng = np.random.default_rng(99)
    dy = (rng.standard_normal((256, 96)) * 2.0 ** -20).astype(np.float32)
    mg = oracle.Meta(16, E5M2)
    q0 = oracle.cast(dy, E5M2, mg.scale)
    assert np.count_nonzero(q0 & 0x7F) == 0
    mg.record(dy)
    oracle.update_metas([mg])
    q1 = oracle.cast(dy, E5M2, mg.scale)
    assert np.count_nonzero(q1 & 0x7F) > 0.99 * q1.size


def test_fp8_forward_error_is_quantisation_sized(oracle):
    """Context from the pages' 768x768 example: FP8 outputs differ from fp32 by
    a few percent of their size, not more."""
    rng = np.random.default_rng(12345)
    x = rng.uniform(0, 1, (128, 768)).astype(np.float32)
    w = rng.uniform(-1 / math.sqrt(768), 1 / math.sqrt(768), (96, 768)).astype(np.float32)
    b = rng.uniform(-1 / math.sqrt(768), 1 / math.sqrt(768), 96).astype(np.float32)
    mx, mw = oracle.Meta(16, E4M3), oracle.Meta(16, E4M3)
    oracle.linear_fwd(x, w, mx, mw, bias=b)
    oracle.update_metas([mx, mw])
    out = oracle.linear_fwd(x, w, mx, mw, bias=b)
    ref = x.astype(np.float64) @ w.astype(np.float64).T + b
    rel = np.linalg.norm(out["y"] - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.06
    assert 0.2 < ref.std() < 0.5


def test_linear_bwd_composition(oracle):
    rng = np.random.default_rng(31)
    m, n, k = 48, 32, 64
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    dy = rng.standard_normal((m, n)).astype(np.float32)
    mx, mw, mg = oracle.Meta(4, E4M3), oracle.Meta(4, E4M3), oracle.Meta(4, E5M2)
    for _ in range(2):
        sv = oracle.linear_fwd(x, w, mx, mw)
        bw = oracle.linear_bwd(dy, sv, mg)
        oracle.update_metas([mx, mw, mg])
    X = oracle.decode_table(E4M3)[sv["xq"]] * np.float64(sv["sinv_x"])
    W = oracle.decode_table(E4M3)[sv["wq"]] * np.float64(sv["sinv_w"])
    G = oracle.decode_table(E5M2)[bw["gq"]] * np.float64(bw["sinv_g"])
    assert np.allclose(bw["dx"], G @ W, rtol=1e-12, atol=1e-12)
    assert np.allclose(bw["dw"], G.T @ X, rtol=1e-12, atol=1e-12)
    assert np.allclose(bw["dbias"], dy.astype(np.float64).sum(0), rtol=1e-12)
    # the FP8 gradients are close to the fp64 ones (E5M2 has 2 mantissa bits)
    ref_dx = dy.astype(np.float64) @ w.astype(np.float64)
    assert np.linalg.norm(bw["dx"] - ref_dx) / np.linalg.norm(ref_dx) < 0.15
