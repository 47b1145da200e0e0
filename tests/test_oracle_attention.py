"""Pins of the attention oracle against what mathematics fixes: finite
differences of the loss <O, G>, closed forms of the softmax (equal keys, one
dominant key), invariance under a joint permutation of keys and values, and
the [Q | K | V] head-major column layout by explicit index arithmetic."""
import numpy as np
import pytest

from oracle import attention as A


def _loss(q, k, v, g):
    o, _, _ = A.head_fwd(q, k, v)
    return float(np.sum(o * g))


@pytest.mark.parametrize("seed", [0, 1])
def test_head_gradient_matches_finite_differences(seed):
    rng = np.random.default_rng(seed)
    s, d = 5, 4
    q, k, v, g = (rng.standard_normal((s, d)) for _ in range(4))
    o, _, _ = A.head_fwd(q, k, v)
    got = A.head_bwd(q, k, v, o, g)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            args_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            num[idx] = (_loss(*args_p, g) - _loss(*args_m, g)) / (2 * eps)
        assert np.allclose(got[name], num, rtol=1e-6, atol=1e-8), name
        # the absolute-term sums bound the gradients (triangle inequality)
        assert np.all(np.abs(got[name]) <= got["t" + name[1]] * (1 + 1e-12))


def test_equal_keys_give_the_mean_of_the_values():
    rng = np.random.default_rng(2)
    s, d = 7, 8
    q = rng.standard_normal((s, d))
    k = np.tile(rng.standard_normal((1, d)), (s, 1))
    v = rng.standard_normal((s, d))
    o, lse, a = A.head_fwd(q, k, v)
    assert np.allclose(o, np.tile(v.mean(axis=0), (s, 1)), rtol=0, atol=1e-14)
    assert np.allclose(lse, q @ k[0] / np.sqrt(d) + np.log(s), rtol=0, atol=1e-12)
    assert np.allclose(a, np.tile(np.abs(v).mean(axis=0), (s, 1)), rtol=0, atol=1e-14)


def test_one_dominant_key_selects_its_value():
    rng = np.random.default_rng(3)
    s, d = 16, 8
    k = rng.standard_normal((s, d)) * 0.01
    k[5] = 40.0 * np.ones(d)
    q = np.ones((3, d))
    v = rng.standard_normal((s, d))
    o, lse, _ = A.head_fwd(q, k, v)
    assert np.allclose(o, np.tile(v[5], (3, 1)), rtol=0, atol=1e-30 + 1e-12)
    assert np.allclose(lse, 40.0 * d / np.sqrt(d), rtol=1e-12)


def test_joint_key_value_permutation_is_invisible():
    rng = np.random.default_rng(4)
    s, d = 33, 16
    q, k, v = (rng.standard_normal((s, d)) for _ in range(3))
    perm = rng.permutation(s)
    o1, l1, _ = A.head_fwd(q, k, v)
    o2, l2, _ = A.head_fwd(q, k[perm], v[perm])
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-14) and np.allclose(l1, l2, rtol=1e-14)
    g = rng.standard_normal((s, d))
    b1 = A.head_bwd(q, k, v, o1, g)
    b2 = A.head_bwd(q, k[perm], v[perm], o1, g)
    assert np.allclose(b1["dq"], b2["dq"], rtol=1e-12, atol=1e-13)
    assert np.allclose(b1["dk"][perm], b2["dk"], rtol=1e-12, atol=1e-13)
    assert np.allclose(b1["dv"][perm], b2["dv"], rtol=1e-12, atol=1e-13)


def test_rows_argument_selects_query_rows():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((40, 8)) for _ in range(3))
    rows = np.array([0, 7, 39])
    o, lse, a = A.head_fwd(q, k, v)
    o2, lse2, a2 = A.head_fwd(q, k, v, rows=rows)
    assert np.array_equal(o[rows], o2) and np.array_equal(lse[rows], lse2) and np.array_equal(a[rows], a2)


def test_column_layout_is_qkv_then_heads():
    b_, s_, h_, d_ = 2, 3, 4, 5
    # value = code of (part, b, h, s, d), written at the column the layout gives
    qkv = np.zeros((b_ * s_, 3 * h_ * d_))
    for part in range(3):
        for b in range(b_):
            for h in range(h_):
                for s in range(s_):
                    for d in range(d_):
                        qkv[b * s_ + s, part * h_ * d_ + h * d_ + d] = (((part * 10 + b) * 10 + h) * 10 + s) * 10 + d
    q, k, v = A.split_heads(qkv, b_, s_, h_)
    for part, x in enumerate((q, k, v)):
        for idx in np.ndindex(x.shape):
            b, h, s, d = idx
            assert x[idx] == (((part * 10 + b) * 10 + h) * 10 + s) * 10 + d
    assert np.array_equal(A.merge_heads(q), qkv[:, :h_ * d_])


def test_whole_layer_gradient_matches_finite_differences():
    """dqkv of attention_bwd against central differences of <ctx, G> through
    attention_fwd, on entries of all three parts and several heads."""
    rng = np.random.default_rng(6)
    b_, s_, h_, d_ = 2, 4, 2, 3
    qkv = rng.standard_normal((b_ * s_, 3 * h_ * d_))
    g = rng.standard_normal((b_ * s_, h_ * d_))
    ctx, _, _ = A.attention_fwd(qkv, b_, s_, h_)
    dqkv, t = A.attention_bwd(qkv, ctx, g, b_, s_, h_)
    eps = 1e-6
    for _ in range(30):
        i, j = rng.integers(qkv.shape[0]), rng.integers(qkv.shape[1])
        p, m = qkv.copy(), qkv.copy()
        p[i, j] += eps
        m[i, j] -= eps
        num = (np.sum(A.attention_fwd(p, b_, s_, h_)[0] * g) - np.sum(A.attention_fwd(m, b_, s_, h_)[0] * g)) / (2 * eps)
        assert abs(dqkv[i, j] - num) <= 1e-6 * (1 + abs(num)), (i, j)
        assert abs(dqkv[i, j]) <= t[i, j] * (1 + 1e-12)


def test_bf16_input_path_decodes_bits():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 6)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)            # truncation: exact bf16 values
    dec = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q1, k1, v1 = A.split_heads(bits, 1, 4, 1)
    q2, k2, v2 = A.split_heads(dec, 1, 4, 1)
    assert np.array_equal(q1, q2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
