"""Oracle for the bf16 softmax attention core between the QKV and output
projections of the transformer layer.

TEST INFRASTRUCTURE ONLY (the same rule as the rest of this package: only
tests/, the smoke check and bench.py's CPU-baseline leg use it).

What is computed: per batch b and head h, scaled dot-product attention with
no mask,
    S = Q K^T / sqrt(D),  P = softmax(S) along the keys,  O = P V,
and its gradient for a loss <O, dO>:
    dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
    dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D).
The pages' vision-transformer workload ([PT-VI], its ViT-Big configuration:
embedding width, depth, number of heads) runs this core in bf16 between FP8
linears; the pages do not write the core out, so the plainest reading is taken:
the textbook scaled dot-product attention, no mask (a vision transformer attends
over all tokens), head width = hidden / heads, and the fused projection's
output columns split as [Q | K | V], each head-major (head h owns columns
h*D .. h*D+D-1 of its part).

Everything is fp64 on the decoded bf16 inputs, with numpy's matmul, exp and
sum as the only library steps.  rowsum(dO * O) equals sum_k P dP exactly when
O is the exact output; the backward takes O as an input (the forward's saved
output, as the method keeps it), so with the oracle's own O it is the exact
gradient (pinned by finite differences in tests/test_oracle_attention.py).
"""
import numpy as np


def _bf16_to_f64(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def split_heads(qkv, batch, seq, heads):
    """[B*S][3*H*D] bf16 bits (or float) -> q, k, v as fp64 [B][H][S][D]."""
    a = np.asarray(qkv)
    x = _bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)
    hd = x.shape[1] // 3
    d = hd // heads
    x = x.reshape(batch, seq, 3, heads, d)
    return (np.ascontiguousarray(x[:, :, 0].transpose(0, 2, 1, 3)),
            np.ascontiguousarray(x[:, :, 1].transpose(0, 2, 1, 3)),
            np.ascontiguousarray(x[:, :, 2].transpose(0, 2, 1, 3)))


def merge_heads(o):
    """[B][H][S][D] -> [B*S][H*D]."""
    b, h, s, d = o.shape
    return np.ascontiguousarray(o.transpose(0, 2, 1, 3)).reshape(b * s, h * d)


def head_fwd(q, k, v, rows=None):
    """One head: q [S][D] (or the query rows `rows` of it), k, v [S][D].
    Returns O [len(rows)][D], the natural-log LSE per query row, and
    A = sum_k P |V| (the sum of absolute terms of each output, for the
    rounding bound of a bf16 implementation)."""
    d = q.shape[1]
    qs = q if rows is None else q[rows]
    s = (qs @ k.T) / np.sqrt(d)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    return p @ v, m[:, 0] + np.log(l[:, 0]), p @ np.abs(v)


def head_probs(q, k, rows=None):
    d = q.shape[1]
    qs = q if rows is None else q[rows]
    s = (qs @ k.T) / np.sqrt(d)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def head_bwd(q, k, v, o, do):
    """Gradient of one head for the loss <O, dO>; o is the forward's output
    (as saved).  Returns dq, dk, dv and, for each, the sum of absolute terms of
    its final contraction with dS replaced by P (|dP| + |D|) (the scale of the
    roundings a bf16 implementation makes on the way)."""
    d = q.shape[1]
    c = 1.0 / np.sqrt(d)
    p = head_probs(q, k)
    dv = p.T @ do
    dp = do @ v.T
    dd = (do * o).sum(axis=1)
    ds = p * (dp - dd[:, None])
    dq = (ds @ k) * c
    dk = (ds.T @ q) * c
    ads = p * (np.abs(dp) + np.abs(dd)[:, None])
    return dict(dq=dq, dk=dk, dv=dv, tq=(ads @ np.abs(k)) * c, tk=(ads.T @ np.abs(q)) * c, tv=p.T @ np.abs(do))


def attention_fwd(qkv, batch, seq, heads):
    """Whole forward: qkv [B*S][3*H*D] (bf16 bits) -> ctx [B*S][H*D] fp64,
    lse [B][H][S] fp64, and the absolute-term sums A [B*S][H*D]."""
    q, k, v = split_heads(qkv, batch, seq, heads)
    o = np.empty_like(q)
    a = np.empty_like(q)
    lse = np.empty(q.shape[:3])
    for b in range(batch):
        for h in range(heads):
            o[b, h], lse[b, h], a[b, h] = head_fwd(q[b, h], k[b, h], v[b, h])
    return merge_heads(o), lse, merge_heads(a)


def attention_bwd(qkv, ctx, dctx, batch, seq, heads):
    """Whole backward: returns dqkv [B*S][3*H*D] fp64 and the matching
    absolute-term sums T [B*S][3*H*D].  ctx is the forward output as saved
    (bf16 bits or float), dctx the incoming gradient."""
    q, k, v = split_heads(qkv, batch, seq, heads)
    hd = q.shape[1] * q.shape[3]
    o = split_heads(np.concatenate([np.asarray(ctx)] * 3, axis=1), batch, seq, heads)[0]
    do = split_heads(np.concatenate([np.asarray(dctx)] * 3, axis=1), batch, seq, heads)[0]
    dq, dk, dv = (np.empty_like(q) for _ in range(3))
    tq, tk, tv = (np.empty_like(q) for _ in range(3))
    for b in range(batch):
        for h in range(heads):
            g = head_bwd(q[b, h], k[b, h], v[b, h], o[b, h], do[b, h])
            dq[b, h], dk[b, h], dv[b, h] = g["dq"], g["dk"], g["dv"]
            tq[b, h], tk[b, h], tv[b, h] = g["tq"], g["tk"], g["tv"]
    d = np.concatenate([merge_heads(dq), merge_heads(dk), merge_heads(dv)], axis=1)
    t = np.concatenate([merge_heads(tq), merge_heads(tk), merge_heads(tv)], axis=1)
    assert d.shape[1] == 3 * hd
    return d, t
