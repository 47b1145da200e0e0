"""CPU oracle for the FP8 linear layer with per-tensor delayed scaling.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
the CPU-baseline leg of bench.py import this package.  The product library
(fp8_mixed_precision_reduce_amd) never imports it, and it never imports the
product library: the two share no code.

The arithmetic lives in oracle.c (plain C, fp64 where the pages leave the
precision open); this module only marshals numpy arrays and chains the plain
steps into a layer step in the order the pages give:

* [TE-KR] "FP8 자동변환(Autocasting)": inside an FP8 region every input is cast
  to FP8, its amax is recorded and its scaling factor is computed.
* [TE-KR] "Backward Pass 처리": the backward pass runs at the precision the
  forward pass fixed, i.e. on the FP8 copies and factors made in the forward.
* [PT-VI] (float8_experimental script): the amax/scale history update runs once
  per step, after backward and before the optimizer step.

Page tags are spelled out in oracle.h.  Functions whose result no pin fixes say
"parity unpinned" in their docstring.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2 = 0, 1
F32, BF16 = 0, 1
STYLE_IEEE, STYLE_FN = 0, 1
FORMAT_NAMES = {"e4m3": E4M3, "e5m2": E5M2}
FP8_MAX = {E4M3: 448.0, E5M2: 57344.0}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
    U8, U32, U16 = ctypes.c_uint8, ctypes.c_uint32, ctypes.c_uint16
    sig = {
        "orc_mf_encode": (U32, [F, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "orc_mf_decode": (D, [U32, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "orc_mf_max": (D, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "orc_mf_encode_array": (None, [P, I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]),
        "orc_mf_decode_array": (None, [P, I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]),
        "orc_bf16_from_f32_array": (None, [P, I64, P]),
        "orc_bf16_from_f64_array": (None, [P, I64, P]),
        "orc_f32_from_f64_array": (None, [P, I64, P]),
        "orc_fp8_max": (D, [ctypes.c_int]),
        "orc_decode": (D, [U8, ctypes.c_int]),
        "orc_encode": (U8, [F, ctypes.c_int]),
        "orc_encode_bruteforce": (U8, [F, ctypes.c_int]),
        "orc_encode_array": (None, [P, I64, ctypes.c_int, P]),
        "orc_encode_bits_range": (None, [ctypes.c_uint64, I64, ctypes.c_int, P]),
        "orc_encode_bruteforce_array": (None, [P, I64, ctypes.c_int, P]),
        "orc_bf16_from_f32": (U16, [F]),
        "orc_bf16_from_f64": (U16, [D]),
        "orc_f32_from_f64": (F, [D]),
        "orc_amax": (F, [P, ctypes.c_int, I64]),
        "orc_scale_update": (None, [P, P, P, P, I32, I32, I32]),
        "orc_cast": (None, [P, ctypes.c_int, I64, ctypes.c_int, F, P]),
        "orc_count_saturated": (I64, [P, ctypes.c_int, I64, ctypes.c_int, F]),
        "orc_cast_transpose": (None, [P, ctypes.c_int, I64, I64, ctypes.c_int, F, P, P]),
        "orc_transpose_u8": (None, [P, I64, I64, P]),
        "orc_dequant": (None, [P, ctypes.c_int, I64, F, P, ctypes.c_int]),
        "orc_colsum": (None, [P, ctypes.c_int, I64, I64, P]),
        "orc_gemm": (None, [P, ctypes.c_int, P, ctypes.c_int, I64, I64, I64, F, F, P, ctypes.c_int,
                            P, I64, P, P]),
        "orc_gemm_exact": (None, [P, ctypes.c_int, P, ctypes.c_int, I64, I64, I64, P, P, P]),
        "orc_gelu": (D, [D]),
        "orc_gelu_grad": (D, [D]),
        "orc_gelu_bwd": (None, [P, P, ctypes.c_int, I64, P]),
        "orc_num_threads": (ctypes.c_int, []),
        "orc_loss_scale_update": (None, [P, I32, I64, P, I32, F, F]),
        "orc_sgd": (None, [P, P, I64, F, P]),
        "orc_scale_by": (None, [P, ctypes.c_int, I64, F, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:          # bf16 bit patterns
        return BF16
    raise TypeError(f"oracle takes float32 or bf16-as-uint16 arrays, got {a.dtype}")


def _c(a):
    return np.ascontiguousarray(a)


def num_threads():
    return _load().orc_num_threads()


# ---------------------------------------------------------------- codec ----

def mf_encode(p, ebits, mbits, style, saturate):
    return _load().orc_mf_encode(float(np.float32(p)), ebits, mbits, style, saturate)


def mf_decode(code, ebits, mbits, style):
    return _load().orc_mf_decode(int(code), ebits, mbits, style)


def mf_max(ebits, mbits, style):
    return _load().orc_mf_max(ebits, mbits, style)


def fp8_max(fmt):
    return _load().orc_fp8_max(fmt)


def decode(code, fmt):
    return _load().orc_decode(int(code), fmt)


def decode_table(fmt):
    """fp64 value of each of the 256 codes."""
    lib = _load()
    return np.array([lib.orc_decode(c, fmt) for c in range(256)], dtype=np.float64)


def encode(p, fmt):
    return _load().orc_encode(float(np.float32(p)), fmt)


def encode_bruteforce(p, fmt):
    return _load().orc_encode_bruteforce(float(np.float32(p)), fmt)


def encode_array(p, fmt):
    p = _c(np.asarray(p, dtype=np.float32))
    out = np.empty(p.shape, dtype=np.uint8)
    _load().orc_encode_array(_ptr(p), p.size, fmt, _ptr(out))
    return out


def encode_bits_range(first_bits, n, fmt):
    """Codes of the fp32 values whose bit patterns are first_bits .. first_bits+n-1."""
    out = np.empty(n, dtype=np.uint8)
    _load().orc_encode_bits_range(first_bits, n, fmt, _ptr(out))
    return out


def encode_bruteforce_array(p, fmt):
    p = _c(np.asarray(p, dtype=np.float32))
    out = np.empty(p.shape, dtype=np.uint8)
    _load().orc_encode_bruteforce_array(_ptr(p), p.size, fmt, _ptr(out))
    return out


def mf_encode_array(p, ebits, mbits, style, saturate):
    p = _c(np.asarray(p, dtype=np.float32))
    out = np.empty(p.shape, dtype=np.uint32)
    _load().orc_mf_encode_array(_ptr(p), p.size, ebits, mbits, style, saturate, _ptr(out))
    return out


def mf_decode_array(codes, ebits, mbits, style):
    codes = _c(np.asarray(codes, dtype=np.uint32))
    out = np.empty(codes.shape, dtype=np.float64)
    _load().orc_mf_decode_array(_ptr(codes), codes.size, ebits, mbits, style, _ptr(out))
    return out


def bf16_from_f32(v):
    """bf16 bit patterns (uint16) of fp32 values, RNE."""
    v = _c(np.asarray(v, dtype=np.float32))
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_bf16_from_f32_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_from_f64(v):
    """bf16 bit patterns of fp64 values, one RNE rounding."""
    v = _c(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_bf16_from_f64_array(_ptr(v), v.size, _ptr(out))
    return out


def f32_from_f64(v):
    """fp32 values of fp64 values, one RNE rounding (through the generic codec)."""
    v = _c(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.float32)
    _load().orc_f32_from_f64_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f64(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------- amax, scale, history ----

def amax(x):
    x = _c(x)
    return np.float32(_load().orc_amax(_ptr(x), _dtype_code(x), x.size))


def scale_update(hist, scale, scale_inv, fmts, margin=0):
    """In place: hist float32 [n][L], scale/scale_inv float32 [n], fmts uint8 [n]."""
    for a in (hist, scale, scale_inv):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    fmts = _c(np.asarray(fmts, dtype=np.uint8))
    n, L = hist.shape
    _load().orc_scale_update(_ptr(hist), _ptr(scale), _ptr(scale_inv), _ptr(fmts), n, L, margin)


# ------------------------------------------------------ cast / dequant ----

def cast(x, fmt, scale):
    x = _c(x)
    q = np.empty(x.shape, dtype=np.uint8)
    _load().orc_cast(_ptr(x), _dtype_code(x), x.size, fmt, float(np.float32(scale)), _ptr(q))
    return q


def count_saturated(x, fmt, scale):
    """Number of elements whose fp32 product with scale exceeds the format's
    largest finite magnitude (the ones the saturating cast clamps; NaN not
    counted) -- [TE-KR] "정확도(Precision)"."""
    x = _c(x)
    return int(_load().orc_count_saturated(_ptr(x), _dtype_code(x), x.size, fmt, float(np.float32(scale))))


def cast_transpose(x, fmt, scale):
    x = _c(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    qt = np.empty((cols, rows), dtype=np.uint8)
    _load().orc_cast_transpose(_ptr(x), _dtype_code(x), rows, cols, fmt, float(np.float32(scale)),
                               _ptr(q), _ptr(qt))
    return q, qt


def transpose_u8(q):
    q = _c(q)
    rows, cols = q.shape
    qt = np.empty((cols, rows), dtype=np.uint8)
    _load().orc_transpose_u8(_ptr(q), rows, cols, _ptr(qt))
    return qt


def dequant(q, fmt, scale_inv, out_dtype=F32):
    q = _c(q)
    out = np.empty(q.shape, dtype=np.float32 if out_dtype == F32 else np.uint16)
    _load().orc_dequant(_ptr(q), fmt, q.size, float(np.float32(scale_inv)), _ptr(out), out_dtype)
    return out


def colsum(x):
    x = _c(x)
    rows, cols = x.shape
    out = np.empty(cols, dtype=np.float64)
    _load().orc_colsum(_ptr(x), _dtype_code(x), rows, cols, _ptr(out))
    return out


# ----------------------------------------------------------------- GEMM ----

def gemm(a, afmt, b, bfmt, sinv_a=1.0, sinv_b=1.0, bias=None, gelu=False, rows=None, want_pre=False):
    """y[i][j] = sum_k dec(a[i,k]) dec(b[j,k]) * sinv_a * sinv_b (+ bias[j]), optional GeLU.

    Returns fp64 values before the output rounding (and y before GeLU if want_pre).
    """
    a, b = _c(a), _c(b)
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    if bias is not None:
        bias = _c(np.asarray(bias, dtype=np.float64))
    if rows is not None:
        rows = _c(np.asarray(rows, dtype=np.int64))
        nr = rows.size
    else:
        nr = m
    out = np.empty((nr, n), dtype=np.float64)
    pre = np.empty((nr, n), dtype=np.float64) if want_pre else None
    _load().orc_gemm(_ptr(a), afmt, _ptr(b), bfmt, m, n, k, float(np.float32(sinv_a)),
                     float(np.float32(sinv_b)), _ptr(bias), int(bool(gelu)),
                     _ptr(rows), nr, _ptr(pre), _ptr(out))
    return (out, pre) if want_pre else out


def gemm_exact(a, afmt, b, bfmt):
    """Exact D = A_dec @ B_dec^T as Python ints times 2**exp2 (small operands only)."""
    a, b = _c(a), _c(b)
    m, k = a.shape
    n, _ = b.shape
    hi = np.empty((m, n), dtype=np.int64)
    lo = np.empty((m, n), dtype=np.uint64)
    e = np.zeros(1, dtype=np.int32)
    _load().orc_gemm_exact(_ptr(a), afmt, _ptr(b), bfmt, m, n, k, _ptr(hi), _ptr(lo), _ptr(e))
    ints = [[(int(hi[i, j]) << 64) + int(lo[i, j]) for j in range(n)] for i in range(m)]
    return ints, int(e[0])


def gelu(z):
    return _load().orc_gelu(float(z))


def gelu_grad(z):
    return _load().orc_gelu_grad(float(z))


def gelu_bwd(dh, z):
    """dz = round(dh * gelu'(z)) in fp64, rounded once to dh's element type."""
    dh, z = _c(dh), _c(z)
    assert dh.dtype == z.dtype and dh.shape == z.shape
    out = np.empty(dh.shape, dtype=dh.dtype)
    _load().orc_gelu_bwd(_ptr(dh), _ptr(z), _dtype_code(dh), dh.size, _ptr(out))
    return out


def round_out(y, out_dtype):
    """Round fp64 GEMM results to the output type: fp32 or bf16 bits (RNE)."""
    if out_dtype == F32:
        return f32_from_f64(y)
    return bf16_from_f64(y)


# ------------------------------------------------- layer composition ----

class Meta:
    """Per-tensor delayed-scaling state: amax history (logical order, slot 0 =
    current step), scale and inverse scale; starts at zeros and scale 1."""

    def __init__(self, hist_len, fmt):
        self.hist = np.zeros(hist_len, dtype=np.float32)
        self.scale = np.float32(1.0)
        self.scale_inv = np.float32(1.0)
        self.fmt = fmt

    def record(self, x):
        """Max-merge amax(x) into slot 0 (as unsigned bit patterns, like the amax itself)."""
        a = np.array([amax(x)], dtype=np.float32).view(np.uint32)[0]
        cur = self.hist[0:1].view(np.uint32)
        cur[0] = max(int(cur[0]), int(a))

    def copy(self):
        m = Meta(self.hist.size, self.fmt)
        m.hist = self.hist.copy()
        m.scale, m.scale_inv = np.float32(self.scale), np.float32(self.scale_inv)
        return m


def update_metas(metas, margin=0):
    """One delayed-scaling update over several metas (the per-step call)."""
    n, L = len(metas), metas[0].hist.size
    hist = np.stack([m.hist for m in metas]).astype(np.float32)
    scale = np.array([m.scale for m in metas], dtype=np.float32)
    sinv = np.array([m.scale_inv for m in metas], dtype=np.float32)
    scale_update(hist, scale, sinv, [m.fmt for m in metas], margin)
    for i, m in enumerate(metas):
        m.hist = hist[i].copy()
        m.scale, m.scale_inv = np.float32(scale[i]), np.float32(sinv[i])


def scale_from_current(meta, margin=0):
    """Just-in-time scaling ([TE-KR] "Scaling factor" strategy: the factor from
    the amax measured at this use): the scale rule applied to the current amax
    alone (slot 0), i.e. the delayed update over a one-entry history, without
    rolling the tensor's history."""
    h = meta.hist[0:1].astype(np.float32).reshape(1, 1).copy()
    sc = np.array([meta.scale], dtype=np.float32)
    si = np.array([meta.scale_inv], dtype=np.float32)
    scale_update(h, sc, si, [meta.fmt], margin)
    meta.scale, meta.scale_inv = np.float32(sc[0]), np.float32(si[0])


def linear_fwd(x, w, mx, mw, bias=None, gelu_=False, rows=None, jit=False):
    """Forward of Y = X W^T + b on FP8 copies of X and W.

    Records amax(X), amax(W) in slot 0, casts both with their current scales
    (with jit: scales taken from those amaxes first) to E4M3 (forward format),
    runs the FP8 GEMM with fp64 accumulation and returns a dict with the
    codes, the inverse scales captured for backward and the fp64 result (y
    before GeLU in 'pre' when gelu_).
    """
    mx.record(x)
    mw.record(w)
    if jit:
        scale_from_current(mx)
        scale_from_current(mw)
    xq, xqt = cast_transpose(x, mx.fmt, mx.scale)
    wq, wqt = cast_transpose(w, mw.fmt, mw.scale)
    b64 = None if bias is None else np.asarray(bias, dtype=np.float32).astype(np.float64)
    y, pre = gemm(xq, mx.fmt, wq, mw.fmt, mx.scale_inv, mw.scale_inv, b64, gelu_, rows, want_pre=True)
    return dict(xq=xq, xqt=xqt, wq=wq, wqt=wqt, sinv_x=np.float32(mx.scale_inv),
                sinv_w=np.float32(mw.scale_inv), fmt_x=mx.fmt, fmt_w=mw.fmt, y=y, pre=pre)


def linear_bwd(dy, saved, mg, rows_dx=None, rows_dw=None, jit=False):
    """Backward of the FP8 linear from the forward's saved FP8 copies.

    Records amax(dY), casts dY with its current scale (with jit: the scale
    taken from that amax first; E5M2 under HYBRID),
    then dX = dYq . Wq (reduction over N, operands dYq [M][N] and Wq^T [K][N])
    and dW = dYq^T . Xq (reduction over M, operands dYq^T [N][M], Xq^T [K][M]).
    dbias = column sums of dY in fp64.
    """
    mg.record(dy)
    if jit:
        scale_from_current(mg)
    gq, gqt = cast_transpose(dy, mg.fmt, mg.scale)
    dx = gemm(gq, mg.fmt, saved["wqt"], saved["fmt_w"], mg.scale_inv, saved["sinv_w"], rows=rows_dx)
    dw = gemm(gqt, mg.fmt, saved["xqt"], saved["fmt_x"], mg.scale_inv, saved["sinv_x"], rows=rows_dw)
    return dict(gq=gq, gqt=gqt, sinv_g=np.float32(mg.scale_inv), dx=dx, dw=dw, dbias=colsum(dy))


def mlp_step(x, w1, w2, dy, metas, rows_w=None):
    """One forward + backward step of the FP8 MLP block FC1 -> GeLU -> FC2
    (no biases), HYBRID formats, followed by the delayed-scaling update.

    x [m][h], w1 [f][h], w2 [h][f], dy [m][h] as bf16 bit patterns (uint16);
    metas: dict of Meta for 'x', 'w1', 'h', 'w2', 'dy', 'dz'.  The GeLU output
    H, its input Z, dH and dZ are rounded to bf16 between the steps, as the
    layer stores them.  rows_w (optional) restricts the weight-gradient rows
    that are computed.  Returns every intermediate.
    """
    fw1 = linear_fwd(x, w1, metas["x"], metas["w1"], gelu_=True)
    h = bf16_from_f64(fw1["y"])
    z = bf16_from_f64(fw1["pre"])
    fw2 = linear_fwd(h, w2, metas["h"], metas["w2"])
    bw2 = linear_bwd(dy, fw2, metas["dy"], rows_dw=rows_w)
    dh = bf16_from_f64(bw2["dx"])
    dz = gelu_bwd(dh, z)
    bw1 = linear_bwd(dz, fw1, metas["dz"], rows_dw=rows_w)
    update_metas([metas[k] for k in ("x", "w1", "h", "w2", "dy", "dz")])
    return dict(fw1=fw1, fw2=fw2, bw1=bw1, bw2=bw2, h=h, z=z, y=bf16_from_f64(fw2["y"]), dh=dh, dz=dz,
                dx=bf16_from_f64(bw1["dx"]), dw1=bw1["dw"], dw2=bw2["dw"])


def mlp_metas(hist_len):
    return {"x": Meta(hist_len, E4M3), "w1": Meta(hist_len, E4M3), "h": Meta(hist_len, E4M3),
            "w2": Meta(hist_len, E4M3), "dy": Meta(hist_len, E5M2), "dz": Meta(hist_len, E5M2)}


# ------------------------------------------- transformer layer step ----
#
# The four FP8 linears of a transformer layer (QKV, attention output, FC1,
# FC2) with the fp32 master weights, dynamic loss scaling and SGD.  The pages
# do not spell out a layer's wiring; this step reads it as the plainest
# pre-norm-free block: Y1 = X + O(ctx), Y = Y1 + FC2(gelu(FC1(Y1))), where ctx
# stands in for the bf16 attention core's output (it is an input here, as is
# the gradient d(QKV) the attention core would return).  All activations and
# activation gradients are stored in bf16, the weight gradients in fp32.

LAYER_TENSORS = ("x", "wqkv", "ctx", "wo", "y1", "w1", "h", "w2", "g_fc2", "g_fc1", "g_o", "g_qkv")
LAYER_GRADS = ("g_fc2", "g_fc1", "g_o", "g_qkv")
LAYER_WEIGHTS = ("wqkv", "wo", "w1", "w2")


def layer_metas(hist_len):
    return {name: Meta(hist_len, E5M2 if name.startswith("g_") else E4M3) for name in LAYER_TENSORS}


def add_residual(y64, r):
    """fp64 GEMM result plus a residual stored as bf16 bits (or fp32)."""
    r = np.asarray(r)
    r64 = bf16_to_f64(r) if r.dtype == np.uint16 else r.astype(np.float64)
    return y64 + r64


def layer_step(x, ctx, g, dqkv, masters, metas, loss_scale, lr):
    """One training step of the FP8 layer: forward, loss-scaled backward, the
    found-inf check and loss-scale update ([MP-KR] dynamic loss scaling: an
    Inf/NaN gradient lowers S and skips the update), the delayed-scaling
    update of all twelve FP8 tensors ([PT-VI]: once per step after backward,
    before the optimizer), and SGD on the fp32 masters ([MP-KR] "FP32 Master
    Copy of Weights": the weight gradient is unscaled by 1/S).

    x, ctx, g [m][h] and dqkv [m][3h] are bf16 bits; masters: dict of float32
    arrays wqkv [3h][h], wo [h][h], w1 [f][h], w2 [h][f], updated in place.
    The weights are cast from their fp32 masters straight to E4M3.  The loss is
    <Y, G> * S, so the gradient entering FC2 is dY = bf16(G * S); the stand-in
    attention-core gradient enters the QKV linear as bf16(dqkv * S).
    """
    S = np.float32(loss_scale.state[0])
    fq = linear_fwd(x, masters["wqkv"], metas["x"], metas["wqkv"])
    qkv = bf16_from_f64(fq["y"])
    fo = linear_fwd(ctx, masters["wo"], metas["ctx"], metas["wo"])
    y1 = bf16_from_f64(add_residual(fo["y"], x))
    f1 = linear_fwd(y1, masters["w1"], metas["y1"], metas["w1"], gelu_=True)
    h, z = bf16_from_f64(f1["y"]), bf16_from_f64(f1["pre"])
    f2 = linear_fwd(h, masters["w2"], metas["h"], metas["w2"])
    y = bf16_from_f64(add_residual(f2["y"], y1))

    dy = scale_by(g, S)
    b2 = linear_bwd(dy, f2, metas["g_fc2"])
    dh = bf16_from_f64(b2["dx"])
    dz = gelu_bwd(dh, z)
    b1 = linear_bwd(dz, f1, metas["g_fc1"])
    dy1 = bf16_from_f64(add_residual(b1["dx"], dy))          # FC branch + the skip path
    bo = linear_bwd(dy1, fo, metas["g_o"])
    dctx = bf16_from_f64(bo["dx"])
    dq = scale_by(dqkv, S)
    bq = linear_bwd(dq, fq, metas["g_qkv"])
    dx = bf16_from_f64(add_residual(bq["dx"], dy1))          # QKV branch + the skip path

    grads = {"wqkv": f32_from_f64(bq["dw"]), "wo": f32_from_f64(bo["dw"]), "w1": f32_from_f64(b1["dw"]),
             "w2": f32_from_f64(b2["dw"])}
    loss_scale.update([metas[n].hist[0] for n in LAYER_GRADS])
    update_metas([metas[n] for n in LAYER_TENSORS])
    for name in LAYER_WEIGHTS:
        sgd(masters[name], grads[name], lr, loss_scale)
    return dict(qkv=qkv, y1=y1, h=h, z=z, y=y, dy=dy, dh=dh, dz=dz, dy1=dy1, dctx=dctx, dqkv=dq, dx=dx,
                grads=grads, fwd=dict(qkv=fq, o=fo, fc1=f1, fc2=f2), bwd=dict(qkv=bq, o=bo, fc1=b1, fc2=b2))


# ------------------------------------------------- loss scaling and SGD ----

class LossScale:
    """Dynamic loss-scale state: [S, clean iterations, found_inf, S of the last step]."""

    def __init__(self, s0=65536.0, interval=5, backoff=0.5, growth=2.0):
        self.state = np.array([s0, 0.0, 0.0, s0], dtype=np.float32)
        self.interval, self.backoff, self.growth = interval, backoff, growth

    def update(self, grad_amaxes):
        a = _c(np.asarray(grad_amaxes, dtype=np.float32))
        _load().orc_loss_scale_update(_ptr(a), a.size, 1, _ptr(self.state), self.interval, float(self.backoff),
                                      float(self.growth))

    @property
    def found_inf(self):
        return bool(self.state[2])


def sgd(w, g, lr, loss_scale):
    """In place on float32 w: w -= lr * g / S (skipped after a found_inf step)."""
    assert w.dtype == np.float32 and w.flags.c_contiguous
    g = _c(np.asarray(g, dtype=np.float32))
    _load().orc_sgd(_ptr(w), _ptr(g), w.size, float(np.float32(lr)), _ptr(loss_scale.state))


def scale_by(x, s):
    """round(x * s) in x's element type (the loss-scaled gradient)."""
    x = _c(x)
    out = np.empty(x.shape, dtype=x.dtype)
    _load().orc_scale_by(_ptr(x), _dtype_code(x), x.size, float(np.float32(s)), _ptr(out))
    return out
