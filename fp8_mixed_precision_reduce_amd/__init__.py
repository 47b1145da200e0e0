"""Python binding of libfp8lin.so, the MI355X FP8 linear layer with per-tensor
delayed scaling.

Argument marshalling only: each function takes torch tensors that already live
on the GPU, passes their data pointers, sizes and the current HIP stream to the
C entry point of the same name (include/fp8lin.h) and raises Fp8LinError on a
non-zero status.  Every step of the computation runs in the library's HIP
kernels; torch only provides device memory and streams.

The library must be built (python fp8_mixed_precision_reduce_amd/build.py or
__graft_entry__.build()); importing this package without it raises
ImportError -- there is no fallback.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8lin.so")

# ---- constants mirrored from include/fp8lin.h
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_ARG, ERR_HIP, ERR_UNSUPPORTED = range(8)
F32, BF16, E4M3, E5M2 = 0, 1, 2, 3
FORMAT_E4M3, FORMAT_HYBRID = 0, 1
AMAX_MAX = 0
EPI_GELU, EPI_ACCUMULATE, EPI_FAST_ACCUM = 1, 2, 4
KIND_NAMES = ["amax", "cast", "cast_transpose", "dequant", "scale_update", "gemm", "dbias", "other", "sgd",
              "attention", "stream"]
ABI_VERSION = 5

FUNCTIONS = [
    "fp8lin_abi_version", "fp8lin_last_error", "fp8lin_status_name", "fp8lin_dbias_workspace_bytes",
    "fp8lin_count_saturation",
    "fp8_amax", "fp8_amax_scale_update", "fp8_scale_from_current_amax", "fp8_cast", "fp8_cast_transpose", "fp8_cast_transpose_dgelu",
    "fp8_cast_transpose_dbias_noalloc",
    "fp8_cast_transpose_dual", "fp8_cast_transpose_dual_update",
    "fp8_dequant", "fp8_gemm", "fp8_linear_fwd", "fp8_linear_bwd", "fp8_loss_scale_update",
    "fp8_loss_scale_apply", "fp8_sgd_step", "fp8_sgd_step_cast", "fp8lin_timing_enable", "fp8lin_timing_read", "fp8lin_clock_sample", "fp8lin_stream_probe",
    "bf16_attention_workspace_bytes", "bf16_attention_fwd", "bf16_attention_bwd",
]


class Fp8LinError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class Recipe(ctypes.Structure):
    """DelayedScaling recipe: format, amax history length, amax algorithm,
    margin, whether the layer GEMMs use the fast (FP8 matrix-core) sums, and
    whether the layer calls scale just in time (from the current amax)."""
    _fields_ = [("format", ctypes.c_int32), ("history_len", ctypes.c_int32),
                ("amax_compute_algo", ctypes.c_int32), ("margin", ctypes.c_int32),
                ("fast_accum", ctypes.c_int32), ("just_in_time", ctypes.c_int32)]

    def __init__(self, format=FORMAT_HYBRID, history_len=16, amax_compute_algo=AMAX_MAX, margin=0, fast_accum=0,
                 just_in_time=0):
        super().__init__(format, history_len, amax_compute_algo, margin, int(bool(fast_accum)),
                         int(bool(just_in_time)))


class _MetaC(ctypes.Structure):
    _fields_ = [("amax_history", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("scale_inv", ctypes.c_void_p)]


class _QOutC(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_void_p), ("q", ctypes.c_void_p), ("q_t", ctypes.c_void_p),
                ("fp8_dtype", ctypes.c_int32)]


class QOut:
    """An FP8 copy of a GEMM output, cast in the epilogue: the scale (device
    float tensor) of the tensor the output becomes, its codes q [m][n] and
    transposed codes q_t [n][m] (either may be None) and the format."""

    def __init__(self, scale, q=None, q_t=None, fmt=E4M3):
        self.scale, self.q, self.q_t, self.fmt = scale, q, q_t, fmt

    def c(self):
        return _QOutC(self.scale.data_ptr(), self.q.data_ptr() if self.q is not None else None,
                      self.q_t.data_ptr() if self.q_t is not None else None, self.fmt)


def _qref(q_out):
    return ctypes.byref(q_out.c()) if q_out is not None else None


class _SavedC(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("xq_t", ctypes.c_void_p), ("wq", ctypes.c_void_p),
                ("wq_t", ctypes.c_void_p), ("sinv", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python fp8_mixed_precision_reduce_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "fp8lin_abi_version": (I32, []),
        "fp8lin_last_error": (ctypes.c_char_p, []),
        "fp8lin_status_name": (ctypes.c_char_p, [I32]),
        "fp8lin_dbias_workspace_bytes": (I64, [I64, I64]),
        "fp8lin_count_saturation": (I32, [P, P]),
        "fp8_amax": (I32, [P, I32, I64, P, P]),
        "fp8_amax_scale_update": (I32, [P, P, P, P, I32, ctypes.POINTER(Recipe), P]),
        "fp8_scale_from_current_amax": (I32, [P, P, P, P, I32, ctypes.POINTER(Recipe), P]),
        "fp8_cast": (I32, [P, I32, I64, I32, P, P, P, P]),
        "fp8_cast_transpose": (I32, [P, I32, I64, I64, I32, P, P, P, P, P, P, P]),
        "fp8_cast_transpose_dgelu": (I32, [P, P, I32, I64, I64, I32, P, P, P, P, P, P, P, P]),
        "fp8_cast_transpose_dbias_noalloc": (I32, [P, I32, I64, I64, I32, P, P, P, P, P, P]),
        "fp8_cast_transpose_dual": (I32, [P, I32, I64, I64, P, P, P, P, P, P, P, P, P]),
        "fp8_cast_transpose_dual_update": (I32, [P, I32, I64, I64, P, P, P, P, P, P, P, ctypes.POINTER(Recipe), P,
                                                 P]),
        "fp8_dequant": (I32, [P, I32, I64, P, P, I32, P]),
        "fp8_gemm": (I32, [P, I32, P, I32, I64, I64, I64, P, P, P, I32, I32, P, I32, P, P, P, P, P]),
        "fp8_linear_fwd": (I32, [I64, I64, I64, P, I32, P, I32, P, I32, I32, P, I32, P, P, P, P,
                                 ctypes.POINTER(Recipe), ctypes.POINTER(_MetaC), ctypes.POINTER(_MetaC),
                                 ctypes.POINTER(_SavedC), P]),
        "fp8_linear_bwd": (I32, [I64, I64, I64, P, I32, P, P, ctypes.POINTER(Recipe), ctypes.POINTER(_MetaC),
                                 ctypes.POINTER(_SavedC), P, P, P, I32, P, P, I32, P, P, P]),
        "fp8_loss_scale_update": (I32, [P, I32, I64, P, I32, ctypes.c_float, ctypes.c_float, P]),
        "fp8_loss_scale_apply": (I32, [P, I32, I64, P, P, P]),
        "fp8_sgd_step": (I32, [P, P, I64, ctypes.c_float, P, P]),
        "fp8_sgd_step_cast": (I32, [P, P, I64, I64, ctypes.c_float, P, P, P, P, P, P]),
        "fp8lin_timing_enable": (I32, [I32]),
        "bf16_attention_workspace_bytes": (I64, [I64, I64, I64, I64, I32]),
        "bf16_attention_fwd": (I32, [P, I64, I64, I64, I64, P, P, P, P]),
        "bf16_attention_bwd": (I32, [P, P, P, P, I64, I64, I64, I64, P, P, P]),
        "fp8lin_timing_read": (I32, [P, P, I32]),
        "fp8lin_clock_sample": (I32, [P, I32, P]),
        "fp8lin_stream_probe": (I32, [P, P, I64, I32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.fp8lin_abi_version() != ABI_VERSION:
        raise ImportError(f"libfp8lin ABI {lib.fp8lin_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


_lib = _load()


def _status_name(s):
    return _lib.fp8lin_status_name(s).decode()


def _check(status):
    if status != OK:
        raise Fp8LinError(status, _lib.fp8lin_last_error().decode())


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"expected a float32 or bfloat16 tensor, got {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def library():
    """The loaded ctypes library (for callers that marshal raw pointers)."""
    return _lib


# ------------------------------------------------------------------- state

class Meta:
    """Delayed-scaling state of one tensor in device memory: amax history
    (float[L], slot 0 = current step), scale and scale_inv (start at 1)."""

    def __init__(self, history_len, fmt, device="cuda"):
        self.fmt = fmt
        self.amax_history = torch.zeros(history_len, dtype=torch.float32, device=device)
        self.scale = torch.ones(1, dtype=torch.float32, device=device)
        self.scale_inv = torch.ones(1, dtype=torch.float32, device=device)

    def c(self):
        return _MetaC(self.amax_history.data_ptr(), self.scale.data_ptr(), self.scale_inv.data_ptr())


class MetaBank:
    """The metas of n tensors in three contiguous buffers, so that one
    fp8_amax_scale_update call updates all of them."""

    def __init__(self, formats, history_len, device="cuda"):
        n = len(formats)
        self.formats = bytes(formats)
        self.history_len = history_len
        self.amax_history = torch.zeros(n, history_len, dtype=torch.float32, device=device)
        self.scale = torch.ones(n, dtype=torch.float32, device=device)
        self.scale_inv = torch.ones(n, dtype=torch.float32, device=device)

    def meta(self, i):
        m = Meta.__new__(Meta)
        m.fmt = self.formats[i]
        m.amax_history = self.amax_history[i]
        m.scale = self.scale[i:i + 1]
        m.scale_inv = self.scale_inv[i:i + 1]
        return m

    def update(self, recipe, stream=None):
        fp8_amax_scale_update(self.amax_history, self.scale, self.scale_inv, self.formats, recipe, stream)

    def count_saturation(self, enable=True):
        """Registers (enable) or removes one saturation counter per tensor:
        self.saturated[i] then accumulates the codes that tensor i's casts
        saturated (cleared by snapshot(clear=True))."""
        if enable:
            if getattr(self, "saturated", None) is None:
                self.saturated = torch.zeros(len(self.formats), dtype=torch.int32, device=self.scale.device)
            for i in range(len(self.formats)):
                count_saturation(self.amax_history[i], self.saturated[i:i + 1])
        else:
            for i in range(len(self.formats)):
                count_saturation(self.amax_history[i], None)
            self.saturated = None

    def __del__(self):
        # a registration must not outlive the slot and counter it names
        if getattr(self, "saturated", None) is not None:
            try:
                self.count_saturation(False)
            except Exception:
                pass

    def snapshot(self, names=None, clear=True):
        """Host copy of each tensor's amax slot 0 (between a step's casts and
        its update: that step's amax), scale and inverse scale (the ones the
        step's casts used) and, when counting, its saturated codes (cleared
        for the next step unless clear is False)."""
        amax = self.amax_history[:, 0].cpu().tolist()
        scale, sinv = self.scale.cpu().tolist(), self.scale_inv.cpu().tolist()
        sat = self.saturated.cpu().tolist() if getattr(self, "saturated", None) is not None else None
        if sat is not None and clear:
            self.saturated.zero_()
        names = names or [str(i) for i in range(len(self.formats))]
        return {n: {"amax": amax[i], "scale": scale[i], "scale_inv": sinv[i],
                    **({"saturated": sat[i]} if sat is not None else {})} for i, n in enumerate(names)}

    def scale_from_current(self, recipe, stream=None):
        fp8_scale_from_current_amax(self.amax_history, self.scale, self.scale_inv, self.formats, recipe, stream)

    def state_dict(self):
        """Host copies of the delayed-scaling state (histories, scales, inverse
        scales): the operator state that a checkpoint keeps."""
        return {"amax_history": self.amax_history.cpu().clone(), "scale": self.scale.cpu().clone(),
                "scale_inv": self.scale_inv.cpu().clone(), "formats": torch.tensor(list(self.formats), dtype=torch.uint8)}

    def load_state_dict(self, state):
        """Restores a state_dict in place (the metas handed out stay valid)."""
        if bytes(state["formats"].tolist()) != self.formats or tuple(state["amax_history"].shape) != tuple(
                self.amax_history.shape):
            raise ValueError("MetaBank.load_state_dict: formats or history shape differ")
        self.amax_history.copy_(state["amax_history"])
        self.scale.copy_(state["scale"])
        self.scale_inv.copy_(state["scale_inv"])


class Saved:
    """Buffers a forward pass leaves for its backward pass (FP8 copies of X
    and W, row-major and transposed, and their inverse scales)."""

    def __init__(self, m, n, k, device="cuda", transposes=True):
        u8 = dict(dtype=torch.uint8, device=device)
        self.xq = torch.empty(m, k, **u8)
        self.wq = torch.empty(n, k, **u8)
        self.xq_t = torch.empty(k, m, **u8) if transposes else None
        self.wq_t = torch.empty(k, n, **u8) if transposes else None
        self.sinv = torch.empty(2, dtype=torch.float32, device=device)

    def c(self):
        return _SavedC(self.xq.data_ptr(), self.xq_t.data_ptr() if self.xq_t is not None else None,
                       self.wq.data_ptr(), self.wq_t.data_ptr() if self.wq_t is not None else None,
                       self.sinv.data_ptr())


# ------------------------------------------------------------ entry points

def count_saturation(amax_slot, counter):
    """Registers a device int32 counter (one element; None unregisters) for
    the casts that use amax_slot (a tensor whose first float is the slot, e.g.
    a meta's amax_history): they add the number of elements they saturated."""
    if counter is not None and (counter.dtype != torch.int32 or counter.numel() < 1 or not counter.is_cuda):
        raise ValueError("count_saturation: counter must be a device int32 tensor")
    _check(_lib.fp8lin_count_saturation(_p(amax_slot), _p(counter)))


def fp8_amax(x, amax_slot, stream=None):
    _check(_lib.fp8_amax(_p(x), _dt(x), x.numel(), _p(amax_slot), _stream(stream)))


def _check_metas(amax_history, scale, scale_inv, formats, recipe, what):
    """The C call takes the history length from the recipe and the tensor count
    from the formats: the buffers must hold exactly that many floats (the
    kernel would otherwise read and roll past the end of the history)."""
    n, L = len(formats), recipe.history_len
    if tuple(amax_history.shape) not in ((n, L),) + (((L,),) if n == 1 else ()) or not amax_history.is_contiguous():
        raise ValueError(f"{what}: amax_history has shape {tuple(amax_history.shape)}, expected a contiguous "
                         f"({n}, {L}) for {n} tensors and recipe.history_len {L}")
    for name, t in (("scale", scale), ("scale_inv", scale_inv)):
        if t.numel() != n or t.dtype != torch.float32:
            raise ValueError(f"{what}: {name} must hold {n} float32 values")
    if amax_history.dtype != torch.float32:
        raise ValueError(f"{what}: amax_history must be float32")


def fp8_amax_scale_update(amax_history, scale, scale_inv, formats, recipe, stream=None):
    _check_metas(amax_history, scale, scale_inv, formats, recipe, "fp8_amax_scale_update")
    fm = (ctypes.c_uint8 * len(formats)).from_buffer_copy(bytes(formats))
    _check(_lib.fp8_amax_scale_update(_p(amax_history), _p(scale), _p(scale_inv), ctypes.cast(fm, ctypes.c_void_p),
                                      len(formats), ctypes.byref(recipe), _stream(stream)))


def fp8_scale_from_current_amax(amax_history, scale, scale_inv, formats, recipe, stream=None):
    _check_metas(amax_history, scale, scale_inv, formats, recipe, "fp8_scale_from_current_amax")
    fm = (ctypes.c_uint8 * len(formats)).from_buffer_copy(bytes(formats))
    _check(_lib.fp8_scale_from_current_amax(_p(amax_history), _p(scale), _p(scale_inv),
                                            ctypes.cast(fm, ctypes.c_void_p), len(formats), ctypes.byref(recipe),
                                            _stream(stream)))


def fp8_cast(x, fmt, scale, q, amax_slot=None, stream=None):
    _check(_lib.fp8_cast(_p(x), _dt(x), x.numel(), fmt, _p(scale), _p(q), _p(amax_slot), _stream(stream)))


def fp8_cast_transpose(x, fmt, scale, q, q_t, amax_slot=None, dbias=None, dbias_ws=None, stream=None):
    rows, cols = x.shape
    _check(_lib.fp8_cast_transpose(_p(x), _dt(x), rows, cols, fmt, _p(scale), _p(q), _p(q_t), _p(amax_slot),
                                   _p(dbias), _p(dbias_ws), _stream(stream)))


def fp8_cast_transpose_dbias_noalloc(x, fmt, scale, q, q_t, dbias, amax_slot=None, stream=None):
    """fp8_cast_transpose with the bias gradient and no workspace: the library
    allocates nothing (its partial sums use a scratch array inside it)."""
    rows, cols = x.shape
    _check(_lib.fp8_cast_transpose_dbias_noalloc(_p(x), _dt(x), rows, cols, fmt, _p(scale), _p(q), _p(q_t),
                                                 _p(amax_slot), _p(dbias), _stream(stream)))


def fp8_cast_transpose_dgelu(dh, z, fmt, scale, q, q_t, amax_slot=None, dbias=None, dbias_ws=None, dz_out=None,
                             stream=None):
    rows, cols = dh.shape
    _check(_lib.fp8_cast_transpose_dgelu(_p(dh), _p(z), _dt(dh), rows, cols, fmt, _p(scale), _p(q), _p(q_t),
                                         _p(amax_slot), _p(dbias), _p(dbias_ws), _p(dz_out), _stream(stream)))


def fp8_cast_transpose_dual(x, scale_e4m3, scale_e5m2, q_e4m3=None, q_e4m3_t=None, q_e5m2=None, q_e5m2_t=None,
                            amax_slot_e4m3=None, amax_slot_e5m2=None, stream=None):
    rows, cols = x.shape
    _check(_lib.fp8_cast_transpose_dual(_p(x), _dt(x), rows, cols, _p(scale_e4m3), _p(q_e4m3), _p(q_e4m3_t),
                                        _p(amax_slot_e4m3), _p(scale_e5m2), _p(q_e5m2), _p(q_e5m2_t),
                                        _p(amax_slot_e5m2), _stream(stream)))


def fp8_cast_transpose_dual_update(x, bank, recipe, ticket, q_e4m3=None, q_e4m3_t=None, q_e5m2=None, q_e5m2_t=None,
                                   stream=None):
    """Dual-format cast-transpose into a two-tensor MetaBank (E4M3, E5M2) with
    the bank's scale update in the same launch; ticket: an int32 device
    tensor of one element, zero before the first call (left zero)."""
    if bank.formats != bytes([E4M3, E5M2]):
        raise ValueError("fp8_cast_transpose_dual_update: the bank must hold (E4M3, E5M2) metas")
    _check_metas(bank.amax_history, bank.scale, bank.scale_inv, bank.formats, recipe, "fp8_cast_transpose_dual_update")
    rows, cols = x.shape
    _check(_lib.fp8_cast_transpose_dual_update(_p(x), _dt(x), rows, cols, _p(q_e4m3), _p(q_e4m3_t), _p(q_e5m2),
                                               _p(q_e5m2_t), _p(bank.amax_history), _p(bank.scale),
                                               _p(bank.scale_inv), ctypes.byref(recipe), _p(ticket), _stream(stream)))


def fp8_dequant(q, fmt, scale_inv, out, stream=None):
    _check(_lib.fp8_dequant(_p(q), fmt, q.numel(), _p(scale_inv), _p(out), _dt(out), _stream(stream)))


def fp8_gemm(a, a_fmt, b, b_fmt, sinv_a, sinv_b, d, bias=None, epilogue=0, aux=None, residual=None, amax_d=None,
             q_out=None, stream=None):
    """d may be None when q_out is given (its values are still rounded to bf16)."""
    m, k = a.shape
    n = b.shape[0]
    bias_dt = _dt(bias) if bias is not None else F32
    d_dt = _dt(d) if d is not None else BF16
    _check(_lib.fp8_gemm(_p(a), a_fmt, _p(b), b_fmt, m, n, k, _p(sinv_a), _p(sinv_b), _p(bias), bias_dt, epilogue,
                         _p(d), d_dt, _p(aux), _p(residual), _p(amax_d), _qref(q_out), _stream(stream)))


def fp8_linear_fwd(x, w, y, recipe, mx, mw, saved, bias=None, epilogue=0, y_aux=None, residual=None,
                   y_amax_slot=None, y_q=None, stream=None):
    """x None: X's codes are already in saved (written by the producer's y_q).
    w None: W's codes are already in saved (written by fp8_sgd_step_cast).
    y None: only the FP8 copy y_q is written (y_dtype bf16)."""
    m, k = saved.xq.shape if x is None else x.shape
    n = saved.wq.shape[0] if w is None else w.shape[0]
    bias_dt = _dt(bias) if bias is not None else F32
    x_dt = _dt(x) if x is not None else BF16
    y_dt = _dt(y) if y is not None else BF16
    cx, cw, cs = mx.c(), mw.c(), saved.c()
    w_dt = _dt(w) if w is not None else F32
    _check(_lib.fp8_linear_fwd(m, n, k, _p(x), x_dt, _p(w), w_dt, _p(bias), bias_dt, epilogue, _p(y), y_dt,
                               _p(y_aux), _p(residual), _p(y_amax_slot), _qref(y_q), ctypes.byref(recipe),
                               ctypes.byref(cx), ctypes.byref(cw), ctypes.byref(cs), _stream(stream)))


def fp8_linear_bwd(dy, k, recipe, mdy, saved, dyq_ws=None, dyq_t_ws=None, dx=None, dw=None, accumulate_dw=False,
                   dbias=None, dbias_ws=None, gelu_z=None, dz_out=None, dx_residual=None, stream=None):
    m, n = dy.shape
    dx_dt = _dt(dx) if dx is not None else F32
    cm, cs = mdy.c(), saved.c()
    _check(_lib.fp8_linear_bwd(m, n, k, _p(dy), _dt(dy), _p(gelu_z), _p(dz_out), ctypes.byref(recipe),
                               ctypes.byref(cm), ctypes.byref(cs), _p(dyq_ws), _p(dyq_t_ws), _p(dx), dx_dt,
                               _p(dx_residual), _p(dw), int(bool(accumulate_dw)), _p(dbias), _p(dbias_ws),
                               _stream(stream)))


def fp8_loss_scale_update(grad_amaxes, state, stride=1, n=None, growth_interval=5, backoff=0.5, growth=2.0,
                          stream=None):
    """found_inf from n gradient amaxes (every `stride`-th float of
    grad_amaxes), then the dynamic loss-scale state float[4] update."""
    if n is None:
        n = (grad_amaxes.numel() + stride - 1) // stride
    _check(_lib.fp8_loss_scale_update(_p(grad_amaxes), n, stride, _p(state), growth_interval, backoff, growth,
                                      _stream(stream)))


def fp8_loss_scale_apply(g, state, out, stream=None):
    _check(_lib.fp8_loss_scale_apply(_p(g), _dt(g), g.numel(), _p(state), _p(out), _stream(stream)))


def fp8_sgd_step(w, g, lr, state, stream=None):
    if w.dtype != torch.float32 or g.dtype != torch.float32:
        raise TypeError("fp8_sgd_step: w and g must be float32")
    _check(_lib.fp8_sgd_step(_p(w), _p(g), w.numel(), lr, _p(state), _stream(stream)))


def fp8_sgd_step_cast(w, g, lr, state, scale, q, q_t, amax_slot=None, stream=None):
    """fp8_sgd_step on the fp32 weight matrix w [rows][cols] fused with its E4M3
    cast-transpose for the next forward (codes q [rows][cols] or None, q_t
    [cols][rows]; amax of the updated w max-merged into amax_slot)."""
    if w.dtype != torch.float32 or g.dtype != torch.float32 or w.dim() != 2 or g.shape != w.shape:
        raise TypeError("fp8_sgd_step_cast: w and g must be float32 matrices of one shape")
    rows, cols = w.shape
    _check(_lib.fp8_sgd_step_cast(_p(w), _p(g), rows, cols, lr, _p(state), _p(scale), _p(q), _p(q_t),
                                  _p(amax_slot), _stream(stream)))


def dbias_workspace_bytes(rows, cols):
    return _lib.fp8lin_dbias_workspace_bytes(rows, cols)


def timing_enable(capacity):
    _check(_lib.fp8lin_timing_enable(capacity))


def timing_read(max_records=1 << 16):
    """[(kind_name, ms), ...] of the launches recorded since timing_enable."""
    kinds = (ctypes.c_int32 * max_records)()
    ms = (ctypes.c_float * max_records)()
    n = _lib.fp8lin_timing_read(ctypes.cast(kinds, ctypes.c_void_p), ctypes.cast(ms, ctypes.c_void_p), max_records)
    return [(KIND_NAMES[kinds[i]], ms[i]) for i in range(n)]


def stream_probe(src, dst, mode, stream=None):
    """Streaming reference kernel over src's bytes: mode 0 reads them (dst: a
    device buffer of at least 8 KiB), mode 1 copies them into dst, mode 2
    copies them with non-temporal stores, modes 3 and 4 copy them twice (dst
    holds twice src's bytes), with plain and with non-temporal stores."""
    nbytes = src.numel() * src.element_size()
    _check(_lib.fp8lin_stream_probe(_p(src), _p(dst), nbytes, mode, _stream(stream)))


class ClockSample:
    """The shader clock while other work runs: start() enqueues the library's
    one-wave clock sample on a stream of its own (it waits wait_us of the
    constant 100 MHz counter), mhz() waits for it and returns the average
    shader clock over that window."""

    def __init__(self, device="cuda"):
        self.buf = torch.zeros(4, dtype=torch.int64, device=device)
        self.stream = torch.cuda.Stream(device=device)

    def start(self, wait_us):
        _check(_lib.fp8lin_clock_sample(_p(self.buf), int(wait_us), ctypes.c_void_p(self.stream.cuda_stream)))

    def mhz(self):
        self.stream.synchronize()
        c0, c1, r0, r1 = self.buf.cpu().tolist()
        return (c1 - c0) / max(r1 - r0, 1) * 100.0


# ------------------------------------------------------------- attention core

def attention_workspace_bytes(batch, seq, heads, head_dim=128, backward=False):
    """Bytes of device workspace bf16_attention_fwd (backward=False: V^T) or
    bf16_attention_bwd (Q^T, dO^T and the per-query rowsum(dO * O)) needs; -1
    for an unsupported shape."""
    return _lib.bf16_attention_workspace_bytes(batch, seq, heads, head_dim, int(bool(backward)))


def _attn_shape(qkv, batch, heads):
    if qkv.dtype != torch.bfloat16 or qkv.dim() != 2:
        raise TypeError("attention: qkv must be a 2-D bfloat16 tensor [batch*seq, 3*heads*head_dim]")
    tokens, cols = qkv.shape
    if tokens % batch or cols % (3 * heads):
        raise ValueError(f"attention: qkv shape {tuple(qkv.shape)} does not split into batch={batch}, heads={heads}")
    return tokens // batch, cols // (3 * heads)


def _check_workspace(workspace, batch, seq, heads, d, backward):
    """The library cannot see the workspace's size: an undersized one would be
    written past its end, so it is refused here."""
    need = attention_workspace_bytes(batch, seq, heads, d, backward)
    have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if need > 0 and have < need:
        raise ValueError(f"attention {'backward' if backward else 'forward'}: workspace of {have} bytes, "
                         f"needs {need} (attention_workspace_bytes)")


def bf16_attention_fwd(qkv, batch, heads, ctx, lse, workspace, stream=None):
    """ctx [batch*seq, heads*D] bf16 = softmax(Q K^T / sqrt(D)) V per (batch,
    head) from qkv [batch*seq, 3*heads*D] ([Q | K | V], head-major); lse
    float32 [batch, heads, seq] (base-2 log-sum-exp, kept for the backward);
    workspace: a uint8 device tensor of attention_workspace_bytes(...) bytes."""
    seq, d = _attn_shape(qkv, batch, heads)
    _check_workspace(workspace, batch, seq, heads, d, False)
    _check(_lib.bf16_attention_fwd(_p(qkv), batch, seq, heads, d, _p(ctx), _p(lse), _p(workspace), _stream(stream)))


def bf16_attention_bwd(qkv, ctx, lse, dctx, batch, heads, dqkv, workspace, stream=None):
    """dqkv [batch*seq, 3*heads*D] bf16 = the gradient of <ctx, dctx> with
    respect to qkv (all three parts written), from the forward's qkv, ctx, lse;
    workspace: a uint8 device tensor of attention_workspace_bytes(..., backward=True) bytes."""
    seq, d = _attn_shape(qkv, batch, heads)
    _check_workspace(workspace, batch, seq, heads, d, True)
    _check(_lib.bf16_attention_bwd(_p(qkv), _p(ctx), _p(lse), _p(dctx), batch, seq, heads, d, _p(dqkv),
                                   _p(workspace), _stream(stream)))
