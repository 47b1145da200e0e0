"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects invalid arguments on the host before launching
anything (so these checks need no device)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

F = pytest.importorskip("fp8_mixed_precision_reduce_amd")
L = F.library()
P = ctypes.c_void_p

A16 = P(1 << 20)          # fake, 16-byte aligned device addresses (never dereferenced)
B16 = P(1 << 24)
C16 = P(1 << 28)
ODD = P((1 << 20) + 4)    # 4-byte aligned, not 16-byte aligned


def _header_functions():
    text = open(os.path.join(ROOT, "include", "fp8lin.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?((?:fp8|bf16)\w*)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function():
    names = _header_functions()
    assert len(names) >= 13
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(F.FUNCTIONS)


def test_abi_version_and_status_names():
    assert L.fp8lin_abi_version() == 5
    assert L.fp8lin_status_name(0) == b"FP8LIN_OK"
    assert L.fp8lin_status_name(2) == b"FP8LIN_ERR_SHAPE"
    assert L.fp8lin_status_name(99) == b"FP8LIN_UNKNOWN_STATUS"


def test_dbias_workspace_size():
    assert L.fp8lin_dbias_workspace_bytes(0, 64) == 0
    assert L.fp8lin_dbias_workspace_bytes(128, 64) == 64 * 4
    assert L.fp8lin_dbias_workspace_bytes(1024, 768) == 8 * 768 * 4


def _err(status):
    assert status != 0
    assert L.fp8lin_last_error()        # a message is left for the caller
    return status


def test_amax_and_cast_validation():
    assert _err(L.fp8_amax(A16, 7, 16, B16, None)) == F.ERR_DTYPE
    assert _err(L.fp8_amax(A16, F.F32, -1, B16, None)) == F.ERR_SHAPE
    assert _err(L.fp8_amax(None, F.F32, 16, B16, None)) == F.ERR_NULL
    assert _err(L.fp8_amax(ODD, F.F32, 16, B16, None)) == F.ERR_ALIGN
    assert L.fp8_amax(A16, F.F32, 0, B16, None) == F.OK                  # empty: nothing to do
    assert _err(L.fp8_cast(A16, F.F32, 16, F.F32, B16, C16, None, None)) == F.ERR_DTYPE
    assert _err(L.fp8_cast(A16, F.BF16, 16, F.E4M3, None, C16, None, None)) == F.ERR_NULL
    assert _err(L.fp8_cast(A16, F.F32, 64, F.E4M3, B16, P((1 << 20) + 16), None, None)) == F.ERR_ARG  # overlap
    assert L.fp8_cast(A16, F.F32, 0, F.E5M2, B16, C16, None, None) == F.OK


def test_cast_transpose_validation():
    ct = L.fp8_cast_transpose
    assert _err(ct(A16, F.BF16, 17, 32, F.E4M3, B16, C16, P(1 << 30), None, None, None, None)) == F.ERR_SHAPE
    assert _err(ct(A16, F.BF16, 32, 24, F.E4M3, B16, C16, P(1 << 30), None, None, None, None)) == F.ERR_SHAPE
    # the kernels' 32-bit tile offsets: rows < 2^24, cols < 2^22 (checked before any pointer is used)
    assert _err(ct(A16, F.BF16, 16, 1 << 22, F.E4M3, B16, C16, P(1 << 30), None, None, None, None)) == F.ERR_SHAPE
    assert _err(ct(A16, F.BF16, 1 << 24, 16, F.E4M3, B16, C16, P(1 << 30), None, None, None, None)) == F.ERR_SHAPE
    assert _err(L.fp8_cast_transpose_dgelu(A16, B16, F.BF16, 16, 1 << 22, F.E4M3, C16, P(1 << 29), P(1 << 30),
                                           None, None, None, None, None)) == F.ERR_SHAPE
    assert _err(ct(A16, F.BF16, 32, 32, F.E4M3, B16, C16, None, None, None, None, None)) == F.ERR_NULL
    assert _err(ct(A16, F.BF16, 32, 32, F.E4M3, B16, C16, P(1 << 30), None, P(1 << 31), None, None)) == F.ERR_NULL
    assert _err(ct(A16, F.BF16, 32, 32, F.E4M3, B16, ODD, P(1 << 30), None, None, None, None)) == F.ERR_ALIGN
    assert _err(ct(A16, F.BF16, 32, 32, F.E4M3, B16, C16, C16, None, None, None, None)) == F.ERR_ARG
    assert ct(A16, F.BF16, 0, 32, F.E4M3, B16, C16, P(1 << 30), None, None, None, None) == F.OK
    dg = L.fp8_cast_transpose_dgelu
    assert _err(dg(A16, None, F.BF16, 32, 32, F.E5M2, B16, C16, P(1 << 30), None, None, None, None, None)) == F.ERR_NULL


def test_cast_transpose_dual_validation():
    du = L.fp8_cast_transpose_dual
    s4, s5 = P(1 << 34), P((1 << 34) + 64)
    q4, q4t, q5, q5t = P(1 << 36), P(1 << 37), P(1 << 38), P(1 << 39)
    assert _err(du(A16, F.BF16, 17, 32, s4, q4, q4t, None, s5, q5, q5t, None, None)) == F.ERR_SHAPE
    assert _err(du(A16, F.E4M3, 32, 32, s4, q4, q4t, None, s5, q5, q5t, None, None)) == F.ERR_DTYPE
    assert _err(du(A16, F.BF16, 32, 32, s4, None, None, None, s5, None, None, None, None)) == F.ERR_NULL
    assert _err(du(A16, F.BF16, 32, 32, None, q4, q4t, None, s5, q5, q5t, None, None)) == F.ERR_NULL
    assert _err(du(A16, F.BF16, 32, 32, s4, q4, q4t, None, s5, P((1 << 36) + 512), q5t, None, None)) == F.ERR_ARG
    assert _err(du(A16, F.BF16, 32, 32, s4, q4, q4t, None, s5, q5, P((1 << 20) + 64), None, None)) == F.ERR_ARG
    assert _err(du(A16, F.BF16, 32, 32, s4, q4, ODD, None, s5, q5, q5t, None, None)) == F.ERR_ALIGN
    assert du(A16, F.BF16, 0, 32, s4, q4, q4t, None, s5, q5, q5t, None, None) == F.OK


def test_dequant_validation():
    assert _err(L.fp8_dequant(A16, F.BF16, 16, B16, C16, F.F32, None)) == F.ERR_DTYPE
    assert _err(L.fp8_dequant(A16, F.E4M3, 16, B16, C16, F.E5M2, None)) == F.ERR_DTYPE
    assert _err(L.fp8_dequant(A16, F.E4M3, 16, None, C16, F.F32, None)) == F.ERR_NULL
    assert L.fp8_dequant(A16, F.E4M3, 0, B16, C16, F.F32, None) == F.OK


def _gemm(m=64, n=64, k=64, a_dt=F.E4M3, b_dt=F.E4M3, d_dt=F.F32, epi=0, aux=None, bias=None, bias_dt=F.F32,
          d=P(1 << 30), sa=P(1 << 32), sb=P(1 << 33), residual=None, q_out=None):
    return L.fp8_gemm(A16, a_dt, B16, b_dt, m, n, k, sa, sb, bias, bias_dt, epi, d, d_dt, aux, residual, None, q_out,
                      None)


def test_gemm_validation():
    assert _err(_gemm(m=65)) == F.ERR_SHAPE
    assert _err(_gemm(k=1 << 23)) == F.ERR_SHAPE
    assert _err(_gemm(a_dt=F.F32)) == F.ERR_DTYPE
    assert _err(_gemm(d_dt=F.E4M3)) == F.ERR_DTYPE
    assert _err(_gemm(epi=8)) == F.ERR_ARG
    assert _err(_gemm(epi=3)) == F.ERR_ARG
    assert _err(_gemm(epi=2, d_dt=F.BF16)) == F.ERR_DTYPE
    assert _err(_gemm(aux=P(1 << 34))) == F.ERR_ARG                    # aux only with GELU
    assert _err(_gemm(sa=None)) == F.ERR_NULL
    assert _err(_gemm(d=P((1 << 20) + 8))) == F.ERR_ALIGN
    assert _err(_gemm(d=P((1 << 20) + 16))) == F.ERR_ARG               # d overlaps A
    assert _gemm(m=0) == F.OK


def test_gemm_residual_validation():
    d = 1 << 30
    assert _err(_gemm(d=P(d), residual=P(d + 16))) == F.ERR_ARG          # partial overlap with d
    assert _err(_gemm(d=P(d), residual=P(d + 8))) == F.ERR_ALIGN
    assert _err(_gemm(epi=F.EPI_ACCUMULATE, residual=P(1 << 34))) == F.ERR_ARG
    assert _err(_gemm(epi=F.EPI_GELU, aux=P(1 << 34), residual=P((1 << 34) + 64))) == F.ERR_ARG
    assert _gemm(m=0, residual=P(d)) == F.OK                              # in place (residual == d) is allowed


def _recipe(**kw):
    return F.Recipe(**kw)


def test_scale_update_validation():
    fm = (ctypes.c_uint8 * 2)(F.E4M3, F.E5M2)
    upd = L.fp8_amax_scale_update
    r = _recipe(history_len=16)
    assert _err(upd(A16, B16, C16, ctypes.cast(fm, P), 0, ctypes.byref(r), None)) == F.ERR_SHAPE
    assert _err(upd(A16, B16, C16, ctypes.cast(fm, P), 2, ctypes.byref(_recipe(history_len=0)), None)) == F.ERR_ARG
    assert _err(upd(A16, B16, C16, ctypes.cast(fm, P), 2, ctypes.byref(_recipe(margin=200)), None)) == F.ERR_ARG
    assert _err(upd(A16, B16, C16, ctypes.cast(fm, P), 2, ctypes.byref(_recipe(amax_compute_algo=1)),
                    None)) == F.ERR_UNSUPPORTED
    bad = (ctypes.c_uint8 * 2)(F.E4M3, F.F32)
    assert _err(upd(A16, B16, C16, ctypes.cast(bad, P), 2, ctypes.byref(r), None)) == F.ERR_DTYPE
    assert _err(upd(A16, A16, C16, ctypes.cast(fm, P), 2, ctypes.byref(r), None)) == F.ERR_ARG      # overlap
    assert _err(upd(None, B16, C16, ctypes.cast(fm, P), 2, ctypes.byref(r), None)) == F.ERR_NULL


def test_linear_validation():
    r = _recipe()
    meta = F._MetaC(1 << 36, (1 << 36) + 4096, (1 << 36) + 8192)
    saved = F._SavedC(1 << 37, 1 << 38, 1 << 39, 1 << 40, 1 << 41)
    fwd = L.fp8_linear_fwd
    args = [A16, F.F32, B16, F.F32, None, F.F32, 0, C16, F.F32, None, None, None, None, ctypes.byref(r), ctypes.byref(meta),
            ctypes.byref(meta), ctypes.byref(saved), None]
    assert _err(fwd(64, 64, 60, *args)) == F.ERR_SHAPE
    args_acc = list(args)
    args_acc[6] = F.EPI_ACCUMULATE
    assert _err(fwd(64, 64, 64, *args_acc)) == F.ERR_ARG
    no_saved = list(args)
    no_saved[16] = None
    assert _err(fwd(64, 64, 64, *no_saved)) == F.ERR_NULL
    bwd = L.fp8_linear_bwd
    saved_no_t = F._SavedC(1 << 37, None, 1 << 39, None, 1 << 41)
    assert _err(bwd(64, 64, 64, A16, F.F32, None, None, ctypes.byref(r), ctypes.byref(meta),
                    ctypes.byref(saved_no_t), B16, C16, P(1 << 42), F.F32, None, None, 0, None, None, None)) == F.ERR_NULL
    assert _err(bwd(64, 64, 64, A16, F.F32, None, P(1 << 42), ctypes.byref(r), ctypes.byref(meta),
                    ctypes.byref(saved), B16, C16, None, F.F32, None, None, 0, None, None, None)) == F.ERR_ARG
    # a residual gradient without dx
    assert _err(bwd(64, 64, 64, A16, F.F32, None, None, ctypes.byref(r), ctypes.byref(meta),
                    ctypes.byref(saved), B16, C16, None, F.F32, P(1 << 42), P(1 << 43), 0, None, None,
                    None)) == F.ERR_ARG
    # dx overlapping dy
    assert _err(bwd(64, 64, 64, A16, F.F32, None, None, ctypes.byref(r), ctypes.byref(meta),
                    ctypes.byref(saved), B16, C16, P((1 << 20) + 64), F.F32, None, None, 0, None, None,
                    None)) == F.ERR_ARG
    bad_fmt = _recipe(format=5)
    assert _err(bwd(64, 64, 64, A16, F.F32, None, None, ctypes.byref(bad_fmt), ctypes.byref(meta),
                    ctypes.byref(saved), B16, C16, None, F.F32, None, None, 0, None, None, None)) == F.ERR_ARG


def test_gemm_q_out_validation():
    qs = P(1 << 35)
    def q(scale=qs, qq=P(1 << 36), qt=P(1 << 37), fmt=F.E4M3):
        return ctypes.byref(F._QOutC(scale, qq, qt, fmt))
    assert _err(_gemm(d_dt=F.F32, q_out=q())) == F.ERR_UNSUPPORTED              # bf16 outputs only
    assert _err(_gemm(d_dt=F.BF16, q_out=q(fmt=F.BF16))) == F.ERR_DTYPE
    assert _err(_gemm(d_dt=F.BF16, q_out=q(scale=None))) == F.ERR_NULL
    assert _err(_gemm(d_dt=F.BF16, q_out=q(qq=None, qt=None))) == F.ERR_NULL
    assert _err(_gemm(d_dt=F.BF16, q_out=q(qq=P((1 << 36) + 8)))) == F.ERR_ALIGN
    assert _err(_gemm(d_dt=F.BF16, q_out=q(qq=P(1 << 30)))) == F.ERR_ARG          # codes overlap d
    assert _err(_gemm(d_dt=F.BF16, q_out=q(qt=P(1 << 36)))) == F.ERR_ARG          # q and q_t overlap
    assert _err(_gemm(d_dt=F.BF16, d=None)) == F.ERR_NULL                         # no output at all
    assert _gemm(m=0, d_dt=F.BF16, d=None, q_out=q()) == F.OK


def test_linear_prequantised_x_validation():
    r = F.Recipe(just_in_time=1)
    meta = F._MetaC(1 << 36, (1 << 36) + 4096, (1 << 36) + 8192)
    saved = F._SavedC(1 << 37, 1 << 38, 1 << 39, 1 << 40, 1 << 41)
    fwd = L.fp8_linear_fwd
    assert _err(fwd(64, 64, 64, None, F.BF16, B16, F.F32, None, F.F32, 0, C16, F.F32, None, None, None, None,
                    ctypes.byref(r), ctypes.byref(meta), ctypes.byref(meta), ctypes.byref(saved), None)) == F.ERR_ARG
    # W pre-cast (w = NULL) is refused under just-in-time scaling too, and needs aligned saved codes
    assert _err(fwd(64, 64, 64, A16, F.BF16, None, F.F32, None, F.F32, 0, C16, F.F32, None, None, None, None,
                    ctypes.byref(r), ctypes.byref(meta), ctypes.byref(meta), ctypes.byref(saved), None)) == F.ERR_ARG
    delayed = F.Recipe()
    bad_saved = F._SavedC(1 << 37, 1 << 38, (1 << 39) + 8, 1 << 40, 1 << 41)
    assert _err(fwd(64, 64, 64, A16, F.BF16, None, F.F32, None, F.F32, 0, C16, F.F32, None, None, None, None,
                    ctypes.byref(delayed), ctypes.byref(meta), ctypes.byref(meta), ctypes.byref(bad_saved),
                    None)) == F.ERR_ALIGN


def test_sgd_step_cast_validation():
    f = L.fp8_sgd_step_cast
    f.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, P, P, P, P, P, P]
    w, g, st, sc = P(1 << 36), P(1 << 37), P(1 << 38), P(1 << 39)
    q, qt, slot = P(1 << 40), P(1 << 41), P(1 << 42)
    assert _err(f(w, g, 64, 60, 1e-3, st, sc, q, qt, slot, None)) == F.ERR_SHAPE
    assert _err(f(w, g, 64, 64, 1e-3, None, sc, q, qt, slot, None)) == F.ERR_NULL         # no state
    assert _err(f(w, None, 64, 64, 1e-3, st, sc, q, qt, slot, None)) == F.ERR_NULL        # no gradient
    assert _err(f(w, g, 64, 64, 1e-3, st, None, q, qt, slot, None)) == F.ERR_NULL         # no scale
    assert _err(f(w, g, 64, 64, 1e-3, st, sc, q, None, slot, None)) == F.ERR_NULL         # q_t is required
    assert _err(f(w, P((1 << 37) + 8), 64, 64, 1e-3, st, sc, q, qt, slot, None)) == F.ERR_ALIGN
    assert _err(f(w, g, 64, 64, 1e-3, st, sc, P((1 << 40) + 4), qt, slot, None)) == F.ERR_ALIGN
    assert _err(f(w, P((1 << 36) + 4096), 64, 64, 1e-3, st, sc, q, qt, slot, None)) == F.ERR_ARG    # g inside w
    assert _err(f(w, g, 64, 64, 1e-3, P((1 << 36) + 64), sc, q, qt, slot, None)) == F.ERR_ARG       # state in w
    assert _err(f(w, g, 64, 64, 1e-3, st, sc, P((1 << 36) + 1024), qt, slot, None)) == F.ERR_ARG    # codes in w
    assert _err(f(w, g, 64, 64, 1e-3, st, sc, q, qt, P((1 << 36) + 256), None)) == F.ERR_ARG        # slot in w
    assert _err(f(w, g, 64, 64, 1e-3, st, sc, P((1 << 37) + 1024), qt, slot, None)) == F.ERR_ARG    # codes in g
    assert f(w, g, 0, 64, 1e-3, st, sc, q, qt, slot, None) == F.OK                                 # empty: nothing runs


def test_loss_scale_and_sgd_validation():
    st = P(1 << 34)
    up = L.fp8_loss_scale_update
    assert _err(up(A16, 0, 1, st, 5, 0.5, 2.0, None)) == F.ERR_SHAPE
    assert _err(up(A16, 4, 0, st, 5, 0.5, 2.0, None)) == F.ERR_SHAPE
    assert _err(up(A16, 4, 1, st, 0, 0.5, 2.0, None)) == F.ERR_ARG
    assert _err(up(A16, 4, 1, st, 5, 1.0, 2.0, None)) == F.ERR_ARG
    assert _err(up(A16, 4, 1, st, 5, 0.5, 1.0, None)) == F.ERR_ARG
    assert _err(up(A16, 4, 1, None, 5, 0.5, 2.0, None)) == F.ERR_NULL
    assert _err(up(A16, 4, 1, P((1 << 20) + 8), 5, 0.5, 2.0, None)) == F.ERR_ARG   # state inside the amaxes
    ap = L.fp8_loss_scale_apply
    assert _err(ap(A16, F.E4M3, 16, st, B16, None)) == F.ERR_DTYPE
    assert _err(ap(A16, F.F32, 16, None, B16, None)) == F.ERR_NULL
    assert _err(ap(A16, F.F32, 64, st, P((1 << 20) + 16), None)) == F.ERR_ARG      # partial overlap
    assert ap(A16, F.F32, 0, st, A16, None) == F.OK
    sgd = L.fp8_sgd_step
    assert _err(sgd(A16, B16, -1, 0.1, st, None)) == F.ERR_SHAPE
    assert _err(sgd(A16, None, 16, 0.1, st, None)) == F.ERR_NULL
    assert _err(sgd(ODD, B16, 16, 0.1, st, None)) == F.ERR_ALIGN
    assert _err(sgd(A16, P((1 << 20) + 16), 16, 0.1, st, None)) == F.ERR_ARG       # w overlaps g
    assert sgd(A16, B16, 0, 0.1, st, None) == F.OK


def test_timing_toggle():
    assert L.fp8lin_timing_enable(-1) == F.ERR_ARG
    assert L.fp8lin_timing_enable(0) == F.OK


def test_attention_validation():
    I64 = ctypes.c_int64
    ws_bytes = L.bf16_attention_workspace_bytes
    ws_bytes.restype = I64
    ws_bytes.argtypes = [I64, I64, I64, I64, ctypes.c_int32]
    assert ws_bytes(2, 4096, 64, 128, 0) == 2 * 4096 * 64 * 128 * 2   # V^T
    assert ws_bytes(2, 4096, 64, 128, 1) == 2 * 2 * 4096 * 64 * 128 * 2 + 2 * 64 * 4096 * 4   # Q^T, dO^T, rowsum
    assert ws_bytes(2, 4096, 64, 64, 0) == -1 and ws_bytes(1, 100, 2, 128, 1) == -1
    fwd, bwd = L.bf16_attention_fwd, L.bf16_attention_bwd
    fwd.argtypes = [P, I64, I64, I64, I64, P, P, P, P]
    bwd.argtypes = [P, P, P, P, I64, I64, I64, I64, P, P, P]
    big = [P(1 << 36), P(1 << 37), P(1 << 38), P(1 << 39), P(1 << 40), P(1 << 41)]
    assert fwd(big[0], 1, 256, 2, 64, big[1], big[2], big[3], None) == F.ERR_UNSUPPORTED
    assert fwd(big[0], 1, 100, 2, 128, big[1], big[2], big[3], None) == F.ERR_SHAPE
    assert fwd(big[0], 0, 256, 2, 128, big[1], big[2], big[3], None) == F.ERR_SHAPE
    assert fwd(big[0], 1 << 12, 4096, 256, 128, big[1], big[2], big[3], None) == F.ERR_SHAPE
    # tile-load byte offsets within one (batch, head) must stay below 2^31
    assert ws_bytes(1, 1 << 16, 42, 128, 1) == 2 * (1 << 16) * 42 * 128 * 2 + 42 * (1 << 16) * 4
    assert ws_bytes(1, 1 << 16, 43, 128, 0) == -1                    # seq*heads*768 >= 2^31
    assert ws_bytes(1 << 7, 1 << 16, 1, 128, 0) == -1                # batch*seq*256 >= 2^31
    assert ws_bytes((1 << 7) - 1, 1 << 16, 1, 128, 1) > 0
    assert fwd(big[0], 1, 1 << 16, 43, 128, big[1], big[2], big[3], None) == F.ERR_SHAPE
    assert fwd(None, 1, 256, 2, 128, big[1], big[2], big[3], None) == F.ERR_NULL
    assert fwd(big[0], 1, 256, 2, 128, ODD, big[2], big[3], None) == F.ERR_ALIGN
    assert fwd(big[0], 1, 256, 2, 128, big[0], big[2], big[3], None) == F.ERR_ARG          # ctx on qkv
    assert fwd(big[0], 1, 256, 2, 128, big[1], big[0], big[3], None) == F.ERR_ARG          # lse on qkv
    assert fwd(big[0], 1, 256, 2, 128, big[1], big[2], big[1], None) == F.ERR_ARG          # workspace on ctx
    assert bwd(big[0], big[1], big[2], big[3], 1, 256, 2, 128, big[0], big[5], None) == F.ERR_ARG   # dqkv on qkv
    assert bwd(big[0], big[1], big[2], big[3], 1, 256, 2, 128, big[4], big[3], None) == F.ERR_ARG   # ws on dctx
    assert bwd(big[0], big[1], None, big[3], 1, 256, 2, 128, big[4], big[5], None) == F.ERR_NULL
    assert bwd(big[0], big[1], big[2], big[3], 1, 512, 2, 96, big[4], big[5], None) == F.ERR_UNSUPPORTED


def test_saturation_counter_registry():
    """fp8lin_count_saturation keeps at most 256 registrations keyed by amax
    slot; re-registering replaces, NULL removes (also for a slot never
    registered); the pointers are not dereferenced."""
    f = L.fp8lin_count_saturation
    f.argtypes = [P, P]
    slots = [P((1 << 40) + 4 * i) for i in range(257)]
    ctrs = [P((1 << 41) + 4 * i) for i in range(257)]
    try:
        assert f(None, ctrs[0]) == F.ERR_NULL
        assert f(slots[0], P((1 << 41) + 2)) == F.ERR_ALIGN
        assert f(P((1 << 40) + 1), ctrs[0]) == F.ERR_ALIGN
        for i in range(256):
            assert f(slots[i], ctrs[i]) == F.OK
        assert f(slots[256], ctrs[256]) == F.ERR_ARG and b"256" in L.fp8lin_last_error()
        assert f(slots[3], ctrs[256]) == F.OK                 # replace: no new entry
        assert f(slots[256], None) == F.OK                    # never registered
        assert f(slots[5], None) == F.OK                      # frees one entry
        assert f(slots[256], ctrs[256]) == F.OK
    finally:
        for i in range(257):
            f(slots[i], None)
    assert f(slots[0], ctrs[0]) == F.OK and f(slots[0], None) == F.OK


def test_binding_checks_meta_buffers_against_the_recipe():
    """The binding refuses a history buffer whose shape differs from (tensors,
    recipe.history_len) before calling the library (the kernel would read and
    roll past its end); host tensors suffice since nothing is launched."""
    import torch
    recipe = F.Recipe(F.FORMAT_HYBRID, 16, F.AMAX_MAX, 0)
    fmts = [F.E4M3, F.E5M2]
    h, s, si = torch.zeros(2, 8), torch.ones(2), torch.ones(2)
    for fn in (F.fp8_amax_scale_update, F.fp8_scale_from_current_amax):
        with pytest.raises(ValueError, match="history_len 16"):
            fn(h, s, si, fmts, recipe)
        with pytest.raises(ValueError, match="history_len 16"):
            fn(torch.zeros(3, 16), torch.ones(3), torch.ones(3), fmts, recipe)
        with pytest.raises(ValueError, match="scale must hold 2"):
            fn(torch.zeros(2, 16), torch.ones(1), torch.ones(2), fmts, recipe)


def test_noalloc_cast_transpose_validation():
    """The allocation-free cast-transpose validates like fp8_cast_transpose,
    requires dbias, and refuses a shape whose partial sums exceed its 8 MiB
    scratch -- all before any HIP call."""
    fn = L.fp8_cast_transpose_dbias_noalloc
    fn.restype, fn.argtypes = ctypes.c_int32, [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                               P, P, P, P, P, P]
    D = P(1 << 30)
    assert _err(fn(A16, F.BF16, 128, 64, F.E4M3, B16, None, C16, None, None, None)) == F.ERR_NULL
    assert _err(fn(A16, F.BF16, 120, 64, F.E4M3, B16, None, C16, None, D, None)) == F.ERR_SHAPE
    assert _err(fn(A16, F.BF16, 128, 64, F.E4M3, B16, None, C16, None, P((1 << 30) + 2), None)) == F.ERR_ALIGN
    assert _err(fn(A16, F.BF16, 128, 64, F.E4M3, B16, None, C16, None, A16, None)) == F.ERR_ARG     # dbias on x
    # 16384 x 16384 fits (128 row tiles x 16384 columns x 4 bytes = 8 MiB); 16512 rows do not
    assert L.fp8lin_dbias_workspace_bytes(16384, 16384) == 8 << 20
    X, QT, DB, S = P(1 << 40), P(1 << 41), P(1 << 42), P(1 << 43)     # far apart: no overlap
    assert _err(fn(X, F.BF16, 16512, 16384, F.E4M3, S, None, QT, None, DB, None)) == F.ERR_ARG
    assert b"scratch" in L.fp8lin_last_error()


def test_clock_sample_validation():
    fn = L.fp8lin_clock_sample
    fn.restype, fn.argtypes = ctypes.c_int32, [P, ctypes.c_int32, P]
    assert _err(fn(None, 100, None)) == F.ERR_NULL
    assert _err(fn(P((1 << 20) + 4), 100, None)) == F.ERR_ALIGN
    assert _err(fn(A16, 0, None)) == F.ERR_ARG
    assert _err(fn(A16, 2000000, None)) == F.ERR_ARG


def test_dual_update_and_stream_probe_validation():
    du = L.fp8_cast_transpose_dual_update
    du.restype = ctypes.c_int32
    du.argtypes = [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, P, P, P, P, P, P, P,
                   ctypes.POINTER(F.Recipe), P, P]
    X, Q, H, S, SI, T = P(1 << 40), P(1 << 41), P(1 << 42), P(1 << 43), P(1 << 44), P(1 << 45)
    r = F.Recipe(F.FORMAT_HYBRID, 16, F.AMAX_MAX, 0)
    ok = lambda **kw: du(kw.get("x", X), F.BF16, kw.get("rows", 128), 64, kw.get("q", Q), None, None, None, H, S, SI,
                         ctypes.byref(kw.get("recipe", r)), kw.get("ticket", T), None)
    assert _err(ok(ticket=None)) == F.ERR_NULL
    assert _err(ok(ticket=P((1 << 45) + 2))) == F.ERR_ALIGN
    assert _err(ok(rows=120)) == F.ERR_SHAPE
    assert _err(ok(recipe=F.Recipe(F.FORMAT_HYBRID, 0, F.AMAX_MAX, 0))) == F.ERR_ARG
    assert _err(ok(ticket=P((1 << 42) + 64))) == F.ERR_ARG          # ticket inside the history
    assert _err(ok(q=P(1 << 40))) == F.ERR_ARG                       # output on the input
    sp = L.fp8lin_stream_probe
    sp.restype, sp.argtypes = ctypes.c_int32, [P, P, ctypes.c_int64, ctypes.c_int32, P]
    assert _err(sp(A16, B16, 1024, 5, None)) == F.ERR_ARG
    assert _err(sp(A16, B16, 1024, -1, None)) == F.ERR_ARG
    # the copy-twice modes write 2 * bytes: a dst whose second copy would reach src is refused
    assert _err(sp(P((1 << 20) + 1536), P(1 << 20), 1024, 3, None)) == F.ERR_ARG
    assert _err(sp(P((1 << 20) + 1024), P(1 << 20), 1024, 4, None)) == F.ERR_ARG
    assert sp(P((1 << 20) + 2048), P(1 << 20), 0, 3, None) == F.OK
    assert _err(sp(A16, B16, 1000, 0, None)) == F.ERR_SHAPE
    assert _err(sp(None, B16, 1024, 1, None)) == F.ERR_NULL
    assert _err(sp(ODD, B16, 1024, 1, None)) == F.ERR_ALIGN
    assert _err(sp(A16, P((1 << 20) + 512), 1024, 1, None)) == F.ERR_ARG
    assert sp(A16, B16, 0, 1, None) == F.OK


def test_attention_workspace_too_small_is_refused():
    """The library cannot see a workspace's size, so the binding refuses an
    undersized one before any call (host tensors: nothing reaches a GPU)."""
    import torch
    batch, seq, heads = 1, 256, 2
    qkv = torch.zeros(batch * seq, 3 * heads * 128, dtype=torch.bfloat16)
    ctx = torch.zeros(batch * seq, heads * 128, dtype=torch.bfloat16)
    lse = torch.zeros(batch, heads, seq)
    dqkv = torch.zeros_like(qkv)
    need_f = F.attention_workspace_bytes(batch, seq, heads)
    need_b = F.attention_workspace_bytes(batch, seq, heads, backward=True)
    assert need_f == batch * seq * heads * 128 * 2 and need_b == 2 * need_f + batch * heads * seq * 4
    with pytest.raises(ValueError, match="forward: workspace of"):
        F.bf16_attention_fwd(qkv, batch, heads, ctx, lse, torch.zeros(need_f - 16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="backward: workspace of"):
        F.bf16_attention_bwd(qkv, ctx, lse, ctx, batch, heads, dqkv, torch.zeros(need_b - 4, dtype=torch.uint8))
    with pytest.raises(ValueError):
        F.bf16_attention_fwd(qkv, batch, heads, ctx, lse, None)
