/*
 * fp8lin.h -- C ABI of libfp8lin.so: an FP8 linear layer with per-tensor
 * delayed scaling for AMD Instinct MI355X (gfx950).
 *
 * Pages the operations come from (titles as published):
 *   [TE-KR]  "Transformer Engine으로 FP8 사용하기" (coniverse.tistory.com)
 *   [MP-KR]  "LLM) Mixed-Precision 개념 및 학습 방법 알아보기" (data-newbie.tistory.com)
 *   [PT-VI]  "Các kiểu dữ liệu FP8 gốc của PyTorch" (hotroai.com)
 *   [TE-RU]  "Как работает FP8 quantization на H100 (Transformer Engine)?" (aivaro.ru)
 *
 * Conventions for every call
 * --------------------------
 * - Pointers are DEVICE pointers unless the comment says "host".  Tensors are
 *   dense and row-major.  FP8 tensors are one byte per element (OCP E4M3 or
 *   OCP E5M2 codes).  bf16 tensors are 16-bit bfloat16 bit patterns.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *   call only enqueues work on that stream and returns; no call synchronises.
 *   Scales and amaxes live in device memory, so delayed scaling never needs a
 *   host round trip.
 * - The library allocates no device memory.  The caller owns every buffer.
 *   Inputs are read-only; the only buffers written are the outputs a call
 *   names, the amax slots it max-merges into, and (fp8_amax_scale_update only)
 *   the metas.  Outputs must not overlap inputs.
 * - Tensor base pointers must be 16-byte aligned (FP8LIN_ERR_ALIGN); scalar
 *   pointers (scale, amax slot, ...) 4-byte aligned.
 * - Arguments are validated on the host before anything is enqueued; a call
 *   that returns an error has had no effect.  A failed launch returns
 *   FP8LIN_ERR_HIP.  fp8lin_last_error() describes the last failure of the
 *   calling thread.  Faults inside a kernel surface at the caller's next
 *   synchronisation, as usual in HIP.
 * - An "amax slot" is a float holding a non-negative value (or NaN).  Calls
 *   max-merge into it: slot = max(slot, amax) compared as IEEE bit patterns of
 *   |x| (so the order of merges does not matter and NaN/Inf propagate).
 */
#ifndef FP8LIN_H
#define FP8LIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8LIN_ABI_VERSION 5

/* Status codes returned by every call. */
enum {
    FP8LIN_OK = 0,
    FP8LIN_ERR_NULL = 1,        /* a required pointer is NULL */
    FP8LIN_ERR_SHAPE = 2,       /* a size is negative, too large, or not a multiple of 16 where required */
    FP8LIN_ERR_ALIGN = 3,       /* a pointer is not aligned as required */
    FP8LIN_ERR_DTYPE = 4,       /* an element type or format is not accepted by this call */
    FP8LIN_ERR_ARG = 5,         /* any other invalid argument (flags, history length, margin, aliasing) */
    FP8LIN_ERR_HIP = 6,         /* the HIP runtime refused a launch */
    FP8LIN_ERR_UNSUPPORTED = 7  /* a valid request the library does not implement */
};

/* Element types. */
enum {
    FP8LIN_F32 = 0,
    FP8LIN_BF16 = 1,
    FP8LIN_E4M3 = 2,            /* OCP E4M3: finite + NaN, max 448  ([TE-KR] "Introduction to FP8") */
    FP8LIN_E5M2 = 3             /* OCP E5M2: IEEE-like, max 57344    ([TE-KR] "Introduction to FP8") */
};

/* Recipe formats ([TE-KR] "FP8 사용방안(recipe)": Format.HYBRID uses E4M3 in the
 * forward pass and E5M2 in the backward pass; [TE-RU] section 4). */
enum {
    FP8LIN_FORMAT_E4M3 = 0,     /* every tensor E4M3 */
    FP8LIN_FORMAT_HYBRID = 1    /* forward tensors E4M3, gradients E5M2 */
};

/* amax_compute_algo: the only algorithm the pages name is "max" over the history. */
enum { FP8LIN_AMAX_MAX = 0 };

/* GEMM epilogue / mode flags. */
enum {
    FP8LIN_EPI_GELU = 1,        /* out = gelu(y), gelu(y) = y * Phi(y) (exact erf form) */
    FP8LIN_EPI_ACCUMULATE = 2,  /* out += y (fp32 outputs only, no GELU) */
    FP8LIN_EPI_FAST_ACCUM = 4   /* native FP8 matrix-core dot products: twice the rate, but the
                                   hardware sums each group of 8 products with ~14 bits kept
                                   below the group's largest product (not fp32-exact).  Without
                                   this flag the products are formed exactly and summed in fp32. */
};

/* Delayed-scaling recipe ([TE-KR] "FP8 사용방안(recipe)", [TE-RU] section 10:
 * DelayedScaling(fp8_format, amax_history_len, amax_compute_algo)).  `margin`
 * divides the scale by 2^margin (0 <= margin <= 127).  `fast_accum` != 0 makes
 * the layer calls run their GEMMs with FP8LIN_EPI_FAST_ACCUM.
 * `just_in_time` != 0 makes the layer calls scale each tensor they cast from
 * its current amax instead of the history ([TE-KR] "Scaling factor" strategy,
 * just-in-time: measure the amax on every use and take the factor from it, at
 * the cost of an extra pass): amax(x) is merged into slot 0, then
 * scale = fp8_max / slot0 / 2^margin (fp8_scale_from_current_amax), then the
 * cast runs with that scale.  Setting it on the first step only gives the
 * "initial amax" behaviour ([PT-VI] training script: enable_amax_init), so
 * that step does not cast with the initial scale 1. */
typedef struct {
    int32_t format;             /* FP8LIN_FORMAT_* */
    int32_t history_len;        /* amax history length L >= 1 */
    int32_t amax_compute_algo;  /* FP8LIN_AMAX_MAX */
    int32_t margin;
    int32_t fast_accum;
    int32_t just_in_time;
} fp8lin_recipe;

/* Per-tensor scaling state ([TE-KR] "Scaling factor" strategy: delayed scaling
 * keeps a history of earlier amaxes as extra state of the FP8 operator).  All
 * three are device pointers: amax_history float[L] in logical order (slot 0 =
 * the current step's amax), scale and scale_inv one float each. */
typedef struct {
    float* amax_history;
    float* scale;
    float* scale_inv;
} fp8lin_meta;

/* What the forward pass leaves for the backward pass ([TE-KR] "Backward Pass
 * 처리": backward runs at the precision fixed in the forward, i.e. on the FP8
 * copies and factors taken there).  Device pointers:
 *   xq [M][K], xq_t [K][M], wq [N][K], wq_t [K][N]  FP8 codes (E4M3)
 *   sinv float[2]: scale_inv of X and of W as they were at the forward pass.
 * xq_t and wq_t may be NULL for inference (no transposes are produced). */
typedef struct {
    uint8_t* xq;
    uint8_t* xq_t;
    uint8_t* wq;
    uint8_t* wq_t;
    float* sinv;
} fp8lin_saved;

/* An FP8 copy of a GEMM's output, cast in the GEMM epilogue.  With delayed
 * scaling the factor of a tensor is known before the tensor exists ([TE-KR]
 * "Scaling factor" strategy: delayed scaling takes it from earlier
 * iterations), so the layer that produces the tensor can emit it in FP8
 * directly, with its amax ([PT-VI] torch._scaled_mm example: the scaled GEMM
 * returns its output and the output's amax), and the next layer skips its
 * input cast.  Device pointers:
 *   scale      the output tensor's current scale
 *   q [m][n], q_t [n][m]   codes, row-major and transposed; either may be NULL
 *   fp8_dtype  FP8LIN_E4M3 or FP8LIN_E5M2
 * The codes are exactly those fp8_cast_transpose would produce from the output
 * as rounded to its type: enc(fl32(bf16(y) * scale)).  bf16 outputs of
 * E4M3 x E4M3 GEMMs (the forward pass) only. */
typedef struct {
    const float* scale;
    uint8_t* q;
    uint8_t* q_t;
    int32_t fp8_dtype;
} fp8lin_qout;

/* ------------------------------------------------------------------------ */

/* FP8LIN_ABI_VERSION of the loaded library. */
int32_t fp8lin_abi_version(void);

/* Message describing the last failed call of the calling thread ("" if none).
 * The string is owned by the library and valid until the thread's next call. */
const char* fp8lin_last_error(void);

/* Name of a status code ("FP8LIN_OK", ...). */
const char* fp8lin_status_name(int32_t status);

/* Bytes of workspace fp8_cast_transpose / fp8_linear_bwd need for a bias
 * gradient of a [rows][cols] tensor (0 if rows or cols is 0). */
int64_t fp8lin_dbias_workspace_bytes(int64_t rows, int64_t cols);

/*
 * fp8_amax -- max-merge amax(x) = max |x_i| into *amax_slot.
 * [TE-KR] "Scaling factor" strategy: scaling is driven by a tensor's absolute
 * maximum; just-in-time scaling measures it on every use.
 *   x         [n] elements of x_dtype (FP8LIN_F32 or FP8LIN_BF16); n >= 0
 *   amax_slot device float, max-merged (bit-pattern max of |x|)
 */
int32_t fp8_amax(const void* x, int32_t x_dtype, int64_t n, float* amax_slot, void* stream);

/*
 * fp8_amax_scale_update -- the per-step delayed-scaling update of n tensors in
 * one launch.  [TE-KR] "Scaling factor" strategy (delayed scaling uses the
 * amaxes of earlier iterations kept as a history); [TE-KR] "FP8 사용방안
 * (recipe)" (amax_compute_algo "max"); [PT-VI] training script (the history
 * and scale update runs once per step after backward, before the optimizer);
 * [TE-RU] section 3 (the tensor is multiplied by the factor before the FP8
 * rounding and the result divided by it after the GEMM).
 * For each tensor t, with h = amax_history + t*L:
 *   A = max over the finite entries of h[0..L-1]
 *   if A > 0:  s = fl32(fl32(fp8_max(fmt[t]) / A) * 2^-margin), s = FLT_MAX if
 *              that overflowed; if s > 0: scale[t] = s, scale_inv[t] = fl32(1/s)
 *   (otherwise scale[t] and scale_inv[t] are kept);
 *   then h rolls one slot: h[i] = h[i-1] (i = L-1..1), h[0] = 0.
 *   amax_history  device float[n][L], updated in place
 *   scale, scale_inv device float[n], updated in place
 *   formats       HOST uint8[n], each FP8LIN_E4M3 or FP8LIN_E5M2 (fp8_max 448 or 57344)
 *   recipe        HOST; uses history_len (L), margin and amax_compute_algo
 * 1 <= n <= 4096, 1 <= L <= 65536.
 */
int32_t fp8_amax_scale_update(float* amax_history, float* scale, float* scale_inv,
                              const uint8_t* formats, int32_t n_tensors,
                              const fp8lin_recipe* recipe, void* stream);

/*
 * fp8_scale_from_current_amax -- just-in-time scaling of n tensors: for each
 * tensor t, with a = amax_history[t*L] (slot 0, the current amax):
 *   if a is finite and > 0: s = fl32(fl32(fp8_max(fmt[t]) / a) * 2^-margin),
 *   FLT_MAX if that overflowed; if s > 0: scale[t] = s, scale_inv[t] = fl32(1/s)
 *   (otherwise both are kept).  The history is not rolled.
 * [TE-KR] "Scaling factor" strategy (just-in-time: the factor from the amax
 * measured now); [PT-VI] training script (enable_amax_init).  Arguments as in
 * fp8_amax_scale_update (recipe: history_len, margin).
 */
int32_t fp8_scale_from_current_amax(float* amax_history, float* scale, float* scale_inv,
                                    const uint8_t* formats, int32_t n_tensors,
                                    const fp8lin_recipe* recipe, void* stream);

/*
 * fp8lin_count_saturation -- opt-in count of saturated codes per tensor, for
 * inspecting how a tensor's values sit against its scale ([TE-KR]
 * "정확도(Precision)": FP8 results differ from higher-precision ones, and
 * debugging needs to see where).  While a counter is registered for amax_slot
 * (a tensor's amax slot: its history's slot 0), every cast of this library
 * that uses that slot for the tensor -- fp8_cast, the fp8_cast_transpose
 * family, and the casts inside fp8_linear_fwd / fp8_linear_bwd of the meta
 * whose amax_history starts at amax_slot, also under just-in-time scaling --
 * adds to *counter the number of elements whose scaled value fl32(x * scale)
 * has a magnitude above the format's largest finite value (448 for E4M3,
 * 57344 for E5M2): the elements the saturating encode clamped (NaN is not
 * counted, +-Inf is).  The FP8 copy written by a GEMM epilogue (q_out) is not
 * counted.  A dual-format cast counts each format into the counter of its own
 * slot.
 *   amax_slot  device float (the key; not dereferenced here)
 *   counter    device uint32, 4-byte aligned, on the device the casts run
 *              on; NULL removes the registration.  Counts accumulate: the
 *              caller clears the counter between steps.  Registering a slot
 *              again replaces its counter.
 * Registrations are process-wide (every device and stream), at most 256 at a
 * time (FP8LIN_ERR_ARG beyond); counting costs a compare per element and one
 * atomic per wave in the casts it applies to, nothing elsewhere.  Remove a
 * registration before freeing its slot or counter: a later cast whose amax
 * slot reused the address would add into whatever then holds the counter's.
 */
int32_t fp8lin_count_saturation(const float* amax_slot, uint32_t* counter);

/*
 * fp8_cast -- q = enc_F(fl32(x * scale)) elementwise, with amax(x) fused.
 * [TE-KR] "FP8 자동변환(Autocasting)": inputs are converted to FP8 and their
 * amax recorded in the same step; [TE-RU] section 3.  enc_F is the saturating
 * round-to-nearest-even encode of format F (fp32 product first, no FMA; NaN ->
 * sign|0x7F; +-Inf and |p| >= fp8_max -> +-max; FP8 subnormals kept; sign of
 * zero kept).
 *   x         [n] of x_dtype (F32 or BF16), n >= 0 (any n, no multiple-of-16 rule)
 *   fp8_dtype FP8LIN_E4M3 or FP8LIN_E5M2
 *   scale     device float
 *   q         [n] codes
 *   amax_slot device float or NULL
 */
int32_t fp8_cast(const void* x, int32_t x_dtype, int64_t n, int32_t fp8_dtype,
                 const float* scale, uint8_t* q, float* amax_slot, void* stream);

/*
 * fp8_cast_transpose -- fp8_cast of a [rows][cols] tensor that writes the codes
 * both row-major (q [rows][cols]) and transposed (q_t [cols][rows]), so each
 * backward GEMM finds its operand contiguous along the reduced dimension.
 * Optionally also the bias gradient dbias[c] = sum_r x[r][c] (fp32).
 * [TE-KR] "Backward Pass 처리" (backward consumes the forward's FP8 copies);
 * [PT-VI] torch._scaled_mm example (the second operand enters transposed).
 *   rows, cols  >= 0 and multiples of 16 ([TE-KR] caution note: FP8 linear
 *               layers need both dimensions divisible by 16); rows < 2^24 and
 *               cols < 2^22 (every cast-transpose entry point), else
 *               FP8LIN_ERR_SHAPE
 *   q           [rows][cols] or NULL (only the transpose is written)
 *   q_t         [cols][rows]
 *   amax_slot   device float or NULL
 *   dbias       device float[cols] or NULL (overwritten, not accumulated)
 *   dbias_ws    workspace of fp8lin_dbias_workspace_bytes(rows, cols) bytes;
 *               required when dbias != NULL, else ignored
 */
int32_t fp8_cast_transpose(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                           int32_t fp8_dtype, const float* scale, uint8_t* q, uint8_t* q_t,
                           float* amax_slot, float* dbias, float* dbias_ws, void* stream);

/*
 * fp8_cast_transpose_dbias_noalloc -- fp8_cast_transpose with the bias
 * gradient, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops, harnesses that forbid hipMalloc): it takes no
 * workspace and allocates nothing; the bias gradient's partial sums go to a
 * scratch array inside the library, one per device, held until the process
 * ends.  Arguments as in fp8_cast_transpose; dbias (device float[cols]) is
 * required.  The scratch holds 8 MiB: rows, cols with
 * fp8lin_dbias_workspace_bytes(rows, cols) > 8 MiB (more than 2^28 elements
 * for any cols; e.g. 16384 x 16384 still fits) return FP8LIN_ERR_ARG.  Calls
 * that overlap in time on one device share that scratch and race: issue them
 * on one stream (or order them), as the library's other calls on shared
 * outputs.  The results equal fp8_cast_transpose's bit for bit.
 */
int32_t fp8_cast_transpose_dbias_noalloc(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                                         int32_t fp8_dtype, const float* scale, uint8_t* q, uint8_t* q_t,
                                         float* amax_slot, float* dbias, void* stream);

/*
 * fp8_cast_transpose_dgelu -- the cast-transpose of the gradient entering a
 * GeLU: dz = round_x(dh * gelu'(z)) is formed on the fly (fp32 math, rounded to
 * the element type of dh), then cast and transposed as fp8_cast_transpose does;
 * amax and dbias are of dz.  gelu'(z) = Phi(z) + z * phi(z).
 *   dh, z       [rows][cols] of x_dtype (F32 or BF16); z is the pre-GeLU value
 *   dz_out      [rows][cols] of x_dtype or NULL (the rounded dz, for inspection)
 *   other arguments as in fp8_cast_transpose
 */
int32_t fp8_cast_transpose_dgelu(const void* dh, const void* z, int32_t x_dtype,
                                 int64_t rows, int64_t cols, int32_t fp8_dtype,
                                 const float* scale, uint8_t* q, uint8_t* q_t,
                                 float* amax_slot, float* dbias, float* dbias_ws,
                                 void* dz_out, void* stream);

/*
 * fp8_cast_transpose_dual -- one read of x, cast with two scales to both
 * formats, each written row-major and transposed: the quantisation of a tensor
 * whose E4M3 and E5M2 copies are both wanted (e.g. a tensor used in the forward
 * pass and as a gradient operand).  [TE-KR] "Introduction to FP8" (the two
 * formats and their roles) and "FP8 자동변환(Autocasting)" (cast with amax);
 * [PT-VI] (the scaled cast of a tensor to either float8 type).
 *   x            [rows][cols] of x_dtype (F32 or BF16); rows, cols multiples of 16
 *   scale_e4m3, scale_e5m2   device floats
 *   q_e4m3 [rows][cols], q_e4m3_t [cols][rows], q_e5m2, q_e5m2_t: codes, each
 *                may be NULL (at least one given); no two may overlap
 *   amax_slot_e4m3, amax_slot_e5m2   device floats or NULL: both get amax(x)
 */
int32_t fp8_cast_transpose_dual(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                                const float* scale_e4m3, uint8_t* q_e4m3, uint8_t* q_e4m3_t, float* amax_slot_e4m3,
                                const float* scale_e5m2, uint8_t* q_e5m2, uint8_t* q_e5m2_t, float* amax_slot_e5m2,
                                void* stream);

/*
 * fp8_cast_transpose_dual_update -- fp8_cast_transpose_dual into the metas of
 * a two-tensor bank (tensor 0 E4M3, tensor 1 E5M2), followed in the same
 * launch by fp8_amax_scale_update of both, run by the last workgroup to
 * finish: amax, cast to both formats in both layouts, and the new scales as
 * one step ([TE-KR] "FP8 자동변환(Autocasting)": inputs are cast, their amax
 * recorded and the factor computed together).  The results equal
 * fp8_cast_transpose_dual (scales scale[0], scale[1]; amax slots
 * amax_history[0], amax_history[L]) followed by fp8_amax_scale_update of the
 * two tensors, bit for bit.
 *   x              [rows][cols] of x_dtype (F32 or BF16), multiples of 16
 *   q_e4m3 [rows][cols], q_e4m3_t [cols][rows], q_e5m2, q_e5m2_t: as in
 *                  fp8_cast_transpose_dual (any may be NULL, not all)
 *   amax_history   device float[2][L]; scale, scale_inv device float[2]
 *   recipe         HOST: history_len L, margin, amax_compute_algo
 *   ticket         device uint32 that is 0 before the first call; every call
 *                  leaves it 0.  Calls in flight at the same time need
 *                  tickets of their own.
 */
int32_t fp8_cast_transpose_dual_update(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                                       uint8_t* q_e4m3, uint8_t* q_e4m3_t, uint8_t* q_e5m2, uint8_t* q_e5m2_t,
                                       float* amax_history, float* scale, float* scale_inv,
                                       const fp8lin_recipe* recipe, uint32_t* ticket, void* stream);

/*
 * fp8_dequant -- out = round_out(fl32(dec_F(q) * scale_inv)) elementwise.
 * [TE-RU] section 3: after the FP8 operation the factor is divided back out;
 * [TE-KR] "정확도(Precision)": the FP8-representable copy of a tensor.
 *   q         [n] codes of fp8_dtype, n >= 0
 *   scale_inv device float
 *   out       [n] of out_dtype (F32, or BF16 rounded to nearest-even)
 */
int32_t fp8_dequant(const uint8_t* q, int32_t fp8_dtype, int64_t n, const float* scale_inv,
                    void* out, int32_t out_dtype, void* stream);

/*
 * fp8_gemm -- the scaled FP8 GEMM with fp32 accumulation and a fused epilogue:
 *   y[i][j] = (sum_k dec(a[i][k]) * dec(b[j][k])) * sinv_a * sinv_b + bias[j]
 *   d[i][j] = gelu(y) | y | d[i][j] + y   (per `epilogue`), then + residual[i][j]
 *             if a residual is given, rounded to d_dtype
 * [PT-VI] torch._scaled_mm example: two FP8 operands (the second transposed),
 * their scales, an optional bias, an output type, and the output's amax;
 * [MP-KR] "Accumulation into FP32"; [TE-RU] section 3 (inverse scaling after
 * the GEMM).  Both operands are contiguous along k ("TN").
 *   a [m][k], b [n][k]  codes; (a_dtype, b_dtype) in {E4M3, E5M2}^2
 *   m, n, k    >= 0 and multiples of 16; k < 2^23
 *   sinv_a, sinv_b  device floats
 *   bias       device [n] of bias_dtype (F32 or BF16) or NULL
 *   epilogue   0, FP8LIN_EPI_GELU or FP8LIN_EPI_ACCUMULATE, optionally | FP8LIN_EPI_FAST_ACCUM
 *   d          [m][n] of d_dtype (F32 or BF16; ACCUMULATE needs F32)
 *   aux        [m][n] of d_dtype or NULL: y before GeLU (only with GELU)
 *   residual   [m][n] of d_dtype or NULL: added in fp32 after the activation,
 *              before the one rounding to d_dtype.  This is the residual
 *              connection of a transformer block, whose branches end in the
 *              linear layers that [PT-VI]'s training script swaps for FP8 ones
 *              (a VisionTransformer); the pages do not spell the wiring out.
 *              It may be d itself (in-place residual add) but must not
 *              otherwise overlap d or aux; not combinable with ACCUMULATE.
 *   amax_d     device float or NULL: max-merged amax of d as written
 *   q_out      HOST struct or NULL: also write the FP8 codes of d (see
 *              fp8lin_qout; needs d_dtype BF16).  With q_out, d may be NULL
 *              (the values are still rounded to bf16 before the cast, and
 *              amax_d is still of those values).
 */
int32_t fp8_gemm(const uint8_t* a, int32_t a_dtype, const uint8_t* b, int32_t b_dtype,
                 int64_t m, int64_t n, int64_t k, const float* sinv_a, const float* sinv_b,
                 const void* bias, int32_t bias_dtype, int32_t epilogue,
                 void* d, int32_t d_dtype, void* aux, const void* residual, float* amax_d,
                 const fp8lin_qout* q_out, void* stream);

/*
 * fp8_linear_fwd -- forward of Y = X W^T + b on FP8 copies of X and W.
 * [TE-KR] "FP8 자동변환(Autocasting)": every input is cast to FP8, its amax
 * recorded and the factor applied; [TE-KR] "Using FP8 with Transformer
 * Engine" (a Linear(768, 768, bias=True) on a 1024x768 input).
 * Steps (all on `stream`): cast(-transpose) X -> saved->xq (+ xq_t) with
 * mx->scale, amax(X) into mx->amax_history[0]; the same for W with mw (with
 * recipe->just_in_time: amax first, then the scale from it, then the cast);
 * saved->sinv = {*mx->scale_inv, *mw->scale_inv}; then fp8_gemm(xq, wq) with
 * sinv = saved->sinv, bias and epilogue, into y (and y_aux, y_amax_slot).
 * The forward format is E4M3 under both recipe formats.
 *   m, n, k   X [m][k], W [n][k], Y [m][n]; multiples of 16
 *   x_dtype, w_dtype  F32 or BF16;  bias: [n] of bias_dtype or NULL
 *   epilogue  0 or FP8LIN_EPI_GELU (then y_aux, if not NULL, gets y before GeLU)
 *   y_dtype   F32 or BF16
 *   residual  [m][n] of y_dtype or NULL, added as in fp8_gemm (may equal y)
 *   y_q       HOST struct or NULL: the FP8 copy of Y for the next layer, cast
 *             in the epilogue (fp8_gemm's q_out; y may then be NULL); pass the
 *             next tensor's meta scale, its saved codes, and its amax slot as
 *             y_amax_slot
 *   mx, mw    HOST structs of device pointers (metas of X and W)
 *   saved     HOST struct of device pointers; xq, wq, sinv required
 * x may be NULL: X's codes are then already in saved->xq (and saved->xq_t),
 * cast with mx->scale by the producer's y_q; the call copies *mx->scale_inv
 * into saved->sinv[0] and records no amax of X (the producer did).  w may be
 * NULL likewise: W's codes are then already in saved->wq and saved->wq_t, cast
 * with mw->scale by the previous step's fp8_sgd_step_cast, which also recorded
 * W's amax; the call copies *mw->scale_inv into saved->sinv[1].  Neither with
 * recipe->just_in_time.
 */
int32_t fp8_linear_fwd(int64_t m, int64_t n, int64_t k,
                       const void* x, int32_t x_dtype, const void* w, int32_t w_dtype,
                       const void* bias, int32_t bias_dtype, int32_t epilogue,
                       void* y, int32_t y_dtype, void* y_aux, const void* residual, float* y_amax_slot,
                       const fp8lin_qout* y_q, const fp8lin_recipe* recipe, const fp8lin_meta* mx,
                       const fp8lin_meta* mw, const fp8lin_saved* saved, void* stream);

/*
 * fp8_linear_bwd -- backward of the FP8 linear from the forward's saved state.
 * [TE-KR] "Backward Pass 처리" (precision fixed by the forward; gradients in
 * E5M2 under HYBRID per "Introduction to FP8"); [MP-KR] "FP32 Master Copy of
 * Weights" (weight gradients feed fp32 masters).
 * Steps: cast-transpose dY (format E5M2 under HYBRID, E4M3 otherwise) with
 * mdy->scale into dyq_ws / dyq_t_ws, amax(dY) into mdy->amax_history[0]
 * (with recipe->just_in_time: amax first, then the scale from it, then the cast),
 * optional dbias = column sums of dY; then
 *   dX [m][k] = (dYq . Wq)   = fp8_gemm(dyq [m][n], wq_t [k][n]) * sinv_dy * saved->sinv[1]
 *   dW [n][k] = (dYq^T . Xq) = fp8_gemm(dyq_t [n][m], xq_t [k][m]) * sinv_dy * saved->sinv[0]
 * If gelu_z is not NULL, dy is the gradient with respect to gelu(Z) of a layer
 * whose forward used FP8LIN_EPI_GELU with pre-activation Z = gelu_z ([m][n],
 * dy's type); the gradient cast is then dZ = round(dy * gelu'(Z)) (see
 * fp8_cast_transpose_dgelu) and dbias is of dZ.
 *   dy        [m][n] of dy_dtype (F32 or BF16)
 *   dz_out    [m][n] of dy_dtype or NULL (only with gelu_z)
 *   mdy       HOST struct of device pointers (meta of the gradient)
 *   saved     HOST struct from the forward; wq_t needed for dX, xq_t for dW
 *   dyq_ws    [m][n] bytes (needed when dx != NULL), dyq_t_ws [n][m] bytes (needed when dw != NULL)
 *   dx        [m][k] of dx_dtype (F32 or BF16) or NULL; must not overlap dy or gelu_z
 *   dx_residual [m][k] of dx_dtype or NULL: added to dX before its rounding
 *             (the gradient arriving through a residual branch; may equal dx)
 *   dw        [n][k] float or NULL; accumulate_dw != 0 adds into it
 *   dbias     float[n] or NULL; dbias_ws as in fp8_cast_transpose
 */
int32_t fp8_linear_bwd(int64_t m, int64_t n, int64_t k,
                       const void* dy, int32_t dy_dtype, const void* gelu_z, void* dz_out,
                       const fp8lin_recipe* recipe, const fp8lin_meta* mdy, const fp8lin_saved* saved,
                       uint8_t* dyq_ws, uint8_t* dyq_t_ws,
                       void* dx, int32_t dx_dtype, const void* dx_residual,
                       float* dw, int32_t accumulate_dw, float* dbias, float* dbias_ws, void* stream);

/*
 * Dynamic loss scaling and the fp32 master-weight step around the FP8 layers.
 * [MP-KR] "Mixed-Precision Training Iteration" (multiply the loss by S before
 * back-propagation, multiply the weight gradients by 1/S, update the fp32
 * master weights) and its dynamic loss-scale procedure (on an Inf/NaN
 * gradient lower S and skip the update; after N iterations without one raise
 * S); [MP-KR] "FP32 Master Copy of Weights".
 * The loss-scale state is a device float[4], 16-byte block owned by the
 * caller: {S, clean iterations, found_inf of the last step, S that the last
 * step's gradients carry}.  Initialise it to {S0, 0, 0, S0}.
 */

/*
 * fp8_loss_scale_update -- once per step, after backward: found_inf = any of
 * the n gradient amaxes grad_amaxes[i*stride] is Inf or NaN (these are the
 * amax slots the backward casts merged into, so overflow is detected without
 * an extra pass over the gradients); state[3] = S; then
 *   found_inf: S *= backoff, clean = 0
 *   else:      clean += 1; if clean >= growth_interval: S *= growth, clean = 0
 *   grad_amaxes  device float, n entries `stride` floats apart; 1 <= n <= 4096
 *   state        device float[4], updated in place
 *   growth_interval >= 1; 0 < backoff < 1 < growth
 */
int32_t fp8_loss_scale_update(const float* grad_amaxes, int32_t n, int64_t stride, float* state,
                              int32_t growth_interval, float backoff, float growth, void* stream);

/*
 * fp8_loss_scale_apply -- out = round(g * state[0]) elementwise (the loss
 * gradient entering back-propagation, scaled by the current S).
 *   g, out   [n] of dtype (F32 or BF16); out may equal g
 *   state    device float[4]
 */
int32_t fp8_loss_scale_apply(const void* g, int32_t dtype, int64_t n, const float* state, void* out,
                             void* stream);

/*
 * fp8_sgd_step -- w = fl32(w - fl32(lr * fl32(g * fl32(1 / state[3])))) on
 * the fp32 master weights, a no-op when state[2] (found_inf) is set.  Run it
 * after fp8_loss_scale_update of the same step.
 *   w      device float[n], updated in place;  g  device float[n] (the scaled
 *          weight gradient);  state  device float[4];  n >= 0
 */
int32_t fp8_sgd_step(float* w, const float* g, int64_t n, float lr, const float* state, void* stream);

/*
 * fp8_sgd_step_cast -- fp8_sgd_step on one fp32 weight matrix fused with the
 * E4M3 cast-transpose that the next forward makes of it: the master weight is
 * read once, updated, written, and cast from registers.  [MP-KR] "FP32 Master
 * Copy of Weights" (the update on the fp32 masters) and [TE-KR] "FP8
 * 자동변환(Autocasting)" (cast and amax in one step): under delayed scaling the
 * scale the next forward casts with is fixed by the metas' update, which runs
 * before this call, so the cast need not wait for that forward.
 *   w       device float[rows][cols], updated in place as fp8_sgd_step does
 *           (a found_inf step leaves it and still casts it)
 *   g       device float[rows][cols];  state  device float[4] (loss-scale state)
 *   scale   device float: the E4M3 scale of W for the next forward (its meta's
 *           scale after the update)
 *   q       [rows][cols] codes, row-major, or NULL;  q_t  [cols][rows] codes
 *   amax_slot device float or NULL: amax of the updated w is max-merged into it
 *           (the meta's slot 0 after the update's roll)
 * rows, cols >= 0, multiples of 16.  q and q_t equal fp8_cast_transpose of the
 * updated w with the same scale bit for bit, and w equals fp8_sgd_step's
 * result bit for bit.  The next fp8_linear_fwd then takes w = NULL (its W
 * codes are in saved->wq / saved->wq_t).  Not for just-in-time scaling, whose
 * scale comes from the updated w's own amax.
 */
int32_t fp8_sgd_step_cast(float* w, const float* g, int64_t rows, int64_t cols, float lr, const float* state,
                          const float* scale, uint8_t* q, uint8_t* q_t, float* amax_slot, void* stream);

/*
 * bf16 attention core between the fused QKV projection and the output
 * projection of a transformer layer ([PT-VI], its vision-transformer
 * workload: multi-head attention in bf16 between FP8 linears; the pages do not
 * write the core out, so this is textbook scaled dot-product attention with no
 * mask).  Per batch b and head h, with D = head_dim:
 *   S = Q K^T / sqrt(D), P = softmax(S) over the keys, O = P V;
 *   backward for dO: dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dO * O)),
 *   dQ = dS K / sqrt(D), dK = dS^T Q / sqrt(D).
 * Layouts (bf16, row-major):
 *   qkv   [batch*seq][3*heads*D]: columns [Q | K | V], head h at columns
 *         h*D .. h*D+D-1 of each part (token index b*seq + s)
 *   ctx   [batch*seq][heads*D]: O, same head layout (the output projection's input)
 *   lse   device float[batch][heads][seq]: m + log2(l) of each query's
 *         softmax in the base-2 domain (scores times log2(e)/sqrt(D)), saved
 *         by the forward for the backward
 * Numerics: bf16 products exact, fp32 sums; softmax in fp32; P and dS rounded
 * to bf16 as operands of the second products; outputs rounded to bf16 (RNE).
 * Inf/NaN inputs give unspecified (non-finite) outputs.
 * Supported: head_dim == 128 (else FP8LIN_ERR_UNSUPPORTED), seq a multiple of
 * 256, batch*seq*heads*128 < 2^31, seq*heads*768 < 2^31 and
 * batch*seq*256 < 2^31 (byte offsets of the tile loads within one (batch,
 * head)); other shapes give FP8LIN_ERR_SHAPE.
 * Workspace (caller-owned device memory, 16-byte aligned, contents not
 * preserved): bf16_attention_workspace_bytes(batch, seq, heads, head_dim,
 * backward) bytes: the forward holds V^T (batch*seq*heads*D bf16), the
 * backward Q^T and dO^T (2 * batch*seq*heads*D bf16) and rowsum(dO * O)
 * (batch*heads*seq fp32); K^T is read from the row-major K tile in the LDS
 * with transposing reads, so no copy of it is made.
 * The library cannot see the workspace's size; a caller that shares one
 * workspace between the two calls sizes it as the larger figure.
 */
int64_t bf16_attention_workspace_bytes(int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                       int32_t backward);

/*
 * bf16_attention_fwd -- ctx = attention(qkv), lse saved for the backward.
 *   qkv in; ctx, lse out (must not overlap qkv, each other or the workspace).
 */
int32_t bf16_attention_fwd(const void* qkv, int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                           void* ctx, float* lse, void* workspace, void* stream);

/*
 * bf16_attention_bwd -- dqkv = gradient of <ctx, dctx> with respect to qkv,
 * from the forward's qkv, ctx and lse.  All three parts of dqkv are written
 * (overwritten, not accumulated).
 *   qkv, ctx, lse, dctx in; dqkv out (must not overlap the inputs or the workspace).
 */
int32_t bf16_attention_bwd(const void* qkv, const void* ctx, const float* lse, const void* dctx, int64_t batch,
                           int64_t seq, int64_t heads, int64_t head_dim, void* dqkv, void* workspace,
                           void* stream);

/*
 * Kernel timing.  fp8lin_timing_enable(capacity) makes the library record a
 * pair of HIP events around each of its next `capacity` kernel launches
 * (0 disables and frees the events).  fp8lin_timing_read waits for the
 * recorded events and returns, for up to `max` launches, the kernel kind
 * (FP8LIN_KIND_*) and the elapsed milliseconds (-1 where the events could not
 * be read); it returns the count and resets the record.  Events are host-side objects; no device memory is used.
 */
enum {
    FP8LIN_KIND_AMAX = 0, FP8LIN_KIND_CAST = 1, FP8LIN_KIND_CAST_TRANSPOSE = 2,
    FP8LIN_KIND_DEQUANT = 3, FP8LIN_KIND_SCALE_UPDATE = 4, FP8LIN_KIND_GEMM = 5,
    FP8LIN_KIND_DBIAS = 6, FP8LIN_KIND_OTHER = 7, FP8LIN_KIND_SGD = 8, FP8LIN_KIND_ATTENTION = 9,
    FP8LIN_KIND_STREAM = 10
};
int32_t fp8lin_timing_enable(int32_t capacity);

/*
 * Shader-clock sample, a measurement aid beside the timer: one wave reads the
 * GPU's shader-clock counter and its constant 100 MHz counter, waits about
 * wait_us microseconds (1..1000000) of the latter, reads both again and writes
 * {clock0, clock1, ref0, ref1} to out (device uint64[4]).  Enqueued on a
 * second stream while other kernels run, (clock1 - clock0) / (ref1 - ref0) *
 * 100 MHz is the shader clock they ran at.
 */
int32_t fp8lin_clock_sample(uint64_t* out, int32_t wait_us, void* stream);

/*
 * Streaming reference kernels, a measurement aid: the HBM rate that the
 * elementwise kernels' load/store layout reaches without their arithmetic.
 * mode 0 reads bytes of src (16-byte vectors, the same grid and layout as
 * fp8_amax) and writes one 32-bit word per workgroup to dst (at most 2048
 * words: dst holds 8 KiB); mode 1 copies bytes of src to dst; mode 2 copies
 * with non-temporal stores (the stores fp8_dequant uses); modes 3 and 4 copy
 * twice, to dst and to dst + bytes (dst holds 2 * bytes), with plain and with
 * non-temporal stores: one read and two writes, the read:write ratio of the
 * dual-format cast-transpose and of the dequant.  bytes is a multiple of 16;
 * src, dst 16-byte aligned and not overlapping.  Timed as FP8LIN_KIND_STREAM.
 */
int32_t fp8lin_stream_probe(const void* src, void* dst, int64_t bytes, int32_t mode, void* stream);
int32_t fp8lin_timing_read(int32_t* kinds, float* ms, int32_t max);

#ifdef __cplusplus
}
#endif
#endif /* FP8LIN_H */
