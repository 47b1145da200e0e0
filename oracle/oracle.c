/*
 * CPU oracle for the FP8 linear layer with per-tensor delayed scaling.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, by the smoke check and by the
 * CPU-baseline leg of the benchmark, never by the product library.
 *
 * Plain C11, compiled with -O2 -ffp-contract=off and no fast-math, so every
 * float/double operation below is one IEEE operation rounded to nearest-even,
 * with subnormals kept.  OpenMP, where used, splits independent outputs (rows,
 * elements) and never changes the order of a reduction, so results do not
 * depend on the thread count.
 *
 * Page tags ([TE-KR], [MP-KR], [PT-VI], [TE-RU]) are spelled out in oracle.h.
 * Where the pages leave a step open, the reading taken is stated at the step.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint64_t f64_bits(double d) { uint64_t u; memcpy(&u, &d, 8); return u; }
static float bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

static float load_elem(const void* x, int dtype, int64_t i) {
    if (dtype == ORC_F32) return ((const float*)x)[i];
    return bf16_to_f32(((const uint16_t*)x)[i]);
}

/* ------------------------------------------------------------------------ */
/* Generic minifloat codec.                                                  */
/*                                                                           */
/* A format has 1 sign bit, `ebits` exponent bits with bias 2^(ebits-1)-1    */
/* and `mbits` mantissa bits.  Two styles:                                   */
/*   IEEE: the all-ones exponent encodes Inf (mantissa 0) and NaN.  E5M2,    */
/*         fp16 and bf16 are of this kind.                                   */
/*   FN:   no Inf; only all-ones exponent with all-ones mantissa is NaN, the */
/*         rest of the top binade holds finite values.  E4M3 is of this kind.*/
/* [TE-KR] "Introduction to FP8" gives E4M3 a range of +-448 and E5M2 one of */
/* +-57344; [PT-VI]'s finfo table lists both with their smallest normals     */
/* (2^-6, 2^-14) and eps (0.125, 0.25); [TE-RU] section 1 names the bit      */
/* splits (4+3 and 5+2).  All of that follows from the layout below.         */
/* ------------------------------------------------------------------------ */

typedef struct { int ebits, mbits, style, bias, emin; } mf_t;

static mf_t mf_make(int ebits, int mbits, int style) {
    mf_t f;
    f.ebits = ebits;
    f.mbits = mbits;
    f.style = style;
    f.bias = (1 << (ebits - 1)) - 1;
    f.emin = 1 - f.bias;
    return f;
}

/* Exponent and mantissa fields of the largest finite magnitude. */
static void mf_max_fields(mf_t f, uint32_t* e, uint32_t* m) {
    if (f.style == ORC_STYLE_IEEE) {
        *e = (1u << f.ebits) - 2;
        *m = (1u << f.mbits) - 1;
    } else {
        *e = (1u << f.ebits) - 1;
        *m = (1u << f.mbits) - 2;
    }
}

double orc_mf_decode(uint32_t code, int ebits, int mbits, int style) {
    mf_t f = mf_make(ebits, mbits, style);
    uint32_t s = (code >> (ebits + mbits)) & 1u;
    uint32_t e = (code >> mbits) & ((1u << ebits) - 1);
    uint32_t m = code & ((1u << mbits) - 1);
    uint32_t etop = (1u << ebits) - 1;
    double mag;
    if (style == ORC_STYLE_IEEE && e == etop)
        mag = (m == 0) ? INFINITY : NAN;
    else if (style == ORC_STYLE_FN && e == etop && m == (1u << mbits) - 1)
        mag = NAN;
    else if (e == 0)
        mag = ldexp((double)m, f.emin - mbits);                      /* subnormal */
    else
        mag = ldexp((double)((1u << mbits) + m), (int)e - f.bias - mbits);
    return s ? -mag : mag;
}

double orc_mf_max(int ebits, int mbits, int style) {
    mf_t f = mf_make(ebits, mbits, style);
    uint32_t e, m;
    mf_max_fields(f, &e, &m);
    return orc_mf_decode((e << mbits) | m, ebits, mbits, style);
}

/* Round sig * 2^-sh to an integer, ties to even (sh may be <= 0). */
static uint64_t round_shift_rne(uint64_t sig, int sh) {
    if (sh <= 0) return sig << (-sh);
    if (sh > 60) return 0;                   /* sig < 2^54: value < 1/64 */
    uint64_t q = sig >> sh;
    uint64_t r = sig & ((1ull << sh) - 1);
    uint64_t half = 1ull << (sh - 1);
    if (r > half || (r == half && (q & 1u))) q += 1;
    return q;
}

/*
 * Encode the exact value (-1)^neg * sig * 2^e2 (sig > 0) into the format:
 * the quantum of |p| is 2^(max(floor(log2|p|), emin) - mbits); |p| / quantum
 * is rounded to the nearest integer with ties to even; a result of
 * 2^(mbits+1) carries into the next binade; a result beyond the largest
 * finite value overflows (to max when saturating, else Inf, or NaN for FN).
 */
static uint32_t mf_encode_exact(uint32_t neg, uint64_t sig, int e2, mf_t f, int saturate) {
    uint32_t maxe, maxm;
    mf_max_fields(f, &maxe, &maxm);
    uint32_t sign = neg << (f.ebits + f.mbits);
    uint32_t nan_code = (1u << (f.ebits + f.mbits)) - 1;
    uint32_t inf_code = ((1u << f.ebits) - 1) << f.mbits;
    uint32_t max_code = (maxe << f.mbits) | maxm;
    uint32_t ovf_code = saturate ? max_code : (f.style == ORC_STYLE_IEEE ? inf_code : nan_code);

    int lg = e2 + (63 - __builtin_clzll(sig));            /* floor(log2 |p|) */
    int qe = (lg > f.emin ? lg : f.emin) - f.mbits;       /* exponent of the quantum */
    uint64_t n = round_shift_rne(sig, qe - e2);
    if (n == 0) return sign;                              /* rounds to zero: keep sign */
    if (n >> (f.mbits + 1)) {                             /* carry: n == 2^(mbits+1) */
        n >>= 1;
        qe += 1;
    }
    uint32_t e_field, m_field;
    if (n < (1ull << f.mbits)) {                          /* subnormal: qe == emin - mbits */
        e_field = 0;
        m_field = (uint32_t)n;
    } else {
        long ef = (long)qe + f.mbits + f.bias;
        if (ef > (long)maxe) return sign | ovf_code;
        e_field = (uint32_t)ef;
        m_field = (uint32_t)(n - (1ull << f.mbits));
    }
    if (e_field > maxe || (e_field == maxe && m_field > maxm)) return sign | ovf_code;
    return sign | (e_field << f.mbits) | m_field;
}

uint32_t orc_mf_encode(float p, int ebits, int mbits, int style, int saturate) {
    mf_t f = mf_make(ebits, mbits, style);
    uint32_t b = f32_bits(p);
    uint32_t neg = b >> 31;
    uint32_t ef = (b >> 23) & 0xFFu, mf = b & 0x7FFFFFu;
    uint32_t sign = neg << (ebits + mbits);
    uint32_t nan_code = (1u << (ebits + mbits)) - 1;
    if (ef == 0xFF && mf != 0) return sign | nan_code;
    if (ef == 0xFF) {                                    /* +-Inf */
        uint32_t maxe, maxm;
        mf_max_fields(f, &maxe, &maxm);
        if (saturate) return sign | (maxe << mbits) | maxm;
        return sign | (style == ORC_STYLE_IEEE ? ((1u << ebits) - 1) << mbits : nan_code);
    }
    uint64_t sig;
    int e2;
    if (ef == 0) { sig = mf; e2 = -149; } else { sig = mf | 0x800000u; e2 = (int)ef - 150; }
    if (sig == 0) return sign;                           /* +-0 */
    return mf_encode_exact(neg, sig, e2, f, saturate);
}

void orc_mf_encode_array(const float* p, int64_t n, int ebits, int mbits, int style, int saturate,
                         uint32_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_mf_encode(p[i], ebits, mbits, style, saturate);
}

void orc_mf_decode_array(const uint32_t* code, int64_t n, int ebits, int mbits, int style, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_mf_decode(code[i], ebits, mbits, style);
}

static uint32_t mf_encode_f64(double p, int ebits, int mbits, int style, int saturate) {
    mf_t f = mf_make(ebits, mbits, style);
    uint64_t b = f64_bits(p);
    uint32_t neg = (uint32_t)(b >> 63);
    uint32_t ef = (uint32_t)((b >> 52) & 0x7FFu);
    uint64_t mf = b & 0xFFFFFFFFFFFFFull;
    uint32_t sign = neg << (ebits + mbits);
    uint32_t nan_code = (1u << (ebits + mbits)) - 1;
    if (ef == 0x7FF && mf != 0) return sign | nan_code;
    if (ef == 0x7FF) {
        uint32_t maxe, maxm;
        mf_max_fields(f, &maxe, &maxm);
        if (saturate) return sign | (maxe << mbits) | maxm;
        return sign | (style == ORC_STYLE_IEEE ? ((1u << ebits) - 1) << mbits : nan_code);
    }
    uint64_t sig;
    int e2;
    if (ef == 0) { sig = mf; e2 = -1074; } else { sig = mf | (1ull << 52); e2 = (int)ef - 1075; }
    if (sig == 0) return sign;
    return mf_encode_exact(neg, sig, e2, f, saturate);
}

/* ------------------------------------------------------------------------ */
/* FP8 codec: E4M3 = FN style 4+3, E5M2 = IEEE style 5+2.                    */
/* ------------------------------------------------------------------------ */

double orc_fp8_max(int fmt) {
    return fmt == ORC_E4M3 ? orc_mf_max(4, 3, ORC_STYLE_FN) : orc_mf_max(5, 2, ORC_STYLE_IEEE);
}

double orc_decode(uint8_t code, int fmt) {
    return fmt == ORC_E4M3 ? orc_mf_decode(code, 4, 3, ORC_STYLE_FN)
                           : orc_mf_decode(code, 5, 2, ORC_STYLE_IEEE);
}

/*
 * Saturating round-to-nearest-even cast of an fp32 value.  NaN gives
 * sign|0x7F in both formats, +-Inf and every |p| >= max give +-max, the sign
 * of zero is kept, FP8 subnormals are produced.  (The pages give the formats
 * and their ranges; saturation and RNE are the reading taken for the cast of
 * a scaled tensor, so that an amax that grew since the scale was chosen
 * clips instead of turning into NaN.)
 */
uint8_t orc_encode(float p, int fmt) {
    if (fmt == ORC_E4M3) return (uint8_t)orc_mf_encode(p, 4, 3, ORC_STYLE_FN, 1);
    return (uint8_t)orc_mf_encode(p, 5, 2, ORC_STYLE_IEEE, 1);
}

/*
 * The same cast by brute force: pick, among the non-negative finite codes,
 * the one whose decoded value is nearest to |p| (ties to the even code), then
 * attach the sign of p.  Used only to pin orc_encode.
 */
uint8_t orc_encode_bruteforce(float p, int fmt) {
    uint8_t sign = signbit(p) ? 0x80 : 0x00;
    if (isnan(p)) return sign | 0x7F;
    uint8_t maxc = fmt == ORC_E4M3 ? 0x7E : 0x7B;
    double a = fabs((double)p);
    if (a >= orc_decode(maxc, fmt)) return sign | maxc;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= maxc; ++c) {
        double d = fabs(orc_decode((uint8_t)c, fmt) - a);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(sign | best);
}

void orc_encode_array(const float* p, int64_t n, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_encode(p[i], fmt);
}

void orc_encode_bits_range(uint64_t first_bits, int64_t n, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_encode(bits_f32((uint32_t)(first_bits + (uint64_t)i)), fmt);
}

void orc_encode_bruteforce_array(const float* p, int64_t n, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_encode_bruteforce(p[i], fmt);
}

/* ------------------------------------------------------------------------ */
/* Output rounding: bf16 (8+7 IEEE) and fp32 (8+23 IEEE), RNE, no saturation */
/* ------------------------------------------------------------------------ */

uint16_t orc_bf16_from_f32(float v) { return (uint16_t)orc_mf_encode(v, 8, 7, ORC_STYLE_IEEE, 0); }
uint16_t orc_bf16_from_f64(double v) { return (uint16_t)mf_encode_f64(v, 8, 7, ORC_STYLE_IEEE, 0); }
float orc_f32_from_f64(double v) { return bits_f32(mf_encode_f64(v, 8, 23, ORC_STYLE_IEEE, 0)); }

void orc_bf16_from_f32_array(const float* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32(v[i]);
}

void orc_bf16_from_f64_array(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f64(v[i]);
}

void orc_f32_from_f64_array(const double* v, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_from_f64(v[i]);
}

/* ------------------------------------------------------------------------ */
/* amax: the largest |x| of the tensor.                                      */
/* [TE-KR] "Scaling factor" strategy: both scaling modes are driven by the   */
/* absolute maximum (amax) of a tensor; the autocast step updates it.        */
/* Computed as the largest (bits & 0x7FFFFFFF) of the fp32 value (bf16 is    */
/* widened exactly first): equal to max|x| for ordinary data, order-free,    */
/* -0 counts as 0, and a NaN or Inf element propagates.                      */
/* ------------------------------------------------------------------------ */

float orc_amax(const void* x, int dtype, int64_t n) {
    uint32_t m = 0;
#pragma omp parallel for reduction(max : m) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b = f32_bits(load_elem(x, dtype, i)) & 0x7FFFFFFFu;
        if (b > m) m = b;
    }
    return bits_f32(m);
}

/* ------------------------------------------------------------------------ */
/* Delayed-scaling update.                                                   */
/* [TE-KR] "Scaling factor" strategy (delayed scaling): the factor comes     */
/* from the amaxes of earlier iterations, kept per FP8 tensor as a history.  */
/* [TE-KR] "recipe": DelayedScaling(amax_history_len, amax_compute_algo =    */
/* "max"); [TE-RU] section 10 uses length 1024.  [PT-VI]'s training script   */
/* runs the amax/scale update once per step, after backward and before the   */
/* optimizer.  [TE-RU] section 3: the tensor is multiplied by the factor     */
/* before rounding to FP8 and the GEMM result is divided by it afterwards.   */
/*                                                                           */
/* Per tensor t, history h[t][0..L-1] in logical order (slot 0 = the amax of */
/* the step just finished):                                                  */
/*   A  = max of the finite entries of h                                     */
/*   if A > 0:  s' = fl32(fl32(fp8_max / A) * 2^-margin)                     */
/*              s' = FLT_MAX if it overflowed to +Inf                        */
/*              if s' > 0: scale = s', scale_inv = fl32(1 / s')              */
/*   otherwise the old scale and scale_inv are kept;                         */
/*   then the history rolls: h[i] = h[i-1] for i = L-1..1, h[0] = 0.         */
/* ------------------------------------------------------------------------ */

void orc_scale_update(float* hist, float* scale, float* scale_inv, const uint8_t* fmt,
                      int32_t n_tensors, int32_t hist_len, int32_t margin) {
    for (int32_t t = 0; t < n_tensors; ++t) {
        float* h = hist + (int64_t)t * hist_len;
        float fp8_max = (float)orc_fp8_max(fmt[t]);
        int found = 0;
        float a = 0.0f;
        for (int32_t i = 0; i < hist_len; ++i) {
            if (!isfinite(h[i])) continue;
            if (!found || h[i] > a) a = h[i];
            found = 1;
        }
        if (found && a > 0.0f) {
            float s = fp8_max / a;                                  /* fp32 IEEE division */
            s = (float)((double)s * ldexp(1.0, -margin));           /* exact, one rounding */
            if (isinf(s)) s = FLT_MAX;
            if (s > 0.0f) {
                scale[t] = s;
                scale_inv[t] = 1.0f / s;                            /* fp32 IEEE division */
            }
        }
        for (int32_t i = hist_len - 1; i >= 1; --i) h[i] = h[i - 1];
        h[0] = 0.0f;
    }
}

/* ------------------------------------------------------------------------ */
/* Cast to FP8: q = enc(fl32(x * s)).                                        */
/* [TE-KR] autocasting: every input of an FP8 op is converted to FP8 with   */
/* its own per-tensor factor ("Mixed Precision Training with FP8").          */
/* [TE-RU] section 3: multiply by the factor, then round to FP8.             */
/* Two roundings by definition: the fp32 product (no FMA), then FP8 RNE.     */
/* ------------------------------------------------------------------------ */

void orc_cast(const void* x, int dtype, int64_t n, int fmt, float scale, uint8_t* q) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float prod = load_elem(x, dtype, i) * scale;
        q[i] = orc_encode(prod, fmt);
    }
}

/* Saturated elements of a cast: those whose fp32 product with the scale has a
 * magnitude above the format's largest finite value -- the values the
 * saturating encode clamps to +-max, where the FP8 copy parts most from the
 * higher-precision tensor ([TE-KR] "정확도(Precision)").  NaN products are not
 * counted, infinite ones are. */
int64_t orc_count_saturated(const void* x, int dtype, int64_t n, int fmt, float scale) {
    const double fmax = orc_fp8_max(fmt);
    int64_t c = 0;
#pragma omp parallel for schedule(static) reduction(+ : c)
    for (int64_t i = 0; i < n; ++i) {
        const float prod = load_elem(x, dtype, i) * scale;
        if (fabs((double)prod) > fmax) ++c;
    }
    return c;
}

void orc_transpose_u8(const uint8_t* q, int64_t rows, int64_t cols, uint8_t* q_t) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c)
        for (int64_t r = 0; r < rows; ++r) q_t[c * rows + r] = q[r * cols + c];
}

/* Cast-transpose: the same codes twice, row-major [rows][cols] and
 * transposed [cols][rows], so that both GEMMs of the backward pass find their
 * operands contiguous along the reduced dimension. */
void orc_cast_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int fmt,
                        float scale, uint8_t* q, uint8_t* q_t) {
    orc_cast(x, dtype, rows * cols, fmt, scale, q);
    orc_transpose_u8(q, rows, cols, q_t);
}

/* Dequantisation: x = round_out(fl32(dec(q) * scale_inv)).
 * [TE-RU] section 3: after the FP8 operation the factor is divided back out;
 * [TE-KR] "정확도(Precision)": casting to FP8 and back gives the
 * FP8-representable copy of a tensor. */
void orc_dequant(const uint8_t* q, int fmt, int64_t n, float scale_inv, void* out, int out_dtype) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float v = (float)orc_decode(q[i], fmt) * scale_inv;        /* decode is exact in fp32 */
        if (out_dtype == ORC_F32) ((float*)out)[i] = v;
        else ((uint16_t*)out)[i] = orc_bf16_from_f32(v);
    }
}

/* Column sums in fp64, rows ascending: the bias gradient sum over rows of dY. */
void orc_colsum(const void* x, int dtype, int64_t rows, int64_t cols, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        double s = 0.0;
        for (int64_t r = 0; r < rows; ++r) s += (double)load_elem(x, dtype, r * cols + c);
        out[c] = s;
    }
}

/* ------------------------------------------------------------------------ */
/* GeLU, exact form z * Phi(z) with Phi the standard normal CDF, written     */
/* Phi(z) = erfc(-z / sqrt 2) / 2 so that the far negative tail keeps its    */
/* relative precision (1 + erf(z/sqrt 2) cancels to 0 there).                */
/* ------------------------------------------------------------------------ */

double orc_gelu(double z) { return 0.5 * z * erfc(-z * M_SQRT1_2); }

double orc_gelu_grad(double z) {
    double cdf = 0.5 * erfc(-z * M_SQRT1_2);
    double pdf = exp(-0.5 * z * z) / sqrt(2.0 * M_PI);
    return cdf + z * pdf;
}

/* dz = round_out(dh * gelu'(z)) in fp64, rounded once to the element type. */
void orc_gelu_bwd(const void* dh, const void* z, int dtype, int64_t n, void* dz) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)load_elem(dh, dtype, i) * orc_gelu_grad((double)load_elem(z, dtype, i));
        if (dtype == ORC_F32) ((float*)dz)[i] = orc_f32_from_f64(v);
        else ((uint16_t*)dz)[i] = orc_bf16_from_f64(v);
    }
}

/* ------------------------------------------------------------------------ */
/* GEMM on decoded FP8 operands, both stored contiguous along the reduction: */
/*   A [m][k], B [n][k];  D[i][j] = sum_k dec(A[i][k]) * dec(B[j][k])        */
/*   y = D * sinv_a * sinv_b + bias[j],  out = gelu(y) or y                  */
/* [MP-KR] "Accumulation into FP32": low-precision products are summed in    */
/* wide precision (here fp64, k ascending).  [PT-VI]'s torch._scaled_mm      */
/* example: two FP8 operands with their scales and an optional bias.         */
/* [TE-RU] section 3: the GEMM result is divided by the scaling factors,     */
/* i.e. multiplied by the inverse scales.                                    */
/* rows == NULL computes all m rows; otherwise only rows[0..n_rows-1], and   */
/* out / out_pre hold n_rows x n values.  out_pre (nullable) gets y.         */
/* ------------------------------------------------------------------------ */

void orc_gemm(const uint8_t* a, int afmt, const uint8_t* b, int bfmt,
              int64_t m, int64_t n, int64_t k, float sinv_a, float sinv_b,
              const double* bias, int gelu, const int64_t* rows, int64_t n_rows,
              double* out_pre, double* out) {
    double ta[256], tb[256];
    for (int c = 0; c < 256; ++c) {
        ta[c] = orc_decode((uint8_t)c, afmt);
        tb[c] = orc_decode((uint8_t)c, bfmt);
    }
    int64_t nr = rows ? n_rows : m;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nr; ++ri) {
        int64_t i = rows ? rows[ri] : ri;
        const uint8_t* ar = a + i * k;
        for (int64_t j = 0; j < n; ++j) {
            const uint8_t* br = b + j * k;
            double d = 0.0;
            for (int64_t kk = 0; kk < k; ++kk) d += ta[ar[kk]] * tb[br[kk]];
            double y = d * (double)sinv_a * (double)sinv_b;
            if (bias) y += bias[j];
            if (out_pre) out_pre[ri * n + j] = y;
            out[ri * n + j] = gelu ? orc_gelu(y) : y;
        }
    }
}

/*
 * The same D exactly, for small finite operands: every E4M3 value is an
 * integer multiple of 2^-9 and every E5M2 value of 2^-16, so the products are
 * integers times 2^-(fa+fb) and the sum is exact in 128-bit integers.
 * D[i][j] = (hi * 2^64 + lo) * 2^exp2 (two's complement across hi:lo).
 * *exp2 is set to INT32_MIN if an operand is NaN or Inf.
 */
void orc_gemm_exact(const uint8_t* a, int afmt, const uint8_t* b, int bfmt,
                    int64_t m, int64_t n, int64_t k, int64_t* hi, uint64_t* lo, int32_t* exp2) {
    int fa = afmt == ORC_E4M3 ? 9 : 16, fb = bfmt == ORC_E4M3 ? 9 : 16;
    int64_t ia[256], ib[256];
    for (int c = 0; c < 256; ++c) {
        double va = orc_decode((uint8_t)c, afmt), vb = orc_decode((uint8_t)c, bfmt);
        ia[c] = isfinite(va) ? (int64_t)ldexp(va, fa) : INT64_MIN;
        ib[c] = isfinite(vb) ? (int64_t)ldexp(vb, fb) : INT64_MIN;
    }
    *exp2 = -(fa + fb);
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            __int128 d = 0;
            for (int64_t kk = 0; kk < k; ++kk) {
                int64_t x = ia[a[i * k + kk]], y = ib[b[j * k + kk]];
                if (x == INT64_MIN || y == INT64_MIN) { *exp2 = INT32_MIN; return; }
                d += (__int128)x * (__int128)y;
            }
            hi[i * n + j] = (int64_t)(d >> 64);
            lo[i * n + j] = (uint64_t)d;
        }
}

/* ------------------------------------------------------------------------ */
/* Loss scaling and the fp32 master-weight update.                           */
/* [MP-KR] "Mixed-Precision Training Iteration": multiply the loss by S,     */
/* back-propagate, multiply the weight gradients by 1/S, update the fp32     */
/* master weights.  [MP-KR] dynamic loss scaling: start with a large S; when */
/* the weight gradients hold Inf or NaN, lower S and skip the update; after  */
/* N iterations without Inf/NaN, raise S.  The pages leave the constants     */
/* open; the caller passes them (reading: S0 = 2^16, x1/2, x2 after N = 5).   */
/* Unscaling happens on the no-overflow path (the extraction's step list     */
/* puts it under the overflow branch; the iteration list before it orders    */
/* unscale -> update).                                                       */
/*                                                                           */
/* state: [0] S, [1] clean iterations, [2] found_inf of the last step (0/1), */
/*        [3] the S the last step's gradients carry.                         */
/* found_inf is read from the amaxes of the step's gradient tensors: the    */
/* amax propagates Inf and NaN, so a non-finite amax means a non-finite      */
/* element.                                                                  */
/* ------------------------------------------------------------------------ */

void orc_loss_scale_update(const float* amaxes, int32_t n, int64_t stride, float* state,
                           int32_t interval, float backoff, float growth) {
    int found = 0;
    for (int32_t i = 0; i < n; ++i)
        if (!isfinite(amaxes[(int64_t)i * stride])) found = 1;
    state[3] = state[0];
    state[2] = (float)found;
    if (found) {
        state[0] = state[0] * backoff;
        state[1] = 0.0f;
    } else {
        state[1] = state[1] + 1.0f;
        if (state[1] >= (float)interval) {
            state[0] = state[0] * growth;
            state[1] = 0.0f;
        }
    }
}

/* w <- fl32(w - fl32(lr * fl32(g * fl32(1/S)))), skipped when found_inf. */
void orc_sgd(float* w, const float* g, int64_t n, float lr, const float* state) {
    if (state[2] != 0.0f) return;
    const float inv = 1.0f / state[3];
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const float u = g[i] * inv;
        const float d = lr * u;
        w[i] = w[i] - d;
    }
}

/* out = round(x * S): the loss-scaled upstream gradient. */
void orc_scale_by(const void* x, int dtype, int64_t n, float s, void* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const float v = load_elem(x, dtype, i) * s;
        if (dtype == ORC_F32) ((float*)out)[i] = v;
        else ((uint16_t*)out)[i] = orc_bf16_from_f32(v);
    }
}
