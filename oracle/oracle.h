/*
 * CPU oracle for the FP8 linear layer with per-tensor delayed scaling.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and liboracle.so are used by the
 * test-suite, by the smoke check and by the CPU-baseline leg of the benchmark.
 * The product library never includes, links or calls anything in oracle/.
 *
 * Everything here is plain, slow and written to be checked by eye against the
 * pages it cites.  Floating-point arithmetic is fp64 unless a step is defined
 * in fp32 (the scaled product x*s, the scale rule, the fp32 output rounding).
 *
 * Pages cited (titles as published; the short tag is used in oracle.c):
 *   [TE-KR]  "Transformer Engine으로 FP8 사용하기" (coniverse.tistory.com), a
 *            walk-through of FP8 training with Transformer Engine on H100.
 *   [MP-KR]  "LLM) Mixed-Precision 개념 및 학습 방법 알아보기"
 *            (data-newbie.tistory.com), FP16 mixed precision and loss scaling.
 *   [PT-VI]  "Các kiểu dữ liệu FP8 gốc của PyTorch" (hotroai.com), PyTorch's
 *            native FP8 dtypes, torch._scaled_mm and delayed-scaling training.
 *   [TE-RU]  "Как работает FP8 quantization на H100 (Transformer Engine)?"
 *            (aivaro.ru/answers/312).
 */
#ifndef FP8_ORACLE_H
#define FP8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FP8 formats: 0 = OCP E4M3 ("fn": finite + NaN), 1 = OCP E5M2 (IEEE-like). */
enum { ORC_E4M3 = 0, ORC_E5M2 = 1 };
/* Element types of high-precision tensors. */
enum { ORC_F32 = 0, ORC_BF16 = 1 };
/* Minifloat styles for the generic codec. */
enum { ORC_STYLE_IEEE = 0, ORC_STYLE_FN = 1 };

/* ---- generic minifloat codec (any exponent / mantissa width up to 8 / 23) ---- */
uint32_t orc_mf_encode(float p, int ebits, int mbits, int style, int saturate);
double   orc_mf_decode(uint32_t code, int ebits, int mbits, int style);
double   orc_mf_max(int ebits, int mbits, int style);
void     orc_mf_encode_array(const float* p, int64_t n, int ebits, int mbits, int style, int saturate,
                             uint32_t* out);
void     orc_mf_decode_array(const uint32_t* code, int64_t n, int ebits, int mbits, int style, double* out);

/* ---- FP8 codec ---- */
double   orc_fp8_max(int fmt);
double   orc_decode(uint8_t code, int fmt);
uint8_t  orc_encode(float p, int fmt);
uint8_t  orc_encode_bruteforce(float p, int fmt);
void     orc_encode_array(const float* p, int64_t n, int fmt, uint8_t* out);
void     orc_encode_bits_range(uint64_t first_bits, int64_t n, int fmt, uint8_t* out);
void     orc_encode_bruteforce_array(const float* p, int64_t n, int fmt, uint8_t* out);

/* ---- rounding of outputs ---- */
uint16_t orc_bf16_from_f32(float v);
uint16_t orc_bf16_from_f64(double v);
float    orc_f32_from_f64(double v);
void     orc_bf16_from_f32_array(const float* v, int64_t n, uint16_t* out);
void     orc_bf16_from_f64_array(const double* v, int64_t n, uint16_t* out);
void     orc_f32_from_f64_array(const double* v, int64_t n, float* out);

/* ---- amax, scale rule, history ---- */
float    orc_amax(const void* x, int dtype, int64_t n);
void     orc_scale_update(float* hist, float* scale, float* scale_inv, const uint8_t* fmt,
                          int32_t n_tensors, int32_t hist_len, int32_t margin);

/* ---- cast, cast-transpose, dequant, column sums ---- */
void     orc_cast(const void* x, int dtype, int64_t n, int fmt, float scale, uint8_t* q);
int64_t  orc_count_saturated(const void* x, int dtype, int64_t n, int fmt, float scale);
void     orc_cast_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int fmt,
                            float scale, uint8_t* q, uint8_t* q_t);
void     orc_transpose_u8(const uint8_t* q, int64_t rows, int64_t cols, uint8_t* q_t);
void     orc_dequant(const uint8_t* q, int fmt, int64_t n, float scale_inv, void* out, int out_dtype);
void     orc_colsum(const void* x, int dtype, int64_t rows, int64_t cols, double* out);

/* ---- GEMM on decoded FP8 operands ---- */
void     orc_gemm(const uint8_t* a, int afmt, const uint8_t* b, int bfmt,
                  int64_t m, int64_t n, int64_t k, float sinv_a, float sinv_b,
                  const double* bias, int gelu, const int64_t* rows, int64_t n_rows,
                  double* out_pre, double* out);
void     orc_gemm_exact(const uint8_t* a, int afmt, const uint8_t* b, int bfmt,
                        int64_t m, int64_t n, int64_t k, int64_t* hi, uint64_t* lo, int32_t* exp2);

/* ---- GeLU (exact erf form) ---- */
double   orc_gelu(double z);
double   orc_gelu_grad(double z);
void     orc_gelu_bwd(const void* dh, const void* z, int dtype, int64_t n, void* dz);

/* ---- loss scaling and SGD on fp32 masters ---- */
void     orc_loss_scale_update(const float* amaxes, int32_t n, int64_t stride, float* state,
                               int32_t interval, float backoff, float growth);
void     orc_sgd(float* w, const float* g, int64_t n, float lr, const float* state);
void     orc_scale_by(const void* x, int dtype, int64_t n, float s, void* out);

int      orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
