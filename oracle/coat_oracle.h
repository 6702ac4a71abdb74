/*
 * coat_oracle.h -- CPU reference of COAT's FP8 AdamW optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: it exists so that tests, the smoke check and the benchmark's
 * CPU baseline can compare the GPU library against an independent, plain,
 * double-precision implementation written from the method's definition.  It
 * shares no code, header, table or constant with the GPU library.
 *
 * Sources (cited by page title and section; "[P1]" below):
 *   [P1] "COAT: Compressing Optimizer States and Activation for Memory-Efficient
 *        FP8 Training" -- paper review at xllm-io.github.io, section 三
 *        (technical architecture), sub-section 核心公式 (core formulas):
 *          - equation "FP8量化"           : per-group absmax quantizer Q
 *          - equation "AdamW优化器更新规则" : AdamW with bias correction and
 *                                           decoupled weight decay
 *          - equations under "动态范围扩展": expansion f(x)=sign(x)|x|^k, the
 *            expanded range R_f(X)=(R_X)^k and the optimal k=log_{R_X}(R_E4M3)
 *        section 三 "混合粒度激活量化" (1xG per-group granularity) and
 *        section 四 table (fused optimizer kernel; shard-local ranges).
 *   [OCP] OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding:
 *        bias 7, no infinities, S.1111.111 is NaN, largest finite 448.
 *
 * Readings where the sources leave a step open (each is repeated next to the
 * code that implements it):
 *   - E4M3 is the OCP "FN" variant (max 448); rounding is round-to-nearest-even;
 *     values above 448 saturate to 448.
 *   - R_E4M3 = 448 / 2^-6 (largest finite over smallest normal).
 *   - R_X uses the smallest NONZERO magnitude of the group (zeros need no range).
 *   - The stored per-group scale is s = max|X| of the group before expansion.
 *     Codes are RNE(448 * (|x|/s)^k), which equals Q applied to f(X).
 *   - k is clamped above at 16.  An all-zero group stores scale 0, k 1, codes 0.
 *     A group whose nonzero magnitudes are all equal (R_X = 1) stores k = 16.
 *   - Groups are G consecutive elements of one flat tensor; the last group of a
 *     tensor may be shorter.  G is any positive integer here.
 *   - The fused step dequantizes m and v, runs AdamW in FP32 in the equation's
 *     literal order, updates w from the unquantized moments, and re-quantizes.
 */
#ifndef COAT_ORACLE_H
#define COAT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define COAT_ORACLE_OK 0
#define COAT_ORACLE_EINVAL 1   /* bad size, group size or hyperparameter */
#define COAT_ORACLE_ESTATE 2   /* state holds a NaN code or a nonpositive k */
#define COAT_ORACLE_ENOMEM 3   /* a scratch allocation failed */

/* [OCP] value of one E4M3 code (NaN for 0x7F / 0xFF). */
double coat_oracle_e4m3_decode(uint8_t code);

/* [OCP] nearest E4M3 code to x, ties to even mantissa, saturating at +-448.
 * The sign bit is set for x < 0 (also when the magnitude rounds to zero);
 * -0.0 and +0.0 both give 0x00.  NaN gives 0x7F. */
uint8_t coat_oracle_e4m3_encode(double x);

/* Element-wise loops over the two functions above. */
void coat_oracle_e4m3_encode_array(const double* x, int64_t n, uint8_t* codes);
void coat_oracle_e4m3_decode_array(const uint8_t* codes, int64_t n, double* x);

/* One group: dre=1 chooses k per [P1] eq. for the optimal k; dre=0 forces
 * k = 1 (plain per-group absmax quantizer, [P1] eq. FP8量化). */
int coat_oracle_expand_quantize(const float* x, int64_t n, int32_t group_size,
                                int32_t dre, uint8_t* codes, float* scale,
                                float* k, double* q_out /* may be NULL */);

/* Inverse: x = sign(c) * scale * (|c|/448)^(1/k); scale 0 gives zeros. */
int coat_oracle_dequantize_expand(const uint8_t* codes, const float* scale,
                                  const float* k, int64_t n, int32_t group_size,
                                  float* x);

/* FP32-state AdamW ([P1] eq. AdamW), in place on w, m, v. */
int coat_oracle_adamw_step_fp32(float* w, const uint16_t* grad_bf16, float* m,
                                float* v, int64_t n, float lr, float beta1,
                                float beta2, float eps, float weight_decay,
                                int64_t step);

/* The fused FP8 step, in place on w and on both states.  Optional outputs
 * (NULL to skip): m_t / v_t before re-quantization, and the unrounded code
 * magnitudes q of both states (for near-tie diagnostics). */
int coat_oracle_adamw_fp8_step(float* w, const uint16_t* grad_bf16,
                               uint8_t* m_codes, float* m_scale, float* m_k,
                               uint8_t* v_codes, float* v_scale, float* v_k,
                               int64_t n, int32_t group_size, int32_t dre,
                               float lr, float beta1, float beta2, float eps,
                               float weight_decay, int64_t step,
                               float* m_out, float* v_out,
                               double* qm_out, double* qv_out);

/* Per-group E4M3 quantization of a row-major BF16 activation matrix
 * ([P1] section 三 "混合粒度激活量化": 1xG groups for non-linear layers, and the
 * non-linear-layer kernel's quantized output plus transposed quantized output;
 * [P1] eq. FP8量化 with S = max|X| / 448 per group).  Each code is the E4M3
 * value nearest to the exact quotient x / S = 448 x / max, ties to even
 * (reading of the equation's rounding), with the sign of x (a negative value
 * that rounds to zero gives 0x80; -0.0 gives 0x00); the stored scale is S
 * rounded once to FP32; an all-zero group stores S = 0 and codes 0.  cols
 * must be a multiple of group_size.
 * codes: rows x cols, scales: rows x cols/group_size, codes_t: cols x rows
 * (the transpose of codes; may be NULL). */
int coat_oracle_quantize_act(const uint16_t* x_bf16, int64_t rows, int64_t cols,
                             int32_t group_size, uint8_t* codes, float* scales,
                             uint8_t* codes_t);

/* Group-scaled FP8 linear layer ([P1] section 三, Triton优化内核 / 线性层优化:
 * the GEMM output is reshaped into 1xG groups along N and each group's max is
 * taken; section 四 table, 组缩放技术).  C = (a_scale * b_scale) * A B^T with
 * A: M x K and B: N x K E4M3 codes, row-major (K contiguous).  Reading: C is
 * the real product (the sum over k is exact in integer arithmetic, the scale
 * is applied in double) rounded to FP32, and its 1xG groups along each row go
 * through the same quantizer as the activation quantizer above (exact
 * quotient, ties to even).
 * codes: M x N, scales: M x N/G; c_exact (M x N doubles) and c_f32 (M x N)
 * are optional (NULL to skip).  K <= 2^17; N a multiple of group_size; NaN
 * codes in A or B give COAT_ORACLE_ESTATE. */
int coat_oracle_gemm_fp8_group_quant(const uint8_t* a, const uint8_t* b, float a_scale,
                                     float b_scale, int64_t M, int64_t N, int64_t K,
                                     int32_t group_size, uint8_t* codes, float* scales,
                                     double* c_exact, float* c_f32);

#ifdef __cplusplus
}
#endif
#endif
