/*
 * coat_fp8.h -- C ABI of the MI355X (gfx950) FP8 AdamW optimizer step with
 * Dynamic Range Expansion (COAT, arXiv:2410.19313).
 *
 * Sources, cited by page and section:
 *   [P1] "COAT: Compressing Optimizer States and Activation for Memory-Efficient
 *        FP8 Training", paper review at xllm-io.github.io.  Section 三
 *        (技术架构) / 核心公式: quantizer equation "FP8量化", AdamW equation
 *        "AdamW优化器更新规则", expansion equations under "动态范围扩展"
 *        (f(x) = sign(x)|x|^k, R_f(X) = (R_X)^k, optimal k = log_{R_X} R_E4M3).
 *        Section 四 table: the optimizer state update is one fused kernel, and
 *        under FSDP each GPU handles its own shard with no cross-GPU range sync.
 *   [OCP] OCP 8-bit Floating Point Specification (OFP8): E4M3, bias 7,
 *        largest finite 448, smallest normal 2^-6, no infinities.
 *
 * State layout (one "moment" = m or v of one tensor of n elements, group size G):
 *   codes[n]            E4M3 codes, element i in byte i.  Sign in bit 7.
 *   scale[ceil(n/G)]    FP32: the group's max |x| before expansion.  0 marks an
 *                       all-zero group (k is then ignored).
 *   k[ceil(n/G)]        FP32: the group's expansion exponent, 0 < k <= 16.
 * Group j covers elements [j*G, min(n, (j+1)*G)).  Groups never cross tensors.
 * A value is stored as code = RNE_E4M3(448 * (|x|/scale)^k) with the sign of x
 * and read back as x = sign(code) * scale * (|code|/448)^(1/k).  Fresh state is
 * all-zero bytes (scale 0 everywhere).
 *
 * Conventions for every entry point:
 *   - Every array argument is DEVICE memory owned by the caller.  The library
 *     allocates nothing, keeps no per-call state, never synchronizes and never
 *     copies host<->device.  Host structs passed by pointer are read during the
 *     call only.
 *   - Work is enqueued on `stream` (0 = the null stream); results are valid
 *     once the caller synchronizes with that stream.
 *   - Arrays must not alias each other.  Codes, FP32 and BF16 element arrays
 *     must be 16-byte aligned; scale and k arrays 4-byte aligned.
 *   - Validation runs before anything is enqueued: any status other than
 *     COAT_ERR_HIP means nothing was launched and no buffer was touched.
 *     COAT_ERR_HIP means a launch failed (earlier launches of the same call may
 *     have run; the state is then undefined).
 *   - n == 0 is a successful no-op (pointers may then be NULL).
 *   - NaN or Inf in inputs is outside the contract.  Exactness (parity with the
 *     CPU reference to the documented tolerance) holds for groups whose
 *     dynamic range max|x| / min-nonzero|x| is at most 2^157.
 */
#ifndef COAT_FP8_H
#define COAT_FP8_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COAT_FP8_ABI_VERSION 1

typedef enum coat_status {
  COAT_OK = 0,
  COAT_ERR_NULL_POINTER = 1,  /* a required pointer is NULL                 */
  COAT_ERR_INVALID_VALUE = 2, /* negative size, bad hyperparameter or step  */
  COAT_ERR_GROUP_SIZE = 3,    /* group_size not in {16, 32, 64, 128}         */
  COAT_ERR_MISALIGNED = 4,    /* an array violates the alignment rule above */
  COAT_ERR_HIP = 5            /* a HIP launch failed                        */
} coat_status_t;

/* One quantized moment (see "State layout"). */
typedef struct coat_fp8_state {
  uint8_t* codes;
  float* scale;
  float* k;
} coat_fp8_state_t;

/* One parameter tensor of an optimizer shard. */
typedef struct coat_adamw_tensor {
  float* w;              /* n FP32 master weights, updated in place      */
  const uint16_t* grad;  /* n BF16 gradient bit patterns, read only      */
  coat_fp8_state_t m;    /* first moment, updated in place               */
  coat_fp8_state_t v;    /* second moment, updated in place              */
  int64_t n;             /* number of elements, >= 0                     */
} coat_adamw_tensor_t;

typedef struct coat_adamw_hparams {
  float lr;           /* eta, finite                                       */
  float beta1;        /* in [0, 1)                                         */
  float beta2;        /* in [0, 1)                                         */
  float eps;          /* added to sqrt(v_hat), finite                      */
  float weight_decay; /* lambda, decoupled: w -= lr * lambda * w, finite   */
  int64_t step;       /* t of this update, >= 1; the caller increments it  */
  int32_t group_size; /* G in {16, 32, 64, 128}                            */
} coat_adamw_hparams_t;

/*
 * One fused AdamW step over a list of tensors ([P1] section 四: fused
 * optimizer kernel; [P1] 核心公式 AdamW, FP8量化 and 动态范围扩展).
 * Per group: dequantize m and v (invert the quantizer, then f), apply
 *   m_t = b1 m + (1-b1) g,  v_t = b2 v + (1-b2) g^2,
 *   w  <- w - lr ( (m_t/(1-b1^t)) / (sqrt(v_t/(1-b2^t)) + eps) + wd w ),
 * using the unquantized m_t and v_t, then store m_t and v_t again with a
 * fresh scale = max|x| and k = min(16, log2(448/2^-6) / log2(max|x|/min|x|))
 * (min over nonzero |x|; k = 16 when all nonzero magnitudes are equal).
 * The step is shard-local: it reads and writes only the given tensors.
 * Errors: COAT_ERR_NULL_POINTER (tensors/hp NULL, or a pointer of a tensor
 * with n > 0), COAT_ERR_INVALID_VALUE (num_tensors < 0, n < 0, step < 1,
 * beta outside [0,1), non-finite lr/eps/weight_decay), COAT_ERR_GROUP_SIZE,
 * COAT_ERR_MISALIGNED, COAT_ERR_HIP.
 */
coat_status_t coat_adamw_fp8_step(const coat_adamw_tensor_t* tensors,
                                  int32_t num_tensors,
                                  const coat_adamw_hparams_t* hp,
                                  hipStream_t stream);

/*
 * Expand and quantize an FP32 vector into a fresh state ([P1] 核心公式:
 * FP8量化 applied per group to f(X) with the group's optimal k).  Used to
 * convert FP32 optimizer states (e.g. a checkpoint) into FP8 state.
 * x: n FP32 values (read only).  out: codes[n], scale/k[ceil(n/G)] (written).
 * Errors: NULL_POINTER, INVALID_VALUE (n < 0), GROUP_SIZE, MISALIGNED, HIP.
 */
coat_status_t coat_fp8_expand_quantize(const float* x, int64_t n,
                                       int32_t group_size, coat_fp8_state_t out,
                                       hipStream_t stream);

/*
 * Dequantize and un-expand a state into FP32 ([P1] 核心公式: inverse of the
 * quantizer, then of f): x = sign(c) * scale * (|c|/448)^(1/k); a group with
 * scale 0 reads as zeros.  codes/scale/k read only; x[n] written.
 * Errors: NULL_POINTER, INVALID_VALUE (n < 0), GROUP_SIZE, MISALIGNED, HIP.
 */
coat_status_t coat_fp8_dequantize_expand(const uint8_t* codes,
                                         const float* scale, const float* k,
                                         int64_t n, int32_t group_size,
                                         float* x, hipStream_t stream);

/*
 * Plain OCP E4M3 conversion, element-wise ([OCP]; the rounding step the
 * quantizer ends in): codes[i] = round-to-nearest-even(x[i]), saturating at
 * +-448, sign kept (a negative value that rounds to zero gives 0x80).
 * Errors: NULL_POINTER, INVALID_VALUE (n < 0), MISALIGNED, HIP.
 */
coat_status_t coat_e4m3_encode(const float* x, int64_t n, uint8_t* codes,
                               hipStream_t stream);

/* Inverse of the above: x[i] = value of codes[i] (NaN for 0x7F / 0xFF). */
coat_status_t coat_e4m3_decode(const uint8_t* codes, int64_t n, float* x,
                               hipStream_t stream);

/*
 * Per-group FP8 quantization of an activation matrix, with its transpose
 * ([P1] section 三, 混合粒度激活量化: non-linear layers quantize per 1xG
 * group; Triton优化内核 / 非线性层优化: that kernel also writes the transposed
 * FP8 tensor the backward pass reads; [P1] 核心公式 FP8量化 with
 * S = max|X| / 448).  No range expansion (k = 1).
 *   x        rows x cols BF16 values (bit patterns), row-major (read only).
 *   codes    rows x cols E4M3 codes, row-major (written).
 *   scales   rows x (cols / group_size) FP32, row-major (written): group
 *            (i, j) covers x[i, j*G .. j*G+G-1] and stores S = max|x| / 448
 *            (IEEE division; 0 for an all-zero group).
 *   codes_t  cols x rows E4M3 codes, the transpose of `codes` (written), or
 *            NULL to skip it.
 * Each code is the E4M3 rounding (nearest, ties to even) of the exact
 * quotient 448 x / max|x|: the kernel forms it in FP32 with one residual
 * correction, which lands on every E4M3 value and midpoint exactly, and for
 * BF16 x no quotient lies close enough to a midpoint for the remaining error
 * to change a code.  Groups with max < 2^-100 are pre-scaled by 2^64.
 * -0 gives code 0x00, a negative x that rounds to zero 0x80, an all-zero
 * group codes 0.
 * cols must be a multiple of group_size.  x, codes and codes_t 16-byte
 * aligned, scales 4-byte aligned; writes into codes_t are 16, 8 or 4 bytes
 * wide when rows is a multiple of 16, 8 or 4, bytes otherwise.
 * Errors: NULL_POINTER (x/codes/scales NULL with rows, cols > 0),
 * INVALID_VALUE (rows or cols < 0, cols % group_size != 0, more than 2^31-1
 * tiles of 128 x 128), GROUP_SIZE, MISALIGNED, HIP.
 */
coat_status_t coat_fp8_quantize_act(const uint16_t* x, int64_t rows,
                                    int64_t cols, int32_t group_size,
                                    uint8_t* codes, float* scales,
                                    uint8_t* codes_t, hipStream_t stream);

/*
 * Group-scaled FP8 linear layer ([P1] section 三, Triton优化内核 / 线性层优化:
 * the GEMM output viewed as (BLOCK_M, BLOCK_N/G, G) with the max taken along
 * the last axis; section 四 table, 组缩放技术: a two-stage max reduction fused
 * into the producing operation; [P1] 核心公式 FP8量化 with S = max|X| / 448).
 *   C = s * A B^T with s = a_scale * b_scale, accumulated in FP32 on the
 *   matrix cores as c = A B^T, then each 1xG group of a row of C is
 *   quantized from C = fl(c s): S = max|C| / 448 (max|C| = fl(max|c| * |s|)
 *   exactly, rounding being monotone) and each code the E4M3 rounding of
 *   448 C / max|C|, formed as in coat_fp8_quantize_act but from the
 *   hardware reciprocal of max/512 (exact at every E4M3 value and midpoint;
 *   elsewhere a code can differ from the exact quotient's only for a
 *   quotient within about 2^-21 relative of a midpoint).  -0 -> 0x00, an all-zero group -> S = 0
 *   and codes 0; groups whose max lies below 2^-100 take the 2^64 pre-scale.
 *   a        M x K E4M3 codes, row-major (read only).
 *   b        N x K E4M3 codes, row-major (read only): the weight of a linear
 *            layer y = x W^T in its usual [out, in] layout.
 *   a_scale, b_scale  per-tensor scales, finite; their product s is
 *            rounded to FP32 once.
 *   codes    M x N E4M3 codes, row-major (written).
 *   scales   M x (N / group_size) FP32, row-major (written).
 *   c_f32    optional M x N FP32 fl(c s) before quantization (written), or NULL.
 * N and K must be multiples of 128, K <= 2^24; M is any size >= 0 (M or N
 * zero is a no-op; K zero gives C = 0, and a, b may then be NULL).  a, b,
 * codes and c_f32 16-byte aligned, scales 4-byte aligned.  NaN codes in a or
 * b are outside the contract.
 * Errors: NULL_POINTER, INVALID_VALUE (negative sizes, N or K not a multiple
 * of 128, K > 2^24, non-finite scales, grid too large), GROUP_SIZE,
 * MISALIGNED, HIP.
 */
coat_status_t coat_fp8_gemm_group_quant(const uint8_t* a, const uint8_t* b,
                                        float a_scale, float b_scale,
                                        int64_t M, int64_t N, int64_t K,
                                        int32_t group_size, uint8_t* codes,
                                        float* scales, float* c_f32,
                                        hipStream_t stream);

/*
 * The same FP8 GEMM with a plain epilogue: C = (a_scale * b_scale) * A B^T
 * rounded to BF16 (nearest even), c_bf16 M x N row-major (written).  It is
 * the reference point for the cost of the group-scaled epilogue above.
 * Arguments, layout and errors as above (no group_size).
 */
coat_status_t coat_fp8_gemm_bf16(const uint8_t* a, const uint8_t* b,
                                 float a_scale, float b_scale, int64_t M,
                                 int64_t N, int64_t K, uint16_t* c_bf16,
                                 hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* coat_status_string(coat_status_t status);

/* HIP error string of the last COAT_ERR_HIP returned on the calling thread
 * (empty string if none). */
const char* coat_last_hip_error(void);

/* COAT_FP8_ABI_VERSION of the loaded library. */
int32_t coat_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* COAT_FP8_H */
