// coat_fp8.hip -- gfx950 kernels and C ABI of COAT's fused FP8 AdamW step
// with Dynamic Range Expansion.
//
// Sources (see include/coat_fp8.h for the full citations):
//   [P1] COAT paper review (xllm-io.github.io), section 三 核心公式:
//        quantizer "FP8量化", AdamW "AdamW优化器更新规则", expansion
//        equations under "动态范围扩展"; section 四 table (fused optimizer
//        kernel, shard-local dynamic ranges).
//   [OCP] OFP8 specification, E4M3 (max 448, min normal 2^-6).
//
// Execution model.  The step is an element-wise update plus a per-group
// reduction, bound by HBM bandwidth (about 14 bytes per parameter), so it uses
// no matrix cores.  One 64-lane wavefront owns a "tile" of 1024 consecutive
// elements of one tensor; each lane owns 16 elements of one group, so a group
// of G elements lives in G/16 neighbouring lanes and its max / min reductions
// are 0..3 DPP steps inside registers (see LaneMap for the interleave that
// keeps every memory instruction on whole cache lines).  LDS holds only a
// 2 KB table for dequantization, filled by each block after its waves have
// issued their tiles' loads.  Each wave takes one tile, found by a binary
// search over the launch's tensors, whose descriptors travel in the kernel
// arguments.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "coat_common.h"

namespace coat {

thread_local char g_last_hip_error[256] = "";

coat_status_t hip_fail(hipError_t e) {
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s", hipGetErrorString(e));
  return COAT_ERR_HIP;
}

namespace {
constexpr int kMaxCachedDevices = 64;
std::atomic<int> g_cu_count[kMaxCachedDevices];  // 0: not queried yet
}  // namespace

hipError_t current_cu_count(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxCachedDevices;
  if (cached) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  int c = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (cached) g_cu_count[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return hipSuccess;
}

}  // namespace coat

using namespace coat;

namespace {

constexpr int kElemsPerLane = 16;
constexpr int kTileElems = kWave * kElemsPerLane;  // 1024
// The step kernel's lanes: 16 elements each, as the codec's.  Measured on the
// 7B-shaped shard, 4 per lane (256 per wave, one 16-byte run of w per lane)
// streams 12% slower: the per-wave work (tensor lookup, table fill, group
// constants replicated over 32 lanes) outweighs the finer access pattern.
constexpr int kStepElems = kElemsPerLane;
constexpr int kStepTileElems = kWave * kStepElems;
constexpr int kMaxTensorsPerLaunch = 40;

// [OCP] E4M3: log2 of the largest finite value 448, and log2 of its dynamic
// range 448 / 2^-6 = 7 * 2^12 ([P1] eq. for the optimal k needs R_E4M3).
constexpr float kLog2Max = 8.807354922057604f;     // log2(448)
constexpr float kLog2Range = 14.807354922057604f;  // log2(28672)
constexpr float kMaxK = 16.0f;                     // upper clamp of k

// ------------------------------------------------- dequantization table
// log2(|c| / 448) for every E4M3 magnitude byte, correctly rounded to FP32 at
// compile time ([OCP] E4M3 values: (1 + f/8) 2^(e-7) for e > 0, f 2^-9 for
// e = 0).  Dequantization reads it from LDS instead of taking log2 of the
// decoded code, which is both cheaper and exact to half an FP32 ulp.

constexpr double kLn2 = 0.69314718055994530941723212145818;

// ln(x) for x >= 1: halve to [1, 2), then 2 atanh((x-1)/(x+1)) as a series.
constexpr double cx_ln(double x) {
  int e = 0;
  while (x >= 2.0) {
    x *= 0.5;
    ++e;
  }
  const double z = (x - 1.0) / (x + 1.0);
  const double z2 = z * z;
  double term = z, sum = 0.0;
  for (int n = 0; n < 60; ++n) {
    sum += term / (2 * n + 1);
    term *= z2;
  }
  return 2.0 * sum + e * kLn2;
}

constexpr double cx_log2(double x) { return cx_ln(x) / kLn2; }

struct Log2Table {
  float v[128];
};

constexpr Log2Table make_log2_table() {
  Log2Table t{};
  const double log2_max = cx_log2(7.0) + 6.0;  // log2 448
  t.v[0] = -__builtin_huge_valf();                // code 0: 2^-inf = 0
  for (int b = 1; b < 128; ++b) {
    const int e = b >> 3, f = b & 7;
    const double l = (e == 0) ? cx_log2((double)f) - 9.0
                              : cx_log2(1.0 + f / 8.0) + (e - 7);
    t.v[b] = (float)(l - log2_max);
  }
  t.v[127] = 0.0f;  // NaN code: outside the contract, read as the scale
  return t;
}

__constant__ Log2Table kLog2Table = make_log2_table();

// The same logarithms in double precision, for the exact dequantization of the
// one element per group that decides k (see exact_min_key).
struct Log2TableD {
  double v[128];
};

constexpr Log2TableD make_log2_table_d() {
  Log2TableD t{};
  const double log2_max = cx_log2(7.0) + 6.0;
  for (int b = 1; b < 127; ++b) {
    const int e = b >> 3, f = b & 7;
    const double l = (e == 0) ? cx_log2((double)f) - 9.0
                              : cx_log2(1.0 + f / 8.0) + (e - 7);
    t.v[b] = l - log2_max;
  }
  return t;
}

__constant__ Log2TableD kLog2TableD = make_log2_table_d();

// Taylor coefficients of 2^f = e^(f ln2): (ln2)^i / i!, i = 0..13.  They
// reach the kernel in its arguments (scalar registers): as compile-time
// constants they would be held in vector registers for the whole kernel.
constexpr int kExp2Terms = 14;

void exp2_coefficients(double* c) {
  double t = 1.0;
  for (int i = 0; i < kExp2Terms; ++i) {
    c[i] = t;
    t = t * kLn2 / (i + 1);
  }
}

// 2^a in double: a = n + f with |f| <= 1/2; the degree-13 series leaves a
// relative error below 1e-16 on that interval.
__device__ __forceinline__ double exp2_f64(double a, const double* coef) {
  const double n = __builtin_rint(a);
  const double f = a - n;
  double p = coef[kExp2Terms - 1];
#pragma unroll
  for (int i = kExp2Terms - 2; i >= 0; --i) p = __builtin_fma(p, f, coef[i]);
  return __builtin_ldexp(p, (int)n);
}

// sign(c) * s * (|c|/448)^(1/k) evaluated in double and rounded once to
// FP32: the dequantized value exactly as a double-precision evaluation of the
// definition rounds it ([P1] inverse of FP8量化 and of f).
__device__ __forceinline__ float dequant_exact(uint32_t code, float scale, float k,
                                              const double* coef) {
  const uint32_t mag = code & 0x7Fu;
  if (!(scale > 0.0f) || !(k > 0.0f) || mag == 0u) return 0.0f;
  const double a = kLog2TableD.v[mag] / (double)k;
  const float x = (float)((double)scale * exp2_f64(a, coef));
  return (code & 0x80u) ? -x : x;
}

// b * x + omb * g with both products and the sum rounded to FP32, in that
// order (no fused multiply-add), as [P1]'s AdamW moment update is written.
__device__ __forceinline__ float moment_literal(float b, float x, float omb, float g) {
#pragma clang fp contract(off)
  return b * x + omb * g;
}

// Per-block copy in LDS, indexed by the whole code byte: {log2(|c|/448), sign}.
__device__ __forceinline__ void load_log2_table(float2* tab) {
  const int c = threadIdx.x;  // blockDim.x == 256
  tab[c] = make_float2(kLog2Table.v[c & 0x7F], (c & 0x80) ? -1.0f : 1.0f);
  __syncthreads();
}

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float hw_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two E4M3 bytes of a word (bytes 0,1 or 2,3) as FP32 values, exact.
template <bool kHigh>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHigh);
}


// Group reductions over the G/16 lanes that hold one group (lanes are
// consecutive and the group starts at a multiple of G/16).  Quad steps swap
// lanes 1 and 2 apart; the third step mirrors each 8-lane half row, which
// joins the two quads of a 128-element group.  Every lane ends with the
// group's result.
template <int kLanes>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  if constexpr (kLanes >= 2)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  if constexpr (kLanes >= 4)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  if constexpr (kLanes >= 8)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  return v;
}

template <int kLanes>
__device__ __forceinline__ uint32_t group_min_u32(uint32_t v) {
  if constexpr (kLanes >= 2)
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  if constexpr (kLanes >= 4)
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  if constexpr (kLanes >= 8)
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  return v;
}

// Running statistics of one lane for one moment: max |x| (FP32), and the
// smallest nonzero |x| kept as the key 2*bits(|x|) - 2 modulo 2^32.  The key
// sends +-0 to 0xFFFFFFFE, above every nonzero magnitude (non-negative floats
// order like unsigned integers), so an unsigned min skips zeros ([P1] eq. for
// R_X with the reading "min over nonzero").
struct Stats {
  float max_abs = 0.0f;
  uint32_t min_key = 0xFFFFFFFFu;
  __device__ __forceinline__ void add(float x) {
    max_abs = __builtin_fmaxf(max_abs, fabsf(x));
    min_key = min(min_key, (__float_as_uint(x) << 1) - 2u);
  }
  // Same, with the element's index j < 16 in the low 4 key bits: the minimum
  // then names its element (ordering ignores magnitude differences below
  // 2^-19 relative, which only matters for which element is re-evaluated).
  __device__ __forceinline__ void add_indexed(float x, uint32_t j) {
    max_abs = __builtin_fmaxf(max_abs, fabsf(x));
    min_key = min(min_key, (((__float_as_uint(x) << 1) - 2u) & 0xFFFFFFF0u) | j);
  }
};

constexpr uint32_t kEmptyKey = 0xFFFFFFF0u;  // keys at or above: no nonzero value

// Dequantization constants of one group: x = sign(c) * s * 2^(L(c) / k) with
// L(c) = log2(|c|/448) from the table.  This is s * (|c|/448)^(1/k), the
// inverse of the quantizer followed by the inverse of f ([P1] FP8量化,
// 动态范围扩展).
struct DequantConst {
  float s, rk, c0;
};

__device__ __forceinline__ DequantConst dequant_const(float scale, float k) {
  DequantConst d;
  const bool empty = !(scale > 0.0f) || !(k > 0.0f);
  float rk = hw_rcp(k);
  rk = fmaf(fmaf(-k, rk, 1.0f), rk, rk);  // one Newton step: 1/k to ~0.5 ulp
  // The smallest nonzero code is 2^-9, so L reaches -(9 + log2 448) and the
  // exponent L/k leaves FP32's normal range below k ~ 0.148; such groups
  // shift the exponent up by 64 and the scale down by 2^64.
  const bool shift = rk > 6.7f;
  d.rk = empty ? 1.0f : rk;
  d.c0 = (!empty && shift) ? 64.0f : 0.0f;
  d.s = empty ? 0.0f : (shift ? scale * 0x1p-64f : scale);
  return d;
}

// Magnitude of one element from its table entry (code 0: 2^-inf = 0).
__device__ __forceinline__ float dequant_mag(float l, const DequantConst& d) {
  return d.s * hw_exp2(fmaf(l, d.rk, d.c0));
}

// Quantization constants of one group: q = 2^(k * log2(|x| * P) + C), which
// is 448 * (|x|/s)^k ([P1] f then FP8量化 with S = s^k / 448).
struct QuantConst {
  float p, k, c, scale;
};

__device__ __forceinline__ QuantConst quant_const(uint32_t max_bits, uint32_t min_key) {
  QuantConst q;
  const float s = __uint_as_float(max_bits);
  if (!(s > 0.0f)) {  // empty group: scale 0, k 1, every code 0
    q.p = 0.0f;
    q.k = 1.0f;
    q.c = kLog2Max;
    q.scale = 0.0f;
    return q;
  }
  const float mu = __uint_as_float((min_key >> 1) + 1u);
  // log2(s / mu) = (exponent difference) + log2(mantissa ratio): exact
  // integer part, and a logarithm of a number in (1/2, 2).
  int es, em;
  const float fs = frexpf(s, &es);
  const float fm = frexpf(mu, &em);
  const float lx = (float)(es - em) + hw_log2(fs * hw_rcp(fm));
  // [P1] optimal k: (R_X)^k = R_E4M3; clamped above at 16 (also R_X = 1).
  const float k = (lx > 0.0f) ? fminf(kMaxK, kLog2Range * hw_rcp(lx)) : kMaxK;
  // |x| * P = 2^off * |x| / s; off keeps it inside FP32's normal range for
  // very large or very small groups and for ranges above 2^100.
  const int off = (s > 0x1p100f || lx > 100.0f) ? 64 : (s < 0x1p-100f ? -64 : 0);
  q.p = hw_rcp(ldexpf(s, -off));
  q.k = k;
  q.c = kLog2Max - k * (float)off;
  q.scale = s;
  return q;
}

// |x| * P <= 2^off (1 + 2^-22), so the exponent stays within a few 1e-6 of
// log2 448 at the group max: q <= 448 (1 + 4e-6), which the conversion rounds
// to 448 (values up to 464 round to 448; no clamp needed).
__device__ __forceinline__ float quant_mag(float x, const QuantConst& q) {
  return hw_exp2(fmaf(q.k, hw_log2(fabsf(x) * q.p), q.c));
}

// Pack four signed magnitudes into four E4M3 bytes (round to nearest even).
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// ------------------------------------------------------------- step kernel

struct TensorDesc {
  float* w;
  const uint16_t* g;
  uint8_t* mc;
  float* ms;
  float* mk;
  uint8_t* vc;
  float* vs;
  float* vk;
  int64_t n;
  int64_t tile_end;  // cumulative tile count up to and including this tensor
};

struct StepParams {
  TensorDesc t[kMaxTensorsPerLaunch];
  int64_t total_tiles;
  float b1, b2;        // beta1, beta2
  float omb1, omb2;    // 1 - beta1, 1 - beta2
  // The update lr * (m_t/bc1) / (sqrt(v_t/bc2) + eps) is evaluated as
  // m_t / (sqrt(v_t) * den_a + den_b) with den_a = 1/(sqrt(bc2) * lr/bc1) and
  // den_b = eps / (lr/bc1); lr = 0 uses den_a = 0, den_b = +inf (no update).
  float den_a;
  float den_b;
  float decay;         // 1 - lr * weight_decay
  double exp2_coef[kExp2Terms];  // see exp2_f64
};

// Registers of one lane: E elements.
template <int E>
struct LaneData {
  float w[E];
  uint32_t g[E / 2];   // BF16 pairs
  uint32_t mc[E / 4];  // E4M3 codes, 4 per word
  uint32_t vc[E / 4];
};

// Which elements a lane owns.  A group of G elements belongs to G/16
// neighbouring lanes.  The lanes of each block of B elements (B = G, except
// B = 16 for G = 32) interleave in runs of 4: lane lb of the block owns runs
// q = 0..3 at
//   block_start + q * B/4 + 4 * lb + (0..3),
// so one memory instruction (fixed q) has each block's lanes covering B/4
// consecutive elements: at B = 128 a w access is whole cache lines, not one
// 16-byte piece per 64-byte segment.  Measured on the 7B-shaped shard, B = 32
// (2 lanes, 32-byte pieces) streams 11% slower than B = 128 and 8% slower
// than B = 16 (each lane's 16 elements contiguous), whatever G, so G = 32
// takes B = 16 -- except in dequantize-expand, which writes 4 bytes for every
// byte it reads and runs 21% faster at G = 32 with B = 32.  Register j =
// 4q + r.
constexpr int default_block(int G) { return G == 32 ? 16 : G; }

template <int G, int E = kElemsPerLane, int B = default_block(G)>
struct LaneMap {
  static_assert(G / E >= 1 && G / E <= 8, "a group spans 1 to 8 lanes (the DPP reductions)");
  static_assert(B >= E && B <= G && G % B == 0, "a block of lanes lies inside one group");
  static constexpr int kLanesPerGroup = G / E;
  static constexpr int kBlock = B;
  static constexpr int kLanesPerBlock = kBlock / E;
  static constexpr int kRunStride = kBlock / 4;
  int64_t grp;   // group index inside the tensor
  int64_t base;  // element of register 0
  __device__ __forceinline__ LaneMap(int64_t tile_start, int lane) {
    grp = tile_start / G + lane / kLanesPerGroup;
    base = tile_start + (int64_t)(lane / kLanesPerBlock) * kBlock + 4 * (lane % kLanesPerBlock);
  }
  __device__ __forceinline__ int64_t run(int q) const { return base + (int64_t)kRunStride * q; }
  __device__ __forceinline__ int64_t elem(int j) const { return run(j >> 2) + (j & 3); }
};

constexpr int kExactRounds = 4;

// Where b1*m and (1-b1)*g cancel, m_t's relative error is the dequantized
// value's (a few FP32 ulps, up to ~4e-6 for the smallest codes at small k)
// times |b1*m| / |m_t|, and the expansion multiplies it by k in the code.
// Below this ratio the product can reach one E4M3 code step (6-12%) even at
// k = 16, so such elements are re-evaluated exactly (about 1e-3 of them).
constexpr float kCancelRatio = 0x1p-11f;

// Smallest nonzero |m_t| of the group as a key (2*bits - 2), evaluated
// exactly for the candidate element; elements found to be exact zeros are
// set to 0 in mt[] and skipped.  Returns a key >= kEmptyKey if the group has
// no nonzero value.  `local` is this lane's indexed minimum key (see
// Stats::add_indexed), `approx` the group's.  Control flow is wave-uniform.
template <int G, int E>
__device__ __forceinline__ uint32_t exact_group_min(const LaneData<E>& L, const StepParams& p,
                                                 float sm, float km, uint32_t local,
                                                 uint32_t approx, float (&mt)[E]) {
  constexpr int kLanes = LaneMap<G, E>::kLanesPerGroup;
  uint32_t result = 0xFFFFFFFFu;
  bool done = approx >= kEmptyKey;
  uint32_t excluded = 0u;
  for (int round = 0; round < kExactRounds; ++round) {
    uint32_t key = 0xFFFFFFFFu;
    if (!done && local == approx) {
      const uint32_t j = approx & 0xFu;
      // the element's code byte and BF16 gradient, picked from registers
      uint32_t cw = L.mc[0], gw = L.g[0];
#pragma unroll
      for (int q = 1; q < E / 4; ++q) cw = ((j >> 2) == (uint32_t)q) ? L.mc[q] : cw;
#pragma unroll
      for (int h = 1; h < E / 2; ++h) gw = ((j >> 1) == (uint32_t)h) ? L.g[h] : gw;
      const uint32_t code = (cw >> (8 * (j & 3u))) & 0xFFu;
      const float g = __uint_as_float((j & 1u) ? (gw & 0xFFFF0000u) : (gw << 16));
      const float m = moment_literal(p.b1, dequant_exact(code, sm, km, p.exp2_coef), p.omb1, g);
      if (m == 0.0f) {
        excluded |= 1u << j;
        key = 0xFFFFFFFEu;  // "exact zero" marker, above every real key
      } else {
        key = (__float_as_uint(m) << 1) - 2u;
      }
    }
    key = group_min_u32<kLanes>(key);
    if (!done && key < kEmptyKey) {
      result = key;
      done = true;
    }
    if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
    // rescan this lane without the excluded elements
    if (!done) {
      uint32_t l2 = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (!((excluded >> j) & 1u))
          l2 = min(l2, (((__float_as_uint(mt[j]) << 1) - 2u) & 0xFFFFFFF0u) | (uint32_t)j);
      local = l2;
    }
    approx = group_min_u32<kLanes>(local);
    if (!done && approx >= kEmptyKey) done = true;  // only exact zeros remain
  }
  if (!done) result = approx & 0xFFFFFFF0u;  // rounds exhausted: FP32 minimum
  if (__builtin_amdgcn_ballot_w64(excluded != 0u) != 0) {
#pragma unroll
    for (int j = 0; j < E; ++j)
      if ((excluded >> j) & 1u) mt[j] = 0.0f;
  }
  return result;
}

template <int G, bool kFull, int E>
__device__ __forceinline__ void load_lane(const TensorDesc& T, const LaneMap<G, E>& map, LaneData<E>& L) {
  if constexpr (kFull) {
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      const int64_t e = map.run(q);
      const float4 w = *reinterpret_cast<const float4*>(T.w + e);
      L.w[4 * q] = w.x;
      L.w[4 * q + 1] = w.y;
      L.w[4 * q + 2] = w.z;
      L.w[4 * q + 3] = w.w;
      const uint2 g = *reinterpret_cast<const uint2*>(T.g + e);
      L.g[2 * q] = g.x;
      L.g[2 * q + 1] = g.y;
      L.mc[q] = *reinterpret_cast<const uint32_t*>(T.mc + e);
      L.vc[q] = *reinterpret_cast<const uint32_t*>(T.vc + e);
    }
  } else {
    // Tail tile: element-wise, zero padding past n.  Zeros leave max|x| and
    // the nonzero minimum of a group unchanged.
#pragma unroll
    for (int j = 0; j < E; ++j) L.w[j] = 0.0f;
#pragma unroll
    for (int j = 0; j < E / 2; ++j) L.g[j] = 0u;
#pragma unroll
    for (int j = 0; j < E / 4; ++j) { L.mc[j] = 0u; L.vc[j] = 0u; }
    for (int j = 0; j < E; ++j) {
      const int64_t e = map.elem(j);
      if (e < T.n) {
        L.w[j] = T.w[e];
        L.g[j >> 1] |= (uint32_t)T.g[e] << (16 * (j & 1));
        L.mc[j >> 2] |= (uint32_t)T.mc[e] << (8 * (j & 3));
        L.vc[j >> 2] |= (uint32_t)T.vc[e] << (8 * (j & 3));
      }
    }
  }
}

// kNT: the nontemporal hint on the full-tile stores.  The stand-alone codec
// takes it (measured on MI355X over an 8 GB vector: expand-quantize 3.3%,
// dequantize-expand 1.2% faster, outputs unchanged); the step does not, as
// it gains nothing there.
template <int G, bool kFull, int E = kElemsPerLane, bool kNT = false>
__device__ __forceinline__ void store_codes(uint8_t* base, const LaneMap<G, E>& map, int64_t n,
                                            const uint32_t (&c)[E / 4]) {
  if constexpr (kFull) {
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      if constexpr (kNT)
        __builtin_nontemporal_store(c[q], reinterpret_cast<uint32_t*>(base + map.run(q)));
      else
        *reinterpret_cast<uint32_t*>(base + map.run(q)) = c[q];
    }
  } else {
    for (int j = 0; j < E; ++j) {
      const int64_t e = map.elem(j);
      if (e < n) base[e] = (uint8_t)(c[j >> 2] >> (8 * (j & 3)));
    }
  }
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int G, bool kFull, int E = kElemsPerLane, int B = default_block(G), bool kNT = false>
__device__ __forceinline__ void store_floats(float* base, const LaneMap<G, E, B>& map, int64_t n,
                                             const float (&x)[E]) {
  if constexpr (kFull) {
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      if constexpr (kNT) {
        const f32x4v v = {x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(base + map.run(q)));
      } else {
        *reinterpret_cast<float4*>(base + map.run(q)) =
            make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
      }
    }
  } else {
    for (int j = 0; j < E; ++j) {
      const int64_t e = map.elem(j);
      if (e < n) base[e] = x[j];
    }
  }
}

// One tile of one wave.  kFill: the block's dequantization table is filled
// here, after this wave's loads are issued and before their first use, so the
// table's latency and barrier overlap the loads; every wave of the block must
// then call it, and `have` = false (a wave past the last tile) only fills.
template <int G, bool kFull, bool kFill>
__device__ __forceinline__ void step_lane(const TensorDesc& T, int64_t tile_start, int lane,
                                          const StepParams& p, float2* tab, bool have) {
  constexpr int E = kStepElems;
  constexpr int kLanesPerGroup = LaneMap<G, E>::kLanesPerGroup;
  const LaneMap<G, E> map(tile_start, lane);
  const int64_t grp = map.grp;
  const int64_t ngroups = (T.n + G - 1) / G;
  const bool grp_ok = kFull || grp < ngroups;

  // a1: loads (all issued before any use)
  LaneData<E> L;
  float sm = 0.0f, km = 0.0f, sv = 0.0f, kv = 0.0f;
  if (have) {
    load_lane<G, kFull>(T, map, L);
    if (grp_ok) {
      sm = T.ms[grp];
      km = T.mk[grp];
      sv = T.vs[grp];
      kv = T.vk[grp];
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load of the tile in flight together
  if constexpr (kFill) load_log2_table(tab);
  if (!have) return;

  // a2: dequantize-expand both moments
  const DequantConst dm = dequant_const(sm, km);
  const DequantConst dv = dequant_const(sv, kv);
  float mt[E], vt[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const float2 em = tab[(L.mc[j >> 2] >> (8 * (j & 3))) & 0xFF];
    const float lv = tab[(L.vc[j >> 2] >> (8 * (j & 3))) & 0xFF].x;
    mt[j] = dequant_mag(em.x, dm) * em.y;
    vt[j] = dequant_mag(lv, dv);  // second moment: codes carry no sign
  }

  // a3: moments
  uint32_t cancel = 0u;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const float g = (j & 1) ? bf16_hi(L.g[j >> 1]) : bf16_lo(L.g[j >> 1]);
    const float m = moment_literal(p.b1, mt[j], p.omb1, g);
    cancel |= (fabsf(m) < kCancelRatio * fabsf(p.b1 * mt[j])) ? (1u << j) : 0u;
    vt[j] = fmaf(p.b2, vt[j], p.omb2 * (g * g));
    mt[j] = m;
  }
  // strongly cancelling first moments, exactly (rare: the block is skipped
  // unless some lane of the wave has one)
  if (__builtin_amdgcn_ballot_w64(cancel != 0u) != 0) {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if ((cancel >> j) & 1u) {
        const float g = (j & 1) ? bf16_hi(L.g[j >> 1]) : bf16_lo(L.g[j >> 1]);
        const uint32_t code = (L.mc[j >> 2] >> (8 * (j & 3))) & 0xFFu;
        mt[j] = moment_literal(p.b1, dequant_exact(code, sm, km, p.exp2_coef), p.omb1, g);
      }
    }
  }

  // a4: bias correction, weight update from the unquantized m_t, v_t
  Stats st_m, st_v;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const float den = fmaf(hw_sqrt(vt[j]), p.den_a, p.den_b);
    L.w[j] = fmaf(L.w[j], p.decay, -(mt[j] * hw_rcp(den)));
    st_m.add_indexed(mt[j], (uint32_t)j);
    st_v.add(vt[j]);
  }
  store_floats<G, kFull, E>(T.w, map, T.n, L.w);

  // a5-a7 for the second moment first, so its registers are free for the
  // first moment's exact minimum below.
  {
    const uint32_t v_max = group_max_u32<kLanesPerGroup>(__float_as_uint(st_v.max_abs));
    const uint32_t v_min = group_min_u32<kLanesPerGroup>(st_v.min_key);
    const QuantConst qv = quant_const(v_max, v_min);
    uint32_t ov[E / 4];
#pragma unroll
    for (int q = 0; q < E / 4; ++q)
      ov[q] = pack4(quant_mag(vt[4 * q], qv), quant_mag(vt[4 * q + 1], qv),
                    quant_mag(vt[4 * q + 2], qv), quant_mag(vt[4 * q + 3], qv));
    store_codes<G, kFull, E>(T.vc, map, T.n, ov);
    if ((lane % kLanesPerGroup) == 0 && grp_ok) {
      T.vs[grp] = qv.scale;
      T.vk[grp] = qv.k;
    }
  }

  // a5: first-moment group statistics across the group's lanes.  Its
  // smallest nonzero magnitude sets k, and it is usually the element where
  // b1*m and (1-b1)*g cancel most, so an FP32 rounding difference in its
  // dequantized m is magnified there: the lane holding the group's FP32
  // minimum re-evaluates that one element exactly as the definition rounds it
  // (see exact_group_min).
  const uint32_t m_max = group_max_u32<kLanesPerGroup>(__float_as_uint(st_m.max_abs));
  const uint32_t m_min_approx = group_min_u32<kLanesPerGroup>(st_m.min_key);
  const uint32_t m_min = exact_group_min<G, E>(L, p, sm, km, st_m.min_key, m_min_approx, mt);

  // a6: expansion exponent and scale (a group whose only nonzero values are
  // exact zeros is empty)
  const QuantConst qm = quant_const(m_min < kEmptyKey ? m_max : 0u, m_min);

  // a7: expand, scale, round, pack, store
  uint32_t om[E / 4];
#pragma unroll
  for (int q = 0; q < E / 4; ++q) {
    float a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = mt[4 * q + r];
      a[r] = copysignf(quant_mag(x, qm), x);
    }
    om[q] = pack4(a[0], a[1], a[2], a[3]);
  }
  store_codes<G, kFull, E>(T.mc, map, T.n, om);
  if ((lane % kLanesPerGroup) == 0 && grp_ok) {
    T.ms[grp] = qm.scale;
    T.mk[grp] = qm.k;
  }
}

// kTail = false: the full tiles of every tensor of the launch (the streaming
// kernel).  kTail = true: the one partial last tile of each tensor whose size
// is not a multiple of the tile (tile_end then counts 0 or 1 per tensor).
// The two are separate kernels so that the rarely used element-wise tail code
// does not set the register budget, and so the occupancy, of the main one.
// The launch's tensor holding `tile`: the first whose cumulative tile count
// exceeds it (entries past the launch's tensors hold INT64_MAX, so the array
// is monotone); tile_begin is the tensor's first tile.
__device__ __forceinline__ int find_tensor(const StepParams& p, int64_t tile, int64_t& tile_begin) {
  int lo = 0, hi = kMaxTensorsPerLaunch - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tile < p.t[mid].tile_end) hi = mid; else lo = mid + 1;
  }
  tile_begin = lo > 0 ? p.t[lo - 1].tile_end : 0;
  return lo;
}

template <int G, bool kTail, bool kFill>
__device__ __forceinline__ void step_tile(const StepParams& p, int64_t tile, int lane, float2* tab,
                                          bool have) {
  int64_t tile_begin = 0;
  const TensorDesc& T = p.t[find_tensor(p, have ? tile : 0, tile_begin)];
  if constexpr (!kTail)
    step_lane<G, true, kFill>(T, (tile - tile_begin) * kStepTileElems, lane, p, tab, have);
  else
    step_lane<G, false, kFill>(T, T.n / kStepTileElems * kStepTileElems, lane, p, tab, have);
}

template <int G, bool kTail>
__global__ __launch_bounds__(kBlockThreads) void adamw_fp8_step_kernel(const StepParams p) {
  __shared__ float2 tab[256];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave =
      (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  // The first tile's loads go out before the table fill (every wave takes
  // part in the fill, also one without a tile); later tiles, only when the
  // grid is capped, find the table ready.
  step_tile<G, kTail, true>(p, wave, lane, tab, wave < p.total_tiles);
  for (int64_t tile = wave + nwaves; tile < p.total_tiles; tile += nwaves)
    step_tile<G, kTail, false>(p, tile, lane, tab, true);
}

// ------------------------------------------- stand-alone quantize kernels

struct CodecParams {
  const float* x;  // expand_quantize input / dequantize output
  float* xo;
  uint8_t* codes;
  const uint8_t* codes_in;
  float* scale;
  float* k;
  const float* scale_in;
  const float* k_in;
  int64_t n;
};

template <int G, bool kFull>
__device__ __forceinline__ void quantize_lane(const CodecParams& p, int64_t tile_start, int lane) {
  constexpr int kLanesPerGroup = LaneMap<G>::kLanesPerGroup;
  const LaneMap<G> map(tile_start, lane);
  const int64_t grp = map.grp;
  const bool grp_ok = kFull || grp < (p.n + G - 1) / G;
  float x[16];
  if constexpr (kFull) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(p.x + map.run(q));
      x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
  } else {
    for (int j = 0; j < 16; ++j) {
      const int64_t e = map.elem(j);
      x[j] = (e < p.n) ? p.x[e] : 0.0f;
    }
  }
  Stats st;
#pragma unroll
  for (int j = 0; j < 16; ++j) st.add(x[j]);
  const QuantConst qc = quant_const(group_max_u32<kLanesPerGroup>(__float_as_uint(st.max_abs)),
                                    group_min_u32<kLanesPerGroup>(st.min_key));
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = copysignf(quant_mag(x[4 * q + r], qc), x[4 * q + r]);
    o[q] = pack4(a[0], a[1], a[2], a[3]);
  }
  store_codes<G, kFull, kElemsPerLane, true>(p.codes, map, p.n, o);
  if ((lane % kLanesPerGroup) == 0 && grp_ok) {
    p.scale[grp] = qc.scale;
    p.k[grp] = qc.k;
  }
}

// kFill and have as in step_lane: the block's table is filled after this
// wave's loads are issued.
template <int G, bool kFull, bool kFill>
__device__ __forceinline__ void dequantize_lane(const CodecParams& p, int64_t tile_start, int lane,
                                                float2* tab, bool have) {
  const LaneMap<G, kElemsPerLane, G> map(tile_start, lane);
  const int64_t grp = map.grp;
  const bool grp_ok = have && (kFull || grp < (p.n + G - 1) / G);
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  if (have) {
    if constexpr (kFull) {
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = *reinterpret_cast<const uint32_t*>(p.codes_in + map.run(q));
    } else {
      for (int j = 0; j < 16; ++j) {
        const int64_t e = map.elem(j);
        if (e < p.n) c[j >> 2] |= (uint32_t)p.codes_in[e] << (8 * (j & 3));
      }
    }
  }
  const float s_in = grp_ok ? p.scale_in[grp] : 0.0f;
  const float k_in = grp_ok ? p.k_in[grp] : 0.0f;
  __builtin_amdgcn_sched_barrier(0);  // the loads go out before the table fill
  if constexpr (kFill) load_log2_table(tab);
  if (!have) return;
  const DequantConst d = dequant_const(s_in, k_in);
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float2 e = tab[(c[j >> 2] >> (8 * (j & 3))) & 0xFF];
    x[j] = dequant_mag(e.x, d) * e.y;
  }
  store_floats<G, kFull, kElemsPerLane, G, true>(p.xo, map, p.n, x);
}

// Same split as the step: kTail = false walks the full tiles, kTail = true
// handles the single partial last tile.
template <int G, bool kQuantize, bool kTail>
__global__ __launch_bounds__(kBlockThreads) void codec_kernel(const CodecParams p) {
  __shared__ float2 tab[256];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave =
      (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t tiles = kTail ? 1 : p.n / kTileElems;
  auto start = [&](int64_t tile) {
    return kTail ? p.n / kTileElems * kTileElems : tile * kTileElems;
  };
  if constexpr (kQuantize) {
    for (int64_t tile = wave; tile < tiles; tile += nwaves)
      quantize_lane<G, !kTail>(p, start(tile), lane);
  } else {
    // the first tile's loads go out before the table fill, in which every
    // wave takes part
    dequantize_lane<G, !kTail, true>(p, start(wave < tiles ? wave : 0), lane, tab, wave < tiles);
    for (int64_t tile = wave + nwaves; tile < tiles; tile += nwaves)
      dequantize_lane<G, !kTail, false>(p, start(tile), lane, tab, true);
  }
}

// ------------------------------------------------ element-wise E4M3 cast

__global__ __launch_bounds__(kBlockThreads) void e4m3_encode_kernel(const float* x, int64_t n,
                                                                    uint8_t* codes) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = x[i];
    const float c = copysignf(fminf(fabsf(v), 448.0f), v);  // saturate
    codes[i] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xFF);
  }
}

__global__ __launch_bounds__(kBlockThreads) void e4m3_decode_kernel(const uint8_t* codes, int64_t n,
                                                                    float* x) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    x[i] = __builtin_amdgcn_cvt_f32_fp8((int)codes[i], 0);
}

// ------------------------------------------------------------ host side


// One wave per tile: the grid covers every tile once (the grid-stride loops
// in the kernels then run one iteration).  Measured on MI355X, this streams
// faster than a grid sized to the resident capacity that loops over tiles:
// the dispatcher keeps handing fresh tiles to whichever CU frees up.
hipError_t launch_tiles(const void* fn, int64_t tiles, void* arg, hipStream_t stream) {
  const int64_t want = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 0x7FFFFFFF));
  void* args[] = {arg};
  return hipLaunchKernel(fn, dim3(blocks), dim3(kBlockThreads), args, 0, stream);
}

template <int G>
const void* step_fn(bool tail) {
  return tail ? reinterpret_cast<const void*>(&adamw_fp8_step_kernel<G, true>)
              : reinterpret_cast<const void*>(&adamw_fp8_step_kernel<G, false>);
}

const void* step_kernel_for(int32_t g, bool tail) {
  switch (g) {
    case 16: return step_fn<16>(tail);
    case 32: return step_fn<32>(tail);
    case 64: return step_fn<64>(tail);
    default: return step_fn<128>(tail);
  }
}

template <int G, bool kQuantize>
const void* codec_fn(bool tail) {
  return tail ? reinterpret_cast<const void*>(&codec_kernel<G, kQuantize, true>)
              : reinterpret_cast<const void*>(&codec_kernel<G, kQuantize, false>);
}

template <bool kQuantize>
const void* codec_kernel_for(int32_t g, bool tail) {
  switch (g) {
    case 16: return codec_fn<16, kQuantize>(tail);
    case 32: return codec_fn<32, kQuantize>(tail);
    case 64: return codec_fn<64, kQuantize>(tail);
    default: return codec_fn<128, kQuantize>(tail);
  }
}

coat_status_t check_state(const coat_fp8_state_t& s) {
  if (!s.codes || !s.scale || !s.k) return COAT_ERR_NULL_POINTER;
  if (!aligned(s.codes, 16) || !aligned(s.scale, 4) || !aligned(s.k, 4)) return COAT_ERR_MISALIGNED;
  return COAT_OK;
}

// Launches the full-tile kernel over the first `used` descriptors of p, then
// the tail kernel over the tensors that end in a partial tile.
hipError_t launch_step(StepParams& p, int used, int32_t group_size, hipStream_t stream) {
  int64_t full = 0, tails = 0;
  for (int i = 0; i < used; ++i) {
    full += p.t[i].n / kStepTileElems;
    p.t[i].tile_end = full;
  }
  for (int i = used; i < kMaxTensorsPerLaunch; ++i) p.t[i].tile_end = INT64_MAX;
  p.total_tiles = full;
  if (full > 0) {
    const hipError_t e = launch_tiles(step_kernel_for(group_size, false), full, &p, stream);
    if (e != hipSuccess) return e;
  }
  for (int i = 0; i < used; ++i) {
    tails += (p.t[i].n % kStepTileElems) ? 1 : 0;
    p.t[i].tile_end = tails;
  }
  for (int i = used; i < kMaxTensorsPerLaunch; ++i) p.t[i].tile_end = INT64_MAX;
  p.total_tiles = tails;
  if (tails > 0) return launch_tiles(step_kernel_for(group_size, true), tails, &p, stream);
  return hipSuccess;
}

template <bool kQuantize>
hipError_t launch_codec(const CodecParams& p, int32_t group_size, hipStream_t stream) {
  CodecParams q = p;
  const int64_t full = p.n / kTileElems;
  if (full > 0) {
    const hipError_t e =
        launch_tiles(codec_kernel_for<kQuantize>(group_size, false), full, &q, stream);
    if (e != hipSuccess) return e;
  }
  if (p.n % kTileElems)
    return launch_tiles(codec_kernel_for<kQuantize>(group_size, true), 1, &q, stream);
  return hipSuccess;
}

}  // namespace

extern "C" {

coat_status_t coat_adamw_fp8_step(const coat_adamw_tensor_t* tensors, int32_t num_tensors,
                                  const coat_adamw_hparams_t* hp, hipStream_t stream) {
  if (!hp) return COAT_ERR_NULL_POINTER;
  if (num_tensors < 0) return COAT_ERR_INVALID_VALUE;
  if (num_tensors > 0 && !tensors) return COAT_ERR_NULL_POINTER;
  if (!valid_group_size(hp->group_size)) return COAT_ERR_GROUP_SIZE;
  if (hp->step < 1 || !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) ||
      !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) || !isfinite(hp->lr) || !isfinite(hp->eps) ||
      !isfinite(hp->weight_decay))
    return COAT_ERR_INVALID_VALUE;
  for (int32_t i = 0; i < num_tensors; ++i) {
    const coat_adamw_tensor_t& t = tensors[i];
    if (t.n < 0) return COAT_ERR_INVALID_VALUE;
    if (t.n == 0) continue;
    if (!t.w || !t.grad) return COAT_ERR_NULL_POINTER;
    coat_status_t s = check_state(t.m);
    if (s == COAT_OK) s = check_state(t.v);
    if (s != COAT_OK) return s;
    if (!aligned(t.w, 16) || !aligned(t.grad, 16)) return COAT_ERR_MISALIGNED;
  }

  // [P1] AdamW: bias corrections 1 - beta^t in double, then FP32 constants.
  StepParams p;
  memset(&p, 0, sizeof(p));
  const double bc1 = 1.0 - pow((double)hp->beta1, (double)hp->step);
  const double bc2 = 1.0 - pow((double)hp->beta2, (double)hp->step);
  p.b1 = hp->beta1;
  p.b2 = hp->beta2;
  p.omb1 = 1.0f - hp->beta1;
  p.omb2 = 1.0f - hp->beta2;
  const double lr_bc1 = (double)hp->lr / (double)(float)bc1;
  if (lr_bc1 != 0.0) {
    p.den_a = (float)(1.0 / (sqrt((double)(float)bc2) * lr_bc1));
    p.den_b = (float)((double)hp->eps / lr_bc1);
  } else {
    p.den_a = 0.0f;
    p.den_b = INFINITY;
  }
  p.decay = (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);
  exp2_coefficients(p.exp2_coef);

  int used = 0;
  for (int32_t i = 0; i < num_tensors; ++i) {
    const coat_adamw_tensor_t& t = tensors[i];
    if (t.n == 0) continue;
    TensorDesc& d = p.t[used++];
    d.w = t.w;
    d.g = t.grad;
    d.mc = t.m.codes;
    d.ms = t.m.scale;
    d.mk = t.m.k;
    d.vc = t.v.codes;
    d.vs = t.v.scale;
    d.vk = t.v.k;
    d.n = t.n;
    if (used == kMaxTensorsPerLaunch) {
      const hipError_t e = launch_step(p, used, hp->group_size, stream);
      if (e != hipSuccess) return hip_fail(e);
      used = 0;
    }
  }
  if (used > 0) {
    // descriptors past `used` are never reached: tile < total_tiles
    const hipError_t e = launch_step(p, used, hp->group_size, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return COAT_OK;
}

coat_status_t coat_fp8_expand_quantize(const float* x, int64_t n, int32_t group_size,
                                       coat_fp8_state_t out, hipStream_t stream) {
  if (n < 0) return COAT_ERR_INVALID_VALUE;
  if (!valid_group_size(group_size)) return COAT_ERR_GROUP_SIZE;
  if (n == 0) return COAT_OK;
  if (!x) return COAT_ERR_NULL_POINTER;
  const coat_status_t s = check_state(out);
  if (s != COAT_OK) return s;
  if (!aligned(x, 16)) return COAT_ERR_MISALIGNED;
  CodecParams p;
  memset(&p, 0, sizeof(p));
  p.x = x;
  p.codes = out.codes;
  p.scale = out.scale;
  p.k = out.k;
  p.n = n;
  const hipError_t e = launch_codec<true>(p, group_size, stream);
  return e == hipSuccess ? COAT_OK : hip_fail(e);
}

coat_status_t coat_fp8_dequantize_expand(const uint8_t* codes, const float* scale,
                                         const float* k, int64_t n, int32_t group_size,
                                         float* x, hipStream_t stream) {
  if (n < 0) return COAT_ERR_INVALID_VALUE;
  if (!valid_group_size(group_size)) return COAT_ERR_GROUP_SIZE;
  if (n == 0) return COAT_OK;
  if (!codes || !scale || !k || !x) return COAT_ERR_NULL_POINTER;
  if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(scale, 4) || !aligned(k, 4))
    return COAT_ERR_MISALIGNED;
  CodecParams p;
  memset(&p, 0, sizeof(p));
  p.codes_in = codes;
  p.scale_in = scale;
  p.k_in = k;
  p.xo = x;
  p.n = n;
  const hipError_t e = launch_codec<false>(p, group_size, stream);
  return e == hipSuccess ? COAT_OK : hip_fail(e);
}

coat_status_t coat_e4m3_encode(const float* x, int64_t n, uint8_t* codes, hipStream_t stream) {
  if (n < 0) return COAT_ERR_INVALID_VALUE;
  if (n == 0) return COAT_OK;
  if (!x || !codes) return COAT_ERR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(codes, 16)) return COAT_ERR_MISALIGNED;
  const int64_t blocks = std::min<int64_t>((n + kBlockThreads - 1) / kBlockThreads, 1 << 16);
  hipLaunchKernelGGL(e4m3_encode_kernel, dim3((unsigned)blocks), dim3(kBlockThreads), 0, stream, x,
                     n, codes);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? COAT_OK : hip_fail(e);
}

coat_status_t coat_e4m3_decode(const uint8_t* codes, int64_t n, float* x, hipStream_t stream) {
  if (n < 0) return COAT_ERR_INVALID_VALUE;
  if (n == 0) return COAT_OK;
  if (!x || !codes) return COAT_ERR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(codes, 16)) return COAT_ERR_MISALIGNED;
  const int64_t blocks = std::min<int64_t>((n + kBlockThreads - 1) / kBlockThreads, 1 << 16);
  hipLaunchKernelGGL(e4m3_decode_kernel, dim3((unsigned)blocks), dim3(kBlockThreads), 0, stream,
                     codes, n, x);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? COAT_OK : hip_fail(e);
}

const char* coat_status_string(coat_status_t status) {
  switch (status) {
    case COAT_OK: return "COAT_OK";
    case COAT_ERR_NULL_POINTER: return "COAT_ERR_NULL_POINTER: a required pointer is NULL";
    case COAT_ERR_INVALID_VALUE: return "COAT_ERR_INVALID_VALUE: bad size, step or hyperparameter";
    case COAT_ERR_GROUP_SIZE: return "COAT_ERR_GROUP_SIZE: group_size must be 16, 32, 64 or 128";
    case COAT_ERR_MISALIGNED: return "COAT_ERR_MISALIGNED: arrays must be 16-byte (scale/k 4-byte) aligned";
    case COAT_ERR_HIP: return "COAT_ERR_HIP: a HIP launch failed";
  }
  return "unknown coat_status_t";
}

const char* coat_last_hip_error(void) { return coat::g_last_hip_error; }

int32_t coat_abi_version(void) { return COAT_FP8_ABI_VERSION; }

}  // extern "C"
