// coat_common.h -- internal declarations shared by the library's HIP sources
// (not part of the C ABI, which is include/coat_fp8.h).
#ifndef COAT_COMMON_H
#define COAT_COMMON_H

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "coat_fp8.h"

namespace coat {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWave * kWavesPerBlock;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

inline bool valid_group_size(int32_t g) { return g == 16 || g == 32 || g == 64 || g == 128; }

// Records hipGetErrorString(e) for coat_last_hip_error() on the calling
// thread and returns COAT_ERR_HIP.
__attribute__((visibility("hidden"))) coat_status_t hip_fail(hipError_t e);

// Compute units of the calling thread's current device.  The attribute query
// costs microseconds, as long as a small kernel, so the count is cached per
// device after its first query (a constant of the device, not call state).
__attribute__((visibility("hidden"))) hipError_t current_cu_count(int* cus);

// BF16 values held in the low / high half of a 32-bit word, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Max over the kLanes neighbouring lanes of a group inside a 16-lane DPP row
// (kLanes a power of two up to 16, groups aligned to kLanes): quad swaps of 1
// and 2 lanes, the half-row mirror (joins two quads) and the row mirror
// (joins two halves).  Every lane of the group ends with the group's max.
template <int kLanes>
__device__ __forceinline__ uint32_t lanes_max_u32(uint32_t v) {
  static_assert(kLanes == 1 || kLanes == 2 || kLanes == 4 || kLanes == 8 || kLanes == 16,
                "group inside one DPP row");
  if constexpr (kLanes >= 2)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  if constexpr (kLanes >= 4)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  if constexpr (kLanes >= 8)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  if constexpr (kLanes >= 16)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return v;
}

// The quotient x / S = 448 x / max of the per-group E4M3 quantizers ([P1]
// FP8量化, S = max / 448), close enough to the exact one that its E4M3
// rounding (round to nearest even) is the exact quotient's.  With
// a = x * (7/8) pre and b = max * pre / 512 (pre = 2^64 for max < 2^-100,
// else 1; both products exact for x with up to 21 significant bits), a / b
// is the quotient.  q0 = a * r with r = fl(1/b) is within two ulps of it.
// When a / b is itself a float -- every E4M3 value and midpoint is one --
// the residual a - q0 * b = (a/b - q0) * b is exact in one FMA and
// q1 = q0 + residual * r lands on a / b exactly, so ties are decided as
// ties.  Otherwise q1 is within about half an ulp of a / b: for BF16 x and
// max, a / b lies at least 2^-13 (relative) from any midpoint (448 x has 11
// significant bits, midpoint * max 13), so q1 rounds to the same code; for
// FP32 x the two can differ only within ~2^-23 of a midpoint.  Signed
// zeros need no extra step: for x = -0.0, q0 = -0, the residual is
// +0 + (-0) = +0 and q1 = +0 + (-0) = +0 (code 0x00), while a negative x
// whose quotient underflows keeps its sign through both FMAs (0x80).
struct GroupQuot {
  float c, b, r;
};

__device__ __forceinline__ GroupQuot group_quot_setup(float amax) {
  const float pre = amax < 0x1p-100f ? 0x1p64f : 1.0f;
  GroupQuot d;
  d.c = 0.875f * pre;
  d.b = amax * pre * 0x1p-9f;
  d.r = 1.0f / d.b;
  return d;
}

__device__ __forceinline__ float group_quot(float x, float c, float b, float r) {
#pragma clang fp contract(off)
  const float a = x * c;
  const float q0 = a * r;
  return __builtin_fmaf(__builtin_fmaf(-q0, b, a), r, q0);
}

__device__ __forceinline__ float group_quot(float x, const GroupQuot& d) {
  return group_quot(x, d.c, d.b, d.r);
}

// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).
// Maps launch index b to a tile index so that each XCD takes one contiguous
// run of tiles (a bijection on [0, nb) for any nb).
__device__ __forceinline__ int64_t xcd_contiguous(int64_t b, int64_t nb) {
  const int64_t q = nb / 8, r = nb % 8;
  const int64_t xcd = b % 8, local = b / 8;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

}  // namespace coat

#endif  // COAT_COMMON_H
