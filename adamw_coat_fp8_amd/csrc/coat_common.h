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

// BF16 values held in the low / high half of a 32-bit word, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace coat

#endif  // COAT_COMMON_H
