// coat_stream_ceiling.hip -- measurement kernels, built into libcoat_bench.so
// (not part of the library's C ABI in include/coat_fp8.h).
//
// The two plainest streams over one contiguous buffer: a read-only stream
// and a write-only stream.  They bound what any kernel can reach on this GPU
// for traffic that only reads or only writes, beside the fused step, whose
// traffic is a mix of 8 bytes read and 6 written per parameter.
//
// A block of 256 threads covers 16 KB: each lane takes four 16-byte chunks
// 4 KB apart, so every wave-wide access is 1 KB of consecutive bytes, and
// the four loads of a lane are issued before any is used.  Past the end of
// the buffer the read stream re-reads the last chunk (the load stays
// unconditional) and the write stream stores nothing.

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kChunks = 4;
constexpr int64_t kBlockChunks = (int64_t)kThreads * kChunks;

// XOR of every loaded word; a lane writes its result to sink only when it
// equals the run-time `magic`, so the loads cannot be dropped and the sink
// (kThreads words) is almost never written.
__global__ __launch_bounds__(kThreads) void read_stream_kernel(const uint4* src, int64_t n16,
                                                               uint32_t magic, uint32_t* sink) {
  const int64_t base = (int64_t)blockIdx.x * kBlockChunks + threadIdx.x;
  uint4 v[kChunks];
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    const int64_t i = base + (int64_t)q * kThreads;
    v[q] = src[i < n16 ? i : n16 - 1];
  }
  uint32_t acc = 0;
#pragma unroll
  for (int q = 0; q < kChunks; ++q) acc ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
  if (acc == magic) sink[threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void write_stream_kernel(uint4* dst, int64_t n16,
                                                                uint32_t value) {
  const int64_t base = (int64_t)blockIdx.x * kBlockChunks + threadIdx.x;
  const uint4 v = make_uint4(value, value, value, value);
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    const int64_t i = base + (int64_t)q * kThreads;
    if (i < n16) dst[i] = v;
  }
}

int stream_blocks(int64_t bytes, int64_t* n16, unsigned* blocks) {
  if (bytes < 16 || bytes % 16) return 1;
  *n16 = bytes / 16;
  const int64_t b = (*n16 + kBlockChunks - 1) / kBlockChunks;
  if (b > 0x7FFFFFFF) return 1;
  *blocks = (unsigned)b;
  return 0;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, at least 16) of device memory at src
// (16-byte aligned); sink holds 256 words of device memory.  Returns 0, 1
// for bad arguments (nothing launched), or 2 + the HIP error.
int coat_bench_read_stream(const void* src, int64_t bytes, uint32_t magic, uint32_t* sink,
                           hipStream_t stream) {
  int64_t n16 = 0;
  unsigned blocks = 0;
  if (!src || !sink || (uintptr_t)src % 16 || stream_blocks(bytes, &n16, &blocks)) return 1;
  const uint4* s = static_cast<const uint4*>(src);
  void* args[] = {&s, &n16, &magic, &sink};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&read_stream_kernel),
                                       dim3(blocks), dim3(kThreads), args, 0, stream);
  return e == hipSuccess ? 0 : 2 + (int)e;
}

// Writes `value` to every 32-bit word of `bytes` (a multiple of 16, at least
// 16) of device memory at dst (16-byte aligned).  Returns as above.
int coat_bench_write_stream(void* dst, int64_t bytes, uint32_t value, hipStream_t stream) {
  int64_t n16 = 0;
  unsigned blocks = 0;
  if (!dst || (uintptr_t)dst % 16 || stream_blocks(bytes, &n16, &blocks)) return 1;
  uint4* d = static_cast<uint4*>(dst);
  void* args[] = {&d, &n16, &value};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&write_stream_kernel),
                                       dim3(blocks), dim3(kThreads), args, 0, stream);
  return e == hipSuccess ? 0 : 2 + (int)e;
}

}  // extern "C"
