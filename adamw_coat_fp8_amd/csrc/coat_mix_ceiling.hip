// coat_mix_ceiling.hip -- a measurement kernel, built into libcoat_bench.so
// (not part of the library's C ABI in include/coat_fp8.h).
//
// It moves exactly the traffic of one fused FP8 AdamW step over a flat
// optimizer shard, with the step kernel's access pattern and no arithmetic:
// per element it reads w (FP32), the BF16 gradient and the m and v codes and
// writes w and both codes back; per group it reads and writes the scale and k
// of both moments (14 + 32/G bytes per parameter).  One 64-lane wave owns a
// tile of 1024 consecutive elements, each lane 16 elements of one group in
// four runs of 4, interleaved over blocks of B = G elements (B = 16 for
// G = 32) exactly as the step kernel lays out its lanes, and all of a tile's
// loads are issued before the first store.  The values written back are the
// values read, combined with a run-time mask of zero through integer XOR, so
// the shard is unchanged and the compiler cannot drop a load.  Its rate is
// the streaming ceiling of the step's own read/write mix on this GPU.

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;
constexpr int kWavesPerBlock = kBlockThreads / kWave;
constexpr int kTileElems = kWave * 16;

struct MixParams {
  uint32_t* w;
  const uint16_t* g;
  uint8_t* mc;
  uint8_t* vc;
  uint32_t* ms;
  uint32_t* mk;
  uint32_t* vs;
  uint32_t* vk;
  int64_t tiles;
  int64_t ngroups;
  uint32_t mask;  // 0 at run time: the XORs below leave every value as read
};

template <int G>
__global__ __launch_bounds__(kBlockThreads) void mix_ceiling_kernel(const MixParams p) {
  constexpr int kBlock = G == 32 ? 16 : G;
  constexpr int kLanesPerBlock = kBlock / 16;
  constexpr int kRunStride = kBlock / 4;
  constexpr int kLanesPerGroup = G / 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t tile =
      (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (tile >= p.tiles) return;
  const int64_t start = tile * kTileElems;
  const int64_t base = start + (int64_t)(lane / kLanesPerBlock) * kBlock + 4 * (lane % kLanesPerBlock);
  int64_t grp = start / G + lane / kLanesPerGroup;
  grp = grp < p.ngroups ? grp : p.ngroups - 1;

  uint4 w[4];
  uint2 g[4];
  uint32_t mc[4], vc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t e = base + (int64_t)kRunStride * q;
    w[q] = *reinterpret_cast<const uint4*>(p.w + e);
    g[q] = *reinterpret_cast<const uint2*>(p.g + e);
    mc[q] = *reinterpret_cast<const uint32_t*>(p.mc + e);
    vc[q] = *reinterpret_cast<const uint32_t*>(p.vc + e);
  }
  uint32_t meta[4] = {p.ms[grp], p.mk[grp], p.vs[grp], p.vk[grp]};
  __builtin_amdgcn_sched_barrier(0);  // every load of the tile in flight together

  const uint32_t m = p.mask;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t e = base + (int64_t)kRunStride * q;
    const uint32_t gm = (g[q].x ^ g[q].y) & m;
    *reinterpret_cast<uint4*>(p.w + e) = make_uint4(w[q].x ^ gm, w[q].y ^ gm, w[q].z ^ gm, w[q].w ^ gm);
    *reinterpret_cast<uint32_t*>(p.mc + e) = mc[q] ^ (vc[q] & m);
    *reinterpret_cast<uint32_t*>(p.vc + e) = vc[q] ^ (mc[q] & m);
  }
  if (lane % kLanesPerGroup == 0) {
    p.ms[grp] = meta[0] ^ (meta[1] & m);
    p.mk[grp] = meta[1] ^ (meta[2] & m);
    p.vs[grp] = meta[2] ^ (meta[3] & m);
    p.vk[grp] = meta[3] ^ (meta[0] & m);
  }
}

template <int G>
const void* mix_fn() {
  return reinterpret_cast<const void*>(&mix_ceiling_kernel<G>);
}

}  // namespace

extern "C" {

// Runs the math-free copy over the first n_tiles * 1024 elements of a flat
// shard (w, g, codes 16-byte aligned; n_groups entries of scale and k).
// Returns 0, 1 for bad arguments (nothing launched), or 2 + the HIP error.
int coat_bench_mix_ceiling(float* w, const uint16_t* g, uint8_t* m_codes, uint8_t* v_codes,
                           float* m_scale, float* m_k, float* v_scale, float* v_k,
                           int64_t n_elems, int64_t n_groups, int32_t group_size,
                           uint32_t mask, hipStream_t stream) {
  if (!w || !g || !m_codes || !v_codes || !m_scale || !m_k || !v_scale || !v_k) return 1;
  if (n_elems < kTileElems || n_groups < 1) return 1;
  if (((uintptr_t)w | (uintptr_t)g | (uintptr_t)m_codes | (uintptr_t)v_codes) % 16) return 1;
  MixParams p;
  p.w = reinterpret_cast<uint32_t*>(w);
  p.g = g;
  p.mc = m_codes;
  p.vc = v_codes;
  p.ms = reinterpret_cast<uint32_t*>(m_scale);
  p.mk = reinterpret_cast<uint32_t*>(m_k);
  p.vs = reinterpret_cast<uint32_t*>(v_scale);
  p.vk = reinterpret_cast<uint32_t*>(v_k);
  p.tiles = n_elems / kTileElems;
  p.ngroups = n_groups;
  p.mask = mask;
  const void* fn;
  switch (group_size) {
    case 16: fn = mix_fn<16>(); break;
    case 32: fn = mix_fn<32>(); break;
    case 64: fn = mix_fn<64>(); break;
    case 128: fn = mix_fn<128>(); break;
    default: return 1;
  }
  const int64_t blocks = (p.tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7FFFFFFF) return 1;
  void* args[] = {&p};
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kBlockThreads), args, 0, stream);
  return e == hipSuccess ? 0 : 2 + (int)e;
}

}  // extern "C"
