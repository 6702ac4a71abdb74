// coat_gemm.hip -- gfx950 FP8 GEMM with a group-scaled FP8 epilogue (COAT's
// linear-layer output quantization) and the same GEMM with a plain BF16
// epilogue, plus their C ABI.
//
// Sources (see include/coat_fp8.h for the full citations):
//   [P1] COAT paper review (xllm-io.github.io), section 三, Triton优化内核 /
//        线性层优化: the GEMM output is viewed as (BLOCK_M, BLOCK_N/G, G) and
//        the max is taken along the last axis; section 四 table, 组缩放技术:
//        a two-stage max reduction fused into the producing operation;
//        核心公式 "FP8量化" for the per-group quantizer.
//   [OCP] OFP8 specification, E4M3.
//
// Execution model (128 x 128 tiles; a 256 x 256 variant further down is used
// when N is a multiple of 256).  C = s * A B^T with A (M x K) and B (N x K)
// E4M3 codes, row-major, s = a_scale * b_scale.  A 256-thread block computes
// a 128 x 128 tile of C; its four waves each own 64 x 64 as 2 x 2 tiles of
// the 32x32x64 FP8 MFMA, accumulating in FP32.  K advances 128 at a time
// through a double buffered LDS copy of the A and B panels, loaded straight
// from global memory into LDS (16-byte chunks XOR-swizzled by row, so the
// MFMA operand reads are free of bank conflicts) while the MFMAs of the
// previous panels run.  In the 32x32 MFMA result a row's 32 columns lie
// across the 32 lanes of a half wave; the epilogue therefore stages the FP32
// accumulator tile through LDS and re-reads it row-contiguously, 8 columns
// per lane, so that the group max is stage one over a lane's 8 values and
// stage two over the group's G/8 lanes (DPP).
//
// Quantization (both kernels).  With c the FP32 accumulator, the group
// maximum of |c s| is fl(max |c| * |s|) exactly (rounding is monotone), the
// stored scale is that maximum / 448, and each code is RNE(c * m) with the
// per-group multiplier m = fl(s * fl(448 / max)): one rounding of c per
// element instead of the two of fl(fl(c s) * 448 / max).  Both agree
// bit for bit when s is a power of two; otherwise they differ by at most one
// FP32 rounding of the value rounded to E4M3.  Groups whose maximum lies
// below 2^-100 or past FP32's range take the two-rounding form.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "coat_common.h"

using namespace coat;

namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kPanelBytes = kBM * kBK;  // one A or B panel in LDS: 16 KB
constexpr int kGroupM = 8;              // tile rows per group of the tile order

// LDS: four distinct 16 KB arrays, the A and B panels of the two pipeline
// stages.  Being distinct objects, the compiler can tell the direct-to-LDS
// loads into one stage from the reads of the other, and does not wait for
// the loads in flight before reading.  The epilogue reuses them as four
// quarters (32 rows x 128 FP32 each) of the C tile.
__shared__ __attribute__((aligned(16))) uint8_t lds_a0[kPanelBytes];
__shared__ __attribute__((aligned(16))) uint8_t lds_b0[kPanelBytes];
__shared__ __attribute__((aligned(16))) uint8_t lds_a1[kPanelBytes];
__shared__ __attribute__((aligned(16))) uint8_t lds_b1[kPanelBytes];

template <int kQ>
__device__ __forceinline__ uint8_t* lds_quarter() {
  if constexpr (kQ == 0) return lds_a0;
  else if constexpr (kQ == 1) return lds_b0;
  else if constexpr (kQ == 2) return lds_a1;
  else return lds_b1;
}

// Float offset of C[row % 32][col] in its quarter: 16-byte chunks XORed by
// bit 2 of the row, so the two half-waves' rows (r and r + 4) fall 32 banks
// apart; 8 consecutive columns (two chunks 2c, 2c + 1) stay adjacent.
__device__ __forceinline__ int quarter_off(int row, int col) {
  return (row & 31) * kBN + (((col >> 2) ^ (((row >> 2) & 1) << 3)) << 2) + (col & 3);
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

enum Epilogue { kGroupQuant = 0, kBF16 = 1 };

struct GemmParams {
  const uint8_t* a;
  const uint8_t* b;
  uint8_t* codes;    // M x N E4M3 (group quant)
  float* scales;     // M x N/G (group quant)
  float* c_f32;      // optional M x N FP32 C (group quant)
  uint16_t* c_bf16;  // M x N BF16 (plain epilogue)
  int64_t M, N, K;
  int64_t n_tiles;   // N / 128 (N / 256 for the 256 x 256 kernel)
  int64_t tile_base; // first tile of this launch in the tile order (256 x 256 kernel)
  float scale;       // a_scale * b_scale, rounded to FP32
};


// Byte offset of 16-byte chunk c of row `row` in a 128-byte-row LDS panel.
// The LDS serves 16 lanes x 16 bytes (all 64 banks) per cycle.  An MFMA
// operand read has 16 lanes on 16 consecutive rows at one logical chunk;
// rows of opposite parity already sit in opposite halves of the banks, so
// the chunk is XORed with (row / 2) % 8 to spread each parity class over the
// 8 chunks of its half.
__device__ __forceinline__ int chunk_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int panel_off(int row, int c) { return row * 128 + 16 * (c ^ chunk_swz(row)); }

__device__ __forceinline__ float scale_acc(float acc, float s) {
#pragma clang fp contract(off)
  return acc * s;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int G, int kEpi>
__global__ __launch_bounds__(kBlockThreads) void gemm_fp8_kernel(const GemmParams p) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  // Tile order: each XCD takes a contiguous run of tile indices, walked in
  // groups of kGroupM tile rows, column by column inside a group, so the A
  // panels of the group stay in the XCD's L2 and each B panel serves kGroupM
  // tiles in a row.
  const int64_t bid = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t m_tiles = (p.M + kBM - 1) / kBM;
  const int64_t group = bid / (kGroupM * p.n_tiles), first_m = group * kGroupM;
  const int64_t gm = m_tiles - first_m < kGroupM ? m_tiles - first_m : kGroupM;
  const int64_t local = bid - group * kGroupM * p.n_tiles;
  const int64_t tm = first_m + local % gm, tn = local / gm;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int64_t K = p.K;

  // Panel loads go straight from global memory into LDS: one wave-wide
  // 16-byte-per-lane load fills 1 KB, 8 rows of a panel, lane L landing at
  // byte 16 L.  So lane L carries row R0 + L/8 and the physical chunk L%8,
  // which under the row swizzle holds logical chunk (L%8) ^ chunk_swz(row);
  // the swizzle is applied on the global side.  Wave w fills rows 32 w .. 32 w + 31 of each
  // panel with 4 loads.  Rows of A past M are not loaded (their LDS bytes are
  // stale and only reach output rows that are never stored).
  const uint8_t* a_blk = p.a + m0 * K;
  const uint8_t* b_blk = p.b + n0 * K;
  uint32_t goff[4];
  bool a_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ chunk_swz(row);
    goff[i] = (uint32_t)row * (uint32_t)K + 16u * (uint32_t)c;
    a_ok[i] = m0 + row < p.M;
  }
  auto issue = [&](int64_t k0, auto S) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value;
    uint8_t* As = lds_quarter<2 * st>();
    uint8_t* Bs = lds_quarter<2 * st + 1>();
    const uint8_t* ak = a_blk + k0;
    const uint8_t* bk = b_blk + k0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint8_t* dst_a = As + 1024 * (4 * wave + i);
      uint8_t* dst_b = Bs + 1024 * (4 * wave + i);
      if (a_ok[i]) __builtin_amdgcn_global_load_lds(ak + goff[i], dst_a, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(bk + goff[i], dst_b, 16, 0, 0);
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)(K / kBK);
  const int half = lane >> 5, l32 = lane & 31;
  // One K step on stage S: start the loads of step kt + 1 into the other
  // stage, run the MFMAs on this one, then wait for this wave's loads and
  // meet the other waves (their loads have landed, nobody reads stage S).
  auto kstep = [&](int kt, auto S) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value;
    if (kt + 1 < nk) issue((int64_t)(kt + 1) * kBK, std::integral_constant<int, 1 - st>{});
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
    const uint8_t* As = lds_quarter<2 * st>();
    const uint8_t* Bs = lds_quarter<2 * st + 1>();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // lane supplies row (l32) and k bytes 64 kk + 32 half .. +31: chunks c0, c0 + 1
      const int c0 = 4 * kk + 2 * half;
      v8i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + 32 * i + l32;
        const uint4 lo = *reinterpret_cast<const uint4*>(As + panel_off(row, c0));
        const uint4 hi = *reinterpret_cast<const uint4*>(As + panel_off(row, c0 + 1));
        fa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wn * 64 + 32 * j + l32;
        const uint4 lo = *reinterpret_cast<const uint4*>(Bs + panel_off(row, c0));
        const uint4 hi = *reinterpret_cast<const uint4*>(Bs + panel_off(row, c0 + 1));
        fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0,
                                                                      0, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next panels have landed
    __syncthreads();
  };
  if (nk > 0) issue(0, std::integral_constant<int, 0>{});
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    kstep(kt, std::integral_constant<int, 0>{});
    kstep(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < nk) kstep(kt, std::integral_constant<int, 0>{});

  // Epilogue.  Value (i, j, r) of this lane is C[row][col] with
  //   row = wm*64 + 32 i + 8 (r/4) + 4 half + r%4,  col = wn*64 + 32 j + l32.
  const float s = p.scale;

  if constexpr (kEpi == kBF16) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = scale_acc(acc[i][j][r], s);
    // BF16 tile: quarter q (rows 32 q .. 32 q + 31) in the first 8 KB of array q.
    auto put = [&](auto Q) __attribute__((always_inline)) {
      constexpr int q = decltype(Q)::value;
      uint16_t* tile = reinterpret_cast<uint16_t*>(lds_quarter<q>());
      if (wm == (q >> 1)) {
        constexpr int i = q & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * half + (r & 3);
            tile[row * kBN + wn * 64 + 32 * j + l32] = bf16_rne(acc[i][j][r]);
          }
      }
    };
    auto get = [&](auto Q) __attribute__((always_inline)) {
      constexpr int q = decltype(Q)::value;
      const uint16_t* tile = reinterpret_cast<const uint16_t*>(lds_quarter<q>());
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int qq = t + kBlockThreads * i, row = qq >> 4, c = qq & 15;
        if (m0 + 32 * q + row < p.M) {
          const uint4 v = *reinterpret_cast<const uint4*>(tile + row * kBN + 8 * c);
          *reinterpret_cast<uint4*>(p.c_bf16 + (m0 + 32 * q + row) * p.N + n0 + 8 * c) = v;
        }
      }
    };
    put(std::integral_constant<int, 0>{});
    put(std::integral_constant<int, 1>{});
    put(std::integral_constant<int, 2>{});
    put(std::integral_constant<int, 3>{});
    __syncthreads();
    get(std::integral_constant<int, 0>{});
    get(std::integral_constant<int, 1>{});
    get(std::integral_constant<int, 2>{});
    get(std::integral_constant<int, 3>{});
  } else {
    // The scaled C tile goes to LDS as FP32 (four 32-row quarters), and
    // the quantizer then walks it like the activation quantizer: a thread
    // takes 8 consecutive columns of a row per pass, so a group of G columns
    // sits on G/8 neighbouring lanes of a 16-lane DPP row.  Stage one of the
    // max is the thread's 8 values, stage two the DPP steps across the group's
    // lanes; the divisions (r and S) are once per 8 values.
    auto put = [&](auto Q) __attribute__((always_inline)) {
      constexpr int q = decltype(Q)::value;
      float* ct = reinterpret_cast<float*>(lds_quarter<q>());
      if (wm == (q >> 1)) {
        constexpr int i = q & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * half + (r & 3);
            ct[quarter_off(row, wn * 64 + 32 * j + l32)] = acc[i][j][r];
          }
      }
    };
    put(std::integral_constant<int, 0>{});
    put(std::integral_constant<int, 1>{});
    put(std::integral_constant<int, 2>{});
    put(std::integral_constant<int, 3>{});
    __syncthreads();
    const int chunk = t & 15, rsub = t >> 4;
    const int64_t gpr = p.N / G;
    const float s_abs = fabsf(s);
    auto quantize = [&](auto Q) __attribute__((always_inline)) {
      constexpr int qq = decltype(Q)::value;
      const float* ct = reinterpret_cast<const float*>(lds_quarter<qq>());
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int lrow = 16 * h2 + rsub;      // row inside the quarter
        const int row = 32 * qq + lrow;       // row inside the tile
        const int col = 8 * chunk;
        const float4 v0 = *reinterpret_cast<const float4*>(ct + quarter_off(lrow, col));
        const float4 v1 = *reinterpret_cast<const float4*>(ct + quarter_off(lrow, col + 4));
        const bool ok = m0 + row < p.M;
        if (p.c_f32 && ok) {
          float* dst = p.c_f32 + (m0 + row) * p.N + n0 + col;
          *reinterpret_cast<float4*>(dst) =
              make_float4(scale_acc(v0.x, s), scale_acc(v0.y, s), scale_acc(v0.z, s), scale_acc(v0.w, s));
          *reinterpret_cast<float4*>(dst + 4) =
              make_float4(scale_acc(v1.x, s), scale_acc(v1.y, s), scale_acc(v1.z, s), scale_acc(v1.w, s));
        }
        // The quarters hold the unscaled accumulators c; the group maximum of
        // |c s| is fl(max |c| * |s|) (rounding is monotone).
        const float mc = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                               fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
        // non-negative floats order like their bit patterns
        const float amax = scale_acc(__uint_as_float(lanes_max_u32<G / 8>(__float_as_uint(mc))), s_abs);
        uint2 c = make_uint2(0u, 0u);
        if (amax >= 0x1p-100f && amax <= 0x1.fffffep127f) {
          // code = RNE(c * m), m = fl(s * fl(448 / max)); fma(c, m, +0) folds -0 to +0
          const float m = scale_acc(448.0f / amax, s);
          int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fmaf(v0.x, m, 0.0f), __builtin_fmaf(v0.y, m, 0.0f), 0, false);
          w0 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fmaf(v0.z, m, 0.0f), __builtin_fmaf(v0.w, m, 0.0f), w0, true);
          int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fmaf(v1.x, m, 0.0f), __builtin_fmaf(v1.y, m, 0.0f), 0, false);
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fmaf(v1.z, m, 0.0f), __builtin_fmaf(v1.w, m, 0.0f), w1, true);
          c = make_uint2((uint32_t)w0, (uint32_t)w1);
        } else if (amax > 0.0f) {
          // maxima below 2^-100 (448 / max would leave FP32's range: scale by
          // 2^64) or past FP32's range: round c s first, as the definition does
          const float pre = amax < 0x1p-100f ? 0x1p64f : 1.0f;
          const float rq = 448.0f / (amax * pre);
          const float4 x0 = make_float4(scale_acc(v0.x, s), scale_acc(v0.y, s), scale_acc(v0.z, s), scale_acc(v0.w, s));
          const float4 x1 = make_float4(scale_acc(v1.x, s), scale_acc(v1.y, s), scale_acc(v1.z, s), scale_acc(v1.w, s));
          int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_nz(x0.x * pre, rq), scaled_nz(x0.y * pre, rq), 0, false);
          w0 = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_nz(x0.z * pre, rq), scaled_nz(x0.w * pre, rq), w0, true);
          int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_nz(x1.x * pre, rq), scaled_nz(x1.y * pre, rq), 0, false);
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_nz(x1.z * pre, rq), scaled_nz(x1.w * pre, rq), w1, true);
          c = make_uint2((uint32_t)w0, (uint32_t)w1);
        }
        if (ok) {
          *reinterpret_cast<uint2*>(p.codes + (m0 + row) * p.N + n0 + col) = c;
          if (chunk % (G / 8) == 0) p.scales[(m0 + row) * gpr + (n0 + col) / G] = amax / 448.0f;
        }
      }
    };
    quantize(std::integral_constant<int, 0>{});
    quantize(std::integral_constant<int, 1>{});
    quantize(std::integral_constant<int, 2>{});
    quantize(std::integral_constant<int, 3>{});
  }
}

// ------------------------------------------------------ 256 x 256 tiles
//
// The same GEMM with 256 x 256 block tiles: 512 threads, eight waves laid
// out 4 (rows) x 2 (columns), each owning 64 rows x 128 columns as 2 x 4
// tiles of the 32x32x64 MFMA.  Per unit of output it moves half the panel
// traffic of the 128 x 128 kernel; the LDS holds 2 stages of 32 KB A and B
// panels (128 KB), so one block runs per CU.  Used when N is a multiple of
// 256.  With kI = 1 a block computes half a tile, 128 x 256 (waves of
// 32 x 128): when the tiles do not fill the last round of CUs, the last
// tiles of the order run as two halves each in a second launch.
//
// The MFMA takes the B panel rows as its first operand, so each 32 x 32
// result is a tile of C^T: register r of lane l holds C[row][col] with
// row = 32 i + l % 32 and col = 32 j + 8 (r / 4) + 4 (l / 32) + r % 4 inside
// the wave's 64 x 128.  A lane therefore holds runs of four consecutive
// columns, and lanes l and l ^ 32 together hold all 128 columns of two rows.
// The group maximum of the quantizing epilogue is a reduction over a lane's
// own registers and one exchange between the half waves; only the finished
// E4M3 codes go through the LDS, for row-contiguous stores.

constexpr int kBM256 = 256;
constexpr int kBN256 = 256;
constexpr int kThreads256 = 512;
constexpr int kPanel256 = kBM256 * kBK;  // 32 KB
constexpr int kGroupM256 = 4;            // tile rows per group of the tile order

__shared__ __attribute__((aligned(16))) uint8_t lds256_a0[kPanel256];
__shared__ __attribute__((aligned(16))) uint8_t lds256_b0[kPanel256];
__shared__ __attribute__((aligned(16))) uint8_t lds256_a1[kPanel256];
__shared__ __attribute__((aligned(16))) uint8_t lds256_b1[kPanel256];

template <int kQ>
__device__ __forceinline__ uint8_t* lds256_part() {
  if constexpr (kQ == 0) return lds256_a0;
  else if constexpr (kQ == 1) return lds256_b0;
  else if constexpr (kQ == 2) return lds256_a1;
  else return lds256_b1;
}

__device__ __forceinline__ uint8_t* lds256_part_rt(int q) {
  return q == 0 ? lds256_a0 : q == 1 ? lds256_b0 : q == 2 ? lds256_a1 : lds256_b1;
}

// Epilogue staging tiles.  Byte `col` of row `row` of a tile of 256-byte
// (codes) or 512-byte (BF16) rows, `rows_per_array` rows to a 32 KB array:
// 16-byte chunks XORed with row % 16, and for the codes the two 8-byte halves
// of a chunk swapped on rows with bit 4 set.  The writes (32 rows x 8 bytes,
// or 32 rows x 16 bytes for BF16, per instruction) and the row reads (16 bytes
// per lane) then meet no bank conflicts.
__device__ __forceinline__ int code_off(int row, int col) {
  return (row & 127) * 256 + ((((col >> 4) ^ (row & 15))) << 4) + ((col & 15) ^ (((row >> 4) & 1) << 3));
}
__device__ __forceinline__ int bf16_off(int row, int col) {
  return (row & 63) * 512 + ((((col >> 4) ^ (row & 15))) << 4) + (col & 15);
}

// Max of x over the lane pair (l, l ^ 32): the exchange returns the pair's
// two values in either order.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int G, int kEpi, int kI>
__global__ __launch_bounds__(kThreads256) void gemm_fp8_kernel_256(const GemmParams p) {
  static_assert(kI == 1 || kI == 2, "row tiles per wave");
  constexpr int kWaveRows = 32 * kI;         // rows of C per wave (128 kI per block)
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave & 3, wn = wave >> 2;   // 4 x 2 waves of kWaveRows x 128
  // Tile order: each XCD takes a contiguous run of tile indices, walked in
  // groups of kGroupM256 tile rows, column by column inside a group, so the A
  // panels of the group stay in the XCD's L2 and each B panel serves kGroupM256
  // tiles in a row.
  // (half tiles: the two halves of a tile are neighbours in the order)
  const int64_t bidx = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t bid = p.tile_base + (kI == 2 ? bidx : bidx >> 1);
  const int64_t m_tiles = (p.M + kBM256 - 1) / kBM256;
  const int64_t group = bid / (kGroupM256 * p.n_tiles), first_m = group * kGroupM256;
  const int64_t gm = m_tiles - first_m < kGroupM256 ? m_tiles - first_m : kGroupM256;
  const int64_t local = bid - group * kGroupM256 * p.n_tiles;
  const int64_t tm = first_m + local % gm, tn = local / gm;
  const int64_t m0 = tm * kBM256 + (kI == 2 ? 0 : 128 * (bidx & 1)), n0 = tn * kBN256;
  if (m0 >= p.M) return;   // second half of a last tile row of at most 128 rows
  const int64_t K = p.K;

  // Panel loads go straight from global memory into LDS: one wave-wide
  // 16-byte-per-lane buffer load fills 1 KB, 8 rows of a panel, lane L
  // landing at byte 16 L.  So lane L carries row R0 + L/8 and the physical
  // chunk L%8, which under the row swizzle holds logical chunk
  // (L%8) ^ chunk_swz(row); the swizzle is applied on the global side.  Wave
  // w fills rows 32 w .. 32 w + 31 of each panel with 4 loads.  The buffer
  // resource holds the panel base, the scalar offset the K position.  A rows
  // past M re-load row M - 1: their products only reach output rows that are
  // never stored.  (Buffer loads count only against vmcnt, so the waits for
  // LDS reads below stay partial while panel loads are in flight.)
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.a + m0 * K), (short)0, (int)0xFFFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.b + n0 * K), (short)0, (int)0xFFFFFFFF, 0x00020000);
  const int64_t a_rows = p.M - m0;
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ chunk_swz(row);
    const int arow = row < a_rows ? row : (int)(a_rows - 1);
    aoff[i] = (uint32_t)arow * (uint32_t)K + 16u * (uint32_t)c;
    boff[i] = (uint32_t)row * (uint32_t)K + 16u * (uint32_t)c;
  }
  // Load q = 0..7 of a K step: A (even q) or B (odd q), rows 32 wave + 8 (q / 2) + lane / 8
  // (a half tile's A panel has 128 rows: waves 0-3 load it).
  const bool a_loader = kI == 2 || wave < 4;
  auto load1 = [&](int64_t k0, auto S, int q) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value;
    uint8_t* As = lds256_part<2 * st>();
    uint8_t* Bs = lds256_part<2 * st + 1>();
    const int i = q >> 1;
    if (q & 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, Bs + 1024 * (4 * wave + i), 16, (int)boff[i], (int)k0, 0, 0);
    else if (a_loader)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, As + 1024 * (4 * wave + i), 16, (int)aoff[i], (int)k0, 0, 0);
  };

  v16f acc[kI][4];
#pragma unroll
  for (int i = 0; i < kI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)(K / kBK);
  const int half = lane >> 5, l32 = lane & 31;
  // Operand fragment: lane supplies row l32 of a 32-row tile and the k bytes
  // 64 kk + 32 half .. +31 (logical chunks c0, c0 + 1 of the panel row).
  auto frag = [&](const uint8_t* panel, int row, int kk) __attribute__((always_inline)) {
    const int c0 = 4 * kk + 2 * half;
    const uint4 lo = *reinterpret_cast<const uint4*>(panel + panel_off(row, c0));
    const uint4 hi = *reinterpret_cast<const uint4*>(panel + panel_off(row, c0 + 1));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  // A K step is four MFMA groups g = (kk, h): both row tiles against column
  // tiles 2h, 2h + 1 at k half kk.  The fragments of group g + 1 are read
  // while the MFMAs of group g run (two register sets fb0 / fb1 for B, one A
  // set per kk), so the waits on LDS reads are partial.
  v8i fa0[kI], fa1[kI], fb0[2], fb1[2];
  auto read_a = [&](v8i* f, const uint8_t* As, int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kI; ++i) f[i] = frag(As, wm * kWaveRows + 32 * i + l32, kk);
  };
  auto read_b = [&](v8i* f, const uint8_t* Bs, int kk, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) f[jj] = frag(Bs, wn * 128 + 32 * (2 * h + jj) + l32, kk);
  };
  // MFMA q (0 .. 2 kI - 1) of a group: row tile q / 2, column tile 2 h + q % 2
  auto mma1 = [&](const v8i* fa, const v8i* fb, int h, int q) __attribute__((always_inline)) {
    if (q < 2 * kI) {
      const int i = q >> 1, jj = q & 1;
      acc[i][2 * h + jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[jj], fa[i], acc[i][2 * h + jj],
                                                                          0, 0, 0, 0, 0, 0);
    }
  };
  // The eight panel loads of a K step are spread one per MFMA over three
  // phases: loads 0-2 of step kt + 2 go out in the last phase of step kt,
  // right after the barrier that frees stage S; loads 3-7 in the first two
  // phases of step kt + 1; all are waited for at the barrier of step kt + 1.
  // Past the last step the loads re-fetch the last K slice into a stage that
  // is not read again.
  const int64_t k_last = K - kBK;
  auto kslice = [&](int k) __attribute__((always_inline)) {
    return k < nk ? (int64_t)k * kBK : k_last;
  };
  auto kstep = [&](int kt, auto S) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value;
    using N = std::integral_constant<int, 1 - st>;
    const uint8_t* As = lds256_part<2 * st>();
    const uint8_t* Bs = lds256_part<2 * st + 1>();
    const int64_t k1 = kslice(kt + 1), k2 = kslice(kt + 2);
    // on entry fa0 / fb0 hold group (0, 0) of stage S
    read_b(fb1, Bs, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      mma1(fa0, fb0, 0, q);
      if (q < 3) load1(k1, N{}, 3 + q);
      __builtin_amdgcn_sched_barrier(0);
    }
    read_b(fb0, Bs, 1, 0);
    read_a(fa1, As, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      mma1(fa0, fb1, 1, q);
      if (q < 2) load1(k1, N{}, 6 + q);
      __builtin_amdgcn_sched_barrier(0);
    }
    read_b(fb1, Bs, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) mma1(fa1, fb0, 0, q);
    __builtin_amdgcn_sched_barrier(0);
    // every wave has read all of stage S and waits for its loads of stage
    // 1 - S; after the barrier stage 1 - S is complete and stage S is free
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // first fragments of the next step (after the last step: read, unused)
    read_b(fb0, lds256_part<2 * (1 - st) + 1>(), 0, 0);
    read_a(fa0, lds256_part<2 * (1 - st)>(), 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      mma1(fa1, fb1, 1, q);
      if (q < 3) load1(k2, S, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (nk > 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) load1(0, std::integral_constant<int, 0>{}, q);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 3; ++q) load1(kslice(1), std::integral_constant<int, 1>{}, q);
    read_b(fb0, lds256_part<1>(), 0, 0);
    read_a(fa0, lds256_part<0>(), 0);
  }
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    kstep(kt, std::integral_constant<int, 0>{});
    kstep(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < nk) kstep(kt, std::integral_constant<int, 0>{});
  __builtin_amdgcn_s_waitcnt(0);  // loads past the last step; the epilogue reuses the arrays
  __syncthreads();

  // Epilogue.  Register 4 q + s of acc[i][j] is C[row][col] with
  //   row = wm * kWaveRows + 32 i + l32,  col = wn * 128 + 32 j + 8 q + 4 half + s.
  const float s = p.scale;
  if constexpr (kEpi == kBF16) {
    // BF16 tile, 64 rows x 512 bytes per array: a lane writes its runs of
    // four columns (8 bytes), then every lane stores 16-byte row chunks.
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wm * kWaveRows + 32 * i + l32;
          uint8_t* wtile = lds256_part_rt((wm * kWaveRows + 32 * i) >> 6);
          const int col = 2 * (wn * 128 + 32 * j + 8 * q + 4 * half);
          const uint32_t lo = bf16_rne(scale_acc(acc[i][j][4 * q], s)) |
                              ((uint32_t)bf16_rne(scale_acc(acc[i][j][4 * q + 1], s)) << 16);
          const uint32_t hi = bf16_rne(scale_acc(acc[i][j][4 * q + 2], s)) |
                              ((uint32_t)bf16_rne(scale_acc(acc[i][j][4 * q + 3], s)) << 16);
          *reinterpret_cast<uint2*>(wtile + bf16_off(row, col)) = make_uint2(lo, hi);
        }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8 * kI; ++k) {
      const int task = k * kThreads256 + t, row = task >> 5, c = task & 31;
      const uint8_t* rtile = lds256_part_rt(row >> 6);
      const uint4 v = *reinterpret_cast<const uint4*>(rtile + bf16_off(row, 16 * c));
      if (m0 + row < p.M)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(p.c_bf16 + (m0 + row) * p.N + n0) + 16 * c) = v;
    }
  } else {
    constexpr int kGW = 128 / G;   // groups per row in the wave's 128 columns
    const int64_t gpr = p.N / G;
    const float s_abs = fabsf(s);
    // optional FP32 copy of C
    if (p.c_f32) {
#pragma unroll
      for (int i = 0; i < kI; ++i) {
        const int64_t row = m0 + wm * kWaveRows + 32 * i + l32;
        if (row < p.M) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(p.c_f32 + row * p.N + n0 + wn * 128 + 32 * j + 8 * q + 4 * half) =
                  make_float4(scale_acc(acc[i][j][4 * q], s), scale_acc(acc[i][j][4 * q + 1], s),
                              scale_acc(acc[i][j][4 * q + 2], s), scale_acc(acc[i][j][4 * q + 3], s));
        }
      }
    }
    // Group maxima of |c| (c the unscaled accumulator): stage one over the
    // lane's registers of the group, stage two over the lane pair.  The group
    // maximum of |c s| is then fl(max |c| * |s|): rounding is monotone.
    float amax[kI][kGW];
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int g = 0; g < kGW; ++g) amax[i][g] = 0.0f;
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int g = (32 * j + 8 * q) / G;
          amax[i][g] = fmaxf(fmaxf(amax[i][g], fmaxf(fabsf(acc[i][j][4 * q]), fabsf(acc[i][j][4 * q + 1]))),
                             fmaxf(fabsf(acc[i][j][4 * q + 2]), fabsf(acc[i][j][4 * q + 3])));
        }
    // Per group: the stored scale max / 448 and the multiplier m with
    // code = RNE(c * m), m = fl(s * fl(448 / max)).  Groups whose max lies
    // outside [2^-100, FLT_MAX] (and zero groups) get m = 0 here and are
    // handled below.
    float mul[kI][kGW];
    bool slow = false;
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int g = 0; g < kGW; ++g) {
        amax[i][g] = scale_acc(pair_max(amax[i][g]), s_abs);
        const bool fast = amax[i][g] >= 0x1p-100f && amax[i][g] <= 0x1.fffffep127f;
        mul[i][g] = fast ? scale_acc(448.0f / amax[i][g], s) : 0.0f;
        slow |= !fast && amax[i][g] > 0.0f;
      }
    uint32_t word[kI][4][4];
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float m = mul[i][(32 * j + 8 * q) / G];
          // fma(c, m, +0) folds an exact -0 product to +0
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fmaf(acc[i][j][4 * q], m, 0.0f),
                                                  __builtin_fmaf(acc[i][j][4 * q + 1], m, 0.0f), 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fmaf(acc[i][j][4 * q + 2], m, 0.0f),
                                              __builtin_fmaf(acc[i][j][4 * q + 3], m, 0.0f), w, true);
          word[i][j][q] = (uint32_t)w;
        }
    if (slow) {
      // Maxima below 2^-100 (448 / max would leave FP32's range: scale by
      // 2^64) or past FP32's range: round c s first, as the definition does.
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float am = amax[i][(32 * j + 8 * q) / G];
            if (!(am >= 0x1p-100f && am <= 0x1.fffffep127f) && am > 0.0f) {
              const float pre = am < 0x1p-100f ? 0x1p64f : 1.0f;
              const float rq = 448.0f / (am * pre);
              const float x0 = scale_acc(acc[i][j][4 * q], s), x1 = scale_acc(acc[i][j][4 * q + 1], s);
              const float x2 = scale_acc(acc[i][j][4 * q + 2], s), x3 = scale_acc(acc[i][j][4 * q + 3], s);
              int w = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_nz(x0 * pre, rq), scaled_nz(x1 * pre, rq), 0, false);
              w = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_nz(x2 * pre, rq), scaled_nz(x3 * pre, rq), w, true);
              word[i][j][q] = (uint32_t)w;
            }
          }
    }
    // scales: the pair shares each maximum; half h stores groups g % 2 == h
#pragma unroll
    for (int i = 0; i < kI; ++i) {
      const int64_t row = m0 + wm * kWaveRows + 32 * i + l32;
      if (row < p.M) {
#pragma unroll
        for (int g = 0; g < kGW; ++g)
          if (kGW == 1 ? half == 0 : (g & 1) == half)
            p.scales[row * gpr + (n0 + wn * 128) / G + g] = amax[i][g] / 448.0f;
      }
    }
    // codes through the LDS (128 kI rows x 256 bytes, 128 rows per array),
    // then 16-byte row chunks to global memory
    uint8_t* wtile = wm * kWaveRows < 128 ? lds256_a0 : lds256_b0;
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wm * kWaveRows + 32 * i + l32;
          const int col = wn * 128 + 32 * j + 8 * q + 4 * half;
          *reinterpret_cast<uint32_t*>(wtile + code_off(row, col)) = word[i][j][q];
        }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4 * kI; ++k) {
      const int task = k * kThreads256 + t, row = task >> 4, c = task & 15;
      const uint8_t* rtile = row < 128 ? lds256_a0 : lds256_b0;
      // chunk base (the 8-byte halves are swapped on rows with bit 4 set)
      uint4 v = *reinterpret_cast<const uint4*>(rtile + (row & 127) * 256 + ((c ^ (row & 15)) << 4));
      if ((row >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
      if (m0 + row < p.M) *reinterpret_cast<uint4*>(p.codes + (m0 + row) * p.N + n0 + 16 * c) = v;
    }
  }
}

// Kernel for a tile shape: 0 = 128 x 128, 1 = 256 x 256, 2 = 128 x 256 half tiles.
template <int G, int kEpi>
const void* kernel_fn(int shape) {
  if (shape == 1) return reinterpret_cast<const void*>(&gemm_fp8_kernel_256<G, kEpi, 2>);
  if (shape == 2) return reinterpret_cast<const void*>(&gemm_fp8_kernel_256<G, kEpi, 1>);
  return reinterpret_cast<const void*>(&gemm_fp8_kernel<G, kEpi>);
}

const void* gemm_kernel_for(int32_t g, int epi, int shape) {
  if (epi == kBF16) return kernel_fn<128, kBF16>(shape);
  switch (g) {
    case 16: return kernel_fn<16, kGroupQuant>(shape);
    case 32: return kernel_fn<32, kGroupQuant>(shape);
    case 64: return kernel_fn<64, kGroupQuant>(shape);
    default: return kernel_fn<128, kGroupQuant>(shape);
  }
}

coat_status_t check_gemm_shape(const uint8_t* a, const uint8_t* b, float a_scale, float b_scale,
                               int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0 || N % kBN != 0 || K % kBK != 0 || K > (1 << 24))
    return COAT_ERR_INVALID_VALUE;
  if (!isfinite(a_scale) || !isfinite(b_scale)) return COAT_ERR_INVALID_VALUE;
  if (M == 0 || N == 0) return COAT_OK;
  if (K > 0 && (!a || !b)) return COAT_ERR_NULL_POINTER;
  if (!aligned(a, 16) || !aligned(b, 16)) return COAT_ERR_MISALIGNED;
  const int64_t m_tiles = (M + kBM - 1) / kBM;
  if (m_tiles > 0x7FFFFFFF / (N / kBN)) return COAT_ERR_INVALID_VALUE;
  return COAT_OK;
}

// 256 x 256 tiles when N allows them (N % 256 == 0), else 128 x 128.  One
// 256 x 256 block runs per CU.  When the tiles leave the last round of CUs
// at most half full, the whole rounds run as 256 x 256 tiles and the
// remaining tiles of the order as two 128 x 256 halves each, in a second
// launch on the same stream: half a round instead of a full one.
hipError_t launch_gemm(GemmParams& p, int32_t group_size, int epi, hipStream_t stream) {
  void* args[] = {&p};
  if (p.N % kBN256 != 0) {
    p.n_tiles = p.N / kBN;
    const int64_t blocks = (p.M + kBM - 1) / kBM * p.n_tiles;
    return hipLaunchKernel(gemm_kernel_for(group_size, epi, 0), dim3((unsigned)blocks),
                           dim3(kBlockThreads), args, 0, stream);
  }
  p.n_tiles = p.N / kBN256;
  const int64_t tiles = (p.M + kBM256 - 1) / kBM256 * p.n_tiles;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t rem = cus > 0 ? tiles % cus : 0;
  const int64_t whole = rem > 0 && 2 * rem <= cus ? tiles - rem : tiles;
  p.tile_base = 0;
  if (whole > 0) {
    e = hipLaunchKernel(gemm_kernel_for(group_size, epi, 1), dim3((unsigned)whole), dim3(kThreads256),
                        args, 0, stream);
    if (e != hipSuccess || whole == tiles) return e;
  }
  p.tile_base = whole;
  return hipLaunchKernel(gemm_kernel_for(group_size, epi, 2), dim3((unsigned)(2 * (tiles - whole))),
                         dim3(kThreads256), args, 0, stream);
}

}  // namespace

extern "C" {

coat_status_t coat_fp8_gemm_group_quant(const uint8_t* a, const uint8_t* b, float a_scale,
                                        float b_scale, int64_t M, int64_t N, int64_t K,
                                        int32_t group_size, uint8_t* codes, float* scales,
                                        float* c_f32, hipStream_t stream) {
  if (!valid_group_size(group_size)) return COAT_ERR_GROUP_SIZE;
  coat_status_t st = check_gemm_shape(a, b, a_scale, b_scale, M, N, K);
  if (st != COAT_OK || M == 0 || N == 0) return st;
  if (!codes || !scales) return COAT_ERR_NULL_POINTER;
  if (!aligned(codes, 16) || !aligned(scales, 4) || (c_f32 && !aligned(c_f32, 16)))
    return COAT_ERR_MISALIGNED;
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = a;
  p.b = b;
  p.codes = codes;
  p.scales = scales;
  p.c_f32 = c_f32;
  p.M = M;
  p.N = N;
  p.K = K;
  p.scale = (float)((double)a_scale * (double)b_scale);
  const hipError_t e = launch_gemm(p, group_size, kGroupQuant, stream);
  return e == hipSuccess ? COAT_OK : hip_fail(e);
}

coat_status_t coat_fp8_gemm_bf16(const uint8_t* a, const uint8_t* b, float a_scale,
                                 float b_scale, int64_t M, int64_t N, int64_t K,
                                 uint16_t* c_bf16, hipStream_t stream) {
  coat_status_t st = check_gemm_shape(a, b, a_scale, b_scale, M, N, K);
  if (st != COAT_OK || M == 0 || N == 0) return st;
  if (!c_bf16) return COAT_ERR_NULL_POINTER;
  if (!aligned(c_bf16, 16)) return COAT_ERR_MISALIGNED;
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = a;
  p.b = b;
  p.c_bf16 = c_bf16;
  p.M = M;
  p.N = N;
  p.K = K;
  p.scale = (float)((double)a_scale * (double)b_scale);
  const hipError_t e = launch_gemm(p, 128, kBF16, stream);
  return e == hipSuccess ? COAT_OK : hip_fail(e);
}

}  // extern "C"
