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
// Execution model.  C = s * A B^T with A (M x K) and B (N x K) E4M3 codes,
// row-major, s = a_scale * b_scale.  A 512-thread block computes a 256 x 256
// tile of C (the last tile column may be 128 wide: N is a multiple of 128);
// its eight waves, laid out 4 (rows) x 2 (columns), each own 64 x 128 as
// 2 x 4 tiles of the 32x32x64 FP8 MFMA, accumulating in FP32.  K advances
// 128 at a time through a double buffered LDS copy of the A and B panels
// (2 stages x 64 KB, one block per CU), loaded straight from global memory
// into LDS by buffer loads (16-byte chunks XOR-swizzled by row, so the MFMA
// operand reads are free of bank conflicts) while the MFMAs of the previous
// panels run.  The epilogue finds each group's maximum and quantizes in
// registers; only the E4M3 codes go through LDS, for row-contiguous stores.
//
// Quantization.  With c the FP32 accumulator and C = fl(c s), the group
// maximum of |C| is fl(max |c| * |s|) exactly (rounding is monotone) and the
// stored scale is that maximum / 448.  Each code is the E4M3 rounding of the
// quotient 448 C / max formed by group_quot (coat_common.h) from the hardware
// reciprocal of max / 512 (within one ulp): the FMA refinement lands exactly
// on a midpoint whenever the quotient is one, so ties are decided exactly,
// and elsewhere the refined quotient lies within about 2^-22 of the exact
// one.  Groups whose maximum lies below 2^-100 take group_quot's 2^64
// pre-scale in a second, rarely taken pass.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "coat_common.h"

using namespace coat;

namespace {

constexpr int kBM = 256;           // rows of C per block (128 for the half-tile variant)
constexpr int kBN = 256;           // columns of C per block
constexpr int kBK = 128;           // K per pipeline step
constexpr int kNQuantum = 128;     // N and K must be multiples of this
constexpr int kThreads = 512;
constexpr int kPanel = kBM * kBK;  // one A or B panel stage in LDS: 32 KB
constexpr int kGroupM = 4;         // tile rows per group of the tile order

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
  int64_t n_tiles;   // tile columns, ceil(N / 256)
  int64_t whole;     // tiles of the order computed whole; each later tile runs as two halves
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

// The output rows leave as 16-byte stores with the nontemporal hint: the
// kernel never reads them back (measured: 0.4-1.9% faster calls across four
// Llama-2-7B shapes, outputs unchanged).
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_out16(void* p, uint4 v) {
  const u32x4v w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4v*>(p));
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ------------------------------------------------------ the kernel
//
// One block computes one tile (kI = 2) or, with kI = 1, half a tile,
// 128 x 256 (waves of 32 x 128): when the tiles do not fill the last round
// of CUs, the last tiles of the order run as two halves each, as the last
// blocks of the same launch.
//
// The MFMA takes the B panel rows as its first operand, so each 32 x 32
// result is a tile of C^T: register r of lane l holds C[row][col] with
// row = 32 i + l % 32 and col = 32 j + 8 (r / 4) + 4 (l / 32) + r % 4 inside
// the wave's 64 x 128.  A lane therefore holds runs of four consecutive
// columns, and lanes l and l ^ 32 together hold all 128 columns of two rows.
// The group maximum of the quantizing epilogue is a reduction over a lane's
// own registers and one exchange between the half waves; only the finished
// E4M3 codes go through the LDS, for row-contiguous stores.

// LDS: four distinct 32 KB arrays, the A and B panels of the two pipeline
// stages.  Being distinct objects, the compiler can tell the loads into one
// stage from the reads of the other, and does not wait for the loads in
// flight before reading.  The epilogue reuses them as its staging tiles.
__shared__ __attribute__((aligned(16))) uint8_t lds_a0[kPanel];
__shared__ __attribute__((aligned(16))) uint8_t lds_b0[kPanel];
__shared__ __attribute__((aligned(16))) uint8_t lds_a1[kPanel];
__shared__ __attribute__((aligned(16))) uint8_t lds_b1[kPanel];

template <int kQ>
__device__ __forceinline__ uint8_t* lds_part() {
  if constexpr (kQ == 0) return lds_a0;
  else if constexpr (kQ == 1) return lds_b0;
  else if constexpr (kQ == 2) return lds_a1;
  else return lds_b1;
}

__device__ __forceinline__ uint8_t* lds_part_rt(int q) {
  return q == 0 ? lds_a0 : q == 1 ? lds_b0 : q == 2 ? lds_a1 : lds_b1;
}

// Epilogue staging tiles.  Byte `col` of row `row` of a tile of 256-byte
// (codes, 128 rows to a 32 KB array) or 512-byte (BF16, 64 rows to an array) rows:
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
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const int64_t bidx) {
  static_assert(kI == 1 || kI == 2, "row tiles per wave");
  constexpr int kWaveRows = 32 * kI;         // rows of C per wave (128 kI per block)
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave & 3, wn = wave >> 2;   // 4 x 2 waves of kWaveRows x 128
  // Tile order: each XCD takes a contiguous run of tile indices, walked in
  // groups of kGroupM tile rows, column by column inside a group, so the A
  // panels of the group stay in the XCD's L2 and each B panel serves kGroupM
  // tiles in a row.
  // (bidx is the block's place in the order of its part, whole or half
  // tiles; the two halves of a tile are neighbours)
  const int64_t bid = kI == 2 ? bidx : p.whole + (bidx >> 1);
  const int64_t m_tiles = (p.M + kBM - 1) / kBM;
  const int64_t group = bid / (kGroupM * p.n_tiles), first_m = group * kGroupM;
  const int64_t gm = m_tiles - first_m < kGroupM ? m_tiles - first_m : kGroupM;
  const int64_t local = bid - group * kGroupM * p.n_tiles;
  const int64_t tm = first_m + local % gm, tn = local / gm;
  const int64_t m0 = tm * kBM + (kI == 2 ? 0 : 128 * (bidx & 1)), n0 = tn * kBN;
  if (m0 >= p.M) return;   // second half of a last tile row of at most 128 rows
  // N is a multiple of 128: the last tile column may be 128 wide, and then
  // the waves with wn = 1 compute columns that are not stored
  const int64_t n_valid = p.N - n0;   // 128 or >= 256
  const bool cols_ok = wn == 0 || n_valid > 128;
  const int64_t K = p.K;

  // Panel loads go straight from global memory into LDS: one wave-wide
  // 16-byte-per-lane buffer load fills 1 KB, 8 rows of a panel, lane L
  // landing at byte 16 L.  So lane L carries row R0 + L/8 and the physical
  // chunk L%8, which under the row swizzle holds logical chunk
  // (L%8) ^ chunk_swz(row); the swizzle is applied on the global side.  The
  // buffer resource holds the panel base, the scalar offset the K position.
  // A rows past M re-load row M - 1 and B rows past N row N - 1: their
  // products only reach output rows and columns that are never stored.
  // (Buffer loads count only against vmcnt, so the waits for LDS reads below
  // stay partial while panel loads are in flight.)
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.a + m0 * K), (short)0, (int)0xFFFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.b + n0 * K), (short)0, (int)0xFFFFFFFF, 0x00020000);
  const int64_t a_rows = p.M - m0, b_rows = n_valid;
  // Wave w fills rows 8 kLA w .. 8 kLA (w + 1) - 1 of the A panel with kLA
  // loads (kBlockRows / 64: 4 for a whole tile, 2 for a half) and rows
  // 32 w .. 32 w + 31 of the B panel with kLB = 4.
  constexpr int kBlockRows = 4 * kWaveRows;   // 256 (whole tile) or 128 (half)
  constexpr int kLA = kBlockRows / 64, kLB = 4, kL = kLA + kLB;
  // s_waitcnt immediate for vmcnt(kL), not waiting on expcnt or lgkmcnt
  // (vmcnt in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8)
  static_assert(kL < 64, "vmcnt holds at most 63");
  constexpr int kVmcntStage1 = (kL & 15) | ((kL >> 4) << 14) | (7 << 4) | (15 << 8);
  uint32_t aoff[kLA], boff[kLB];
#pragma unroll
  for (int i = 0; i < kLA; ++i) {
    const int row = 8 * (kLA * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ chunk_swz(row);
    const int arow = row < a_rows ? row : (int)(a_rows - 1);
    aoff[i] = (uint32_t)arow * (uint32_t)K + 16u * (uint32_t)c;
  }
#pragma unroll
  for (int i = 0; i < kLB; ++i) {
    const int row = 8 * (kLB * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ chunk_swz(row);
    const int brow = row < b_rows ? row : (int)(b_rows - 1);
    boff[i] = (uint32_t)brow * (uint32_t)K + 16u * (uint32_t)c;
  }
  // Load q = 0 .. kL - 1 of a K step into stage S: A loads first, then B.
  auto load1 = [&](int64_t k0, auto S, int q) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value;
    uint8_t* As = lds_part<2 * st>();
    uint8_t* Bs = lds_part<2 * st + 1>();
    if (q < kLA)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, As + 1024 * (kLA * wave + q), 16, (int)aoff[q], (int)k0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, Bs + 1024 * (kLB * wave + q - kLA), 16, (int)boff[q - kLA],
                                               (int)k0, 0, 0);
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
  auto frag_lo = [&](const uint8_t* panel, int row, int kk) __attribute__((always_inline)) {
    return *reinterpret_cast<const uint4*>(panel + panel_off(row, 4 * kk + 2 * half));
  };
  auto frag_hi = [&](const uint8_t* panel, int row, int kk) __attribute__((always_inline)) {
    return *reinterpret_cast<const uint4*>(panel + panel_off(row, 4 * kk + 2 * half + 1));
  };
  // Fragments of the two k halves of a step: set f = kk.  Read r of a set
  // (0 .. 2 (4 + kI) - 1): B tiles 0-3 first, then A tiles, low 16 bytes then high.
  uint4 fa[2][kI][2], fb[2][4][2];
  auto read1 = [&](int f, const uint8_t* As, const uint8_t* Bs, int kk, int r) __attribute__((always_inline)) {
    if (r < 8) {
      const int j = r >> 1, row = wn * 128 + 32 * j + l32;
      fb[f][j][r & 1] = (r & 1) ? frag_hi(Bs, row, kk) : frag_lo(Bs, row, kk);
    } else {
      const int i = (r - 8) >> 1, row = wm * kWaveRows + 32 * i + l32;
      fa[f][i][r & 1] = (r & 1) ? frag_hi(As, row, kk) : frag_lo(As, row, kk);
    }
  };
  auto as_v8 = [](const uint4* v) __attribute__((always_inline)) {
    return v8i{(int)v[0].x, (int)v[0].y, (int)v[0].z, (int)v[0].w,
               (int)v[1].x, (int)v[1].y, (int)v[1].z, (int)v[1].w};
  };
  // MFMA n of set f: row tile n / 4, column tile n % 4
  auto mma1 = [&](int f, int n) __attribute__((always_inline)) {
    const int i = n >> 2, j = n & 3;
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_v8(fb[f][j]), as_v8(fa[f][i]), acc[i][j],
                                                                0, 0, 0, 0, 0, 0);
  };
  // A K step is two phases of 4 kI MFMAs, one per k half.  Phase 0 runs on
  // set 0 while set 1 (k half 1 of the same stage) is read.  Then every wave
  // waits for its reads and for its loads into the other stage, and the block
  // meets at the one barrier of the step: the stage being computed on has been
  // read in full, and the other stage is complete.  Phase 1 runs on set 1
  // while set 0 of the next step is read from the other stage and the loads of
  // the step after next go into this one, so each load has a whole phase and
  // more before the barrier that waits for it.  Past the last step the loads
  // re-fetch the last K slice into a stage that is not read again.
  constexpr int kMF = 4 * kI, kR = 2 * (4 + kI);
  const int64_t k_last = K - kBK;
  auto kslice = [&](int k) __attribute__((always_inline)) {
    return k < nk ? (int64_t)k * kBK : k_last;
  };
  auto kstep = [&](int kt, auto S) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value;
    const uint8_t* As = lds_part<2 * st>();
    const uint8_t* Bs = lds_part<2 * st + 1>();
    const uint8_t* An = lds_part<2 * (1 - st)>();
    const uint8_t* Bn = lds_part<2 * (1 - st) + 1>();
    const int64_t k2 = kslice(kt + 2);
#pragma unroll
    for (int n = 0; n < kMF; ++n) {
      mma1(0, n);
#pragma unroll
      for (int r = n * kR / kMF; r < (n + 1) * kR / kMF; ++r) read1(1, As, Bs, 1, r);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kMF; ++n) {
      mma1(1, n);
#pragma unroll
      for (int r = n * kR / kMF; r < (n + 1) * kR / kMF; ++r) read1(0, An, Bn, 0, r);
#pragma unroll
      for (int q = n * kL / kMF; q < (n + 1) * kL / kMF; ++q) load1(k2, S, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (nk > 0) {
    // both stages' loads go out at once; the first barrier waits only for
    // stage 0 (loads complete in issue order: vmcnt(kL) leaves the kL loads
    // of stage 1 in flight)
#pragma unroll
    for (int q = 0; q < kL; ++q) load1(0, std::integral_constant<int, 0>{}, q);
#pragma unroll
    for (int q = 0; q < kL; ++q) load1(kslice(1), std::integral_constant<int, 1>{}, q);
    // (no release fence here: it would wait for every load, and each wave
    // has already waited for its own loads of stage 0)
    __builtin_amdgcn_s_waitcnt(kVmcntStage1);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
    for (int r = 0; r < kR; ++r) read1(0, lds_part<0>(), lds_part<1>(), 0, r);
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
          uint8_t* wtile = lds_part_rt((wm * kWaveRows + 32 * i) >> 6);
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
      const int task = k * kThreads + t, row = task >> 5, c = task & 31;
      const uint8_t* rtile = lds_part_rt(row >> 6);
      const uint4 v = *reinterpret_cast<const uint4*>(rtile + bf16_off(row, 16 * c));
      if (m0 + row < p.M && 8 * c < n_valid)
        store_out16(reinterpret_cast<uint8_t*>(p.c_bf16 + (m0 + row) * p.N + n0) + 16 * c, v);
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
        if (row < p.M && cols_ok) {
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
          // two three-input maxima per four values (v_max3 with |.| modifiers)
          amax[i][g] = fmaxf(fmaxf(amax[i][g], fabsf(acc[i][j][4 * q])), fabsf(acc[i][j][4 * q + 1]));
          amax[i][g] = fmaxf(fmaxf(amax[i][g], fabsf(acc[i][j][4 * q + 2])), fabsf(acc[i][j][4 * q + 3]));
        }
    // Per group: the stored scale max / 448 and the divisor b = max / 512 with
    // its reciprocal r (v_rcp_f32; the refinement in group_quot keeps ties
    // exact), for group_quot on C = fl(c s) (a = C * 7/8, q = a / b).  With
    // G = 16 a lane forms 16 of these per tile: the hardware reciprocal cut
    // the call by 1-2% there against a rounded division.
    // Groups whose max lies below 2^-100 (or past FP32's range) need the
    // 2^64 pre-scale; they get b = r = 0 here (all codes 0) and are redone
    // below.
    float qb[kI][kGW], qr[kI][kGW];
    bool slow = false;
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int g = 0; g < kGW; ++g) {
        amax[i][g] = scale_acc(pair_max(amax[i][g]), s_abs);
        const bool fast = amax[i][g] >= 0x1p-100f && amax[i][g] <= 0x1.fffffep127f;
        qb[i][g] = fast ? amax[i][g] * 0x1p-9f : 0.0f;
        qr[i][g] = fast ? __builtin_amdgcn_rcpf(qb[i][g]) : 0.0f;
        slow |= !fast && amax[i][g] > 0.0f;
      }
    uint32_t word[kI][4][4];
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int g = (32 * j + 8 * q) / G;
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[e] = group_quot(scale_acc(acc[i][j][4 * q + e], s), 0.875f, qb[i][g], qr[i][g]);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
          word[i][j][q] = (uint32_t)w;
        }
    if (slow) {
#pragma unroll
      for (int i = 0; i < kI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float am = amax[i][(32 * j + 8 * q) / G];
            if (!(am >= 0x1p-100f && am <= 0x1.fffffep127f) && am > 0.0f) {
              const GroupQuot d = group_quot_setup(am);
              float x[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) x[e] = group_quot(scale_acc(acc[i][j][4 * q + e], s), d);
              int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
              w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
              word[i][j][q] = (uint32_t)w;
            }
          }
    }
    // scales: the pair shares each maximum; half h stores groups g % 2 == h
#pragma unroll
    for (int i = 0; i < kI; ++i) {
      const int64_t row = m0 + wm * kWaveRows + 32 * i + l32;
      if (row < p.M && cols_ok) {
#pragma unroll
        for (int g = 0; g < kGW; ++g)
          if (kGW == 1 ? half == 0 : (g & 1) == half)
            p.scales[row * gpr + (n0 + wn * 128) / G + g] = amax[i][g] / 448.0f;
      }
    }
    // codes through the LDS (128 kI rows x 256 bytes, 128 rows per array),
    // then 16-byte row chunks to global memory
    uint8_t* wtile = wm * kWaveRows < 128 ? lds_a0 : lds_b0;
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
      const int task = k * kThreads + t, row = task >> 4, c = task & 15;
      const uint8_t* rtile = row < 128 ? lds_a0 : lds_b0;
      // chunk base (the 8-byte halves are swapped on rows with bit 4 set)
      uint4 v = *reinterpret_cast<const uint4*>(rtile + (row & 127) * 256 + ((c ^ (row & 15)) << 4));
      if ((row >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
      if (m0 + row < p.M && 16 * c < n_valid)
        store_out16(p.codes + (m0 + row) * p.N + n0 + 16 * c, v);
    }
  }
}

// One launch: blocks 0 .. whole - 1 compute whole tiles, the blocks after
// them half tiles.  Blocks are dispatched in index order, so the half tiles
// go to the CUs that finish their whole tiles first, with no launch boundary
// in between.  Workgroups are dealt to the XCDs round-robin; whole is a
// multiple of the CU count (so of 8), and each part is mapped XCD-contiguous
// on its own.
template <int G, int kEpi>
__global__ __launch_bounds__(kThreads) void gemm_fp8_kernel(const GemmParams p) {
  const int64_t b = blockIdx.x;
  if (b < p.whole)
    gemm_tile<G, kEpi, 2>(p, xcd_contiguous(b, p.whole));
  else
    gemm_tile<G, kEpi, 1>(p, xcd_contiguous(b - p.whole, (int64_t)gridDim.x - p.whole));
}

const void* gemm_kernel_for(int32_t g, int epi) {
  if (epi == kBF16) return reinterpret_cast<const void*>(&gemm_fp8_kernel<128, kBF16>);
  switch (g) {
    case 16: return reinterpret_cast<const void*>(&gemm_fp8_kernel<16, kGroupQuant>);
    case 32: return reinterpret_cast<const void*>(&gemm_fp8_kernel<32, kGroupQuant>);
    case 64: return reinterpret_cast<const void*>(&gemm_fp8_kernel<64, kGroupQuant>);
    default: return reinterpret_cast<const void*>(&gemm_fp8_kernel<128, kGroupQuant>);
  }
}

coat_status_t check_gemm_shape(const uint8_t* a, const uint8_t* b, float a_scale, float b_scale,
                               int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0 || N % kNQuantum != 0 || K % kNQuantum != 0 || K > (1 << 24))
    return COAT_ERR_INVALID_VALUE;
  if (!isfinite(a_scale) || !isfinite(b_scale)) return COAT_ERR_INVALID_VALUE;
  if (M == 0 || N == 0) return COAT_OK;
  if (K > 0 && (!a || !b)) return COAT_ERR_NULL_POINTER;
  if (!aligned(a, 16) || !aligned(b, 16)) return COAT_ERR_MISALIGNED;
  const int64_t m_tiles = (M + kNQuantum - 1) / kNQuantum;   // half tiles, the finest grid
  if (m_tiles > 0x7FFFFFFF / ((N + kBN - 1) / kBN)) return COAT_ERR_INVALID_VALUE;
  return COAT_OK;
}

// One block runs per CU.  When the tiles leave the last round of CUs at most
// half full, the whole rounds run as 256 x 256 tiles and the remaining tiles
// of the order as two 128 x 256 halves each: half a round instead of a full
// one.
hipError_t launch_gemm(GemmParams& p, int32_t group_size, int epi, hipStream_t stream) {
  void* args[] = {&p};
  p.n_tiles = (p.N + kBN - 1) / kBN;
  const int64_t tiles = (p.M + kBM - 1) / kBM * p.n_tiles;
  int cus = 0;
  hipError_t e = current_cu_count(&cus);
  if (e != hipSuccess) return e;
  const int64_t rem = cus > 0 ? tiles % cus : 0;
  p.whole = rem > 0 && 2 * rem <= cus ? tiles - rem : tiles;
  const int64_t blocks = p.whole + 2 * (tiles - p.whole);
  return hipLaunchKernel(gemm_kernel_for(group_size, epi), dim3((unsigned)blocks), dim3(kThreads), args,
                         0, stream);
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
