// coat_act.hip -- gfx950 kernel and C ABI of the per-group FP8 activation
// quantizer with transposed output (COAT's non-linear-layer quantization).
//
// Sources (see include/coat_fp8.h for the full citations):
//   [P1] COAT paper review (xllm-io.github.io), section 三: mixed-granularity
//        activation quantization (混合粒度激活量化) and the non-linear-layer
//        kernel notes (非线性层优化); 核心公式 "FP8量化".
//   [OCP] OFP8 specification, E4M3 (max 448).

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "coat_common.h"

using namespace coat;

namespace {

// ------------------------------------------- per-group activation quantizer
//
// [P1] section 三, mixed-granularity activation quantization: the tensors of
// non-linear layers are quantized per 1xG group of a row with the FP8量化
// equation (S = max|X| / 448, X_FP8 = round(X / S)), and the non-linear-layer
// kernel emits the FP8 tensor together with its transpose for the backward
// pass.  No expansion here (k = 1).
//
// One block of 256 threads takes a tile of kRows rows x 128 columns (kRows =
// 128; 64 when 128-row tiles would leave at most two per CU, where the finer
// split balances the CUs better: measured at 2048 x 4096, 9.7 -> 8.0 us).
// Load phase: 16 threads cover one 128-column row (16 B = 8 BF16 each), so a
// wave reads 4 rows and a group of G columns sits on G/8 consecutive lanes of
// one 16-lane DPP row.  Each lane reduces its 8 magnitudes, DPP joins the
// group, and the lane converts its values and writes 8 code bytes both to the
// row-major output and to an LDS copy of the tile.  Transpose phase: a thread
// reads a 16-row x 4-column block of the LDS tile as 16 dwords, transposes it
// in registers with byte permutes and writes four 16-byte column runs, so 8
// consecutive lanes fill 128 contiguous bytes of one row of the transpose.

constexpr int kActTileCols = 128;

struct ActParams {
  const uint16_t* x;
  uint8_t* codes;
  float* scales;
  uint8_t* codes_t;
  int64_t rows;
  int64_t cols;
  int64_t col_tiles;
  int64_t groups_per_row;
  int32_t t_store;  // bytes per store into the transpose: 16, 8 or 4 (rows a multiple of it), else 1
};

// Largest BF16 magnitude (as its 15 bits) among the 8 values of a chunk:
// sign-cleared BF16 patterns order like the magnitudes they encode.
__device__ __forceinline__ uint32_t bf16x8_max_mag(uint4 r) {
  const uint32_t a = max(r.x & 0x7FFFu, (r.x >> 16) & 0x7FFFu);
  const uint32_t b = max(r.y & 0x7FFFu, (r.y >> 16) & 0x7FFFu);
  const uint32_t c = max(r.z & 0x7FFFu, (r.z >> 16) & 0x7FFFu);
  const uint32_t d = max(r.w & 0x7FFFu, (r.w >> 16) & 0x7FFFu);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t act_pack4(uint32_t w0, uint32_t w1, const GroupQuot& d) {
  const float q0 = group_quot(bf16_lo(w0), d), q1 = group_quot(bf16_hi(w0), d);
  const float q2 = group_quot(bf16_lo(w1), d), q3 = group_quot(bf16_hi(w1), d);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, v, true);
  return (uint32_t)v;
}

// Streaming accesses of the quantizer: every byte is read or written once, so
// the loads and stores are nontemporal.  Measured on MI355X with inputs that
// do not fit in the last-level cache, this lifts the transposing kernel from
// about 4.6 to 5.1 TB/s at 8192 x 11008.
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream8(void* p, uint2 v) {
  const u32x2v w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2v*>(p));
}

__device__ __forceinline__ void store_stream16(void* p, uint4 v) {
  const u32x4v w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4v*>(p));
}

// LDS tile: kRows rows of 32 dwords.  The dword column is XOR-swizzled by the
// row's 16-row block so that the transpose phase's column reads (one dword
// from each of 16 consecutive rows, 32 lanes on distinct columns and blocks)
// fall on distinct banks.
template <int kRows>
__device__ __forceinline__ int act_swz(int row_block) {
  return (row_block * (512 / kRows)) & 31;
}

template <int G, bool kTranspose, int kRows>
__global__ __launch_bounds__(kBlockThreads) void quantize_act_kernel(const ActParams p) {
  constexpr int kLanes = G / 8;
  constexpr int kActPasses = kRows / 16;
  constexpr int kActRowBlocks = kRows / 16;
  __shared__ uint32_t tile[kTranspose ? kRows * 32 : 1];
  const int t = threadIdx.x;
  const int64_t b = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t tr = b / p.col_tiles;
  const int64_t tc = b - tr * p.col_tiles;
  const int64_t r0 = tr * kRows, c0 = tc * kActTileCols;
  const int chunk = t & 15, rsub = t >> 4;
  const int64_t col = c0 + 8 * chunk;
  const bool col_ok = col < p.cols;

  uint4 raw[kActPasses];
#pragma unroll
  for (int q = 0; q < kActPasses; ++q) {
    const int64_t row = r0 + 16 * q + rsub;
    raw[q] = make_uint4(0, 0, 0, 0);
    if (col_ok && row < p.rows)
      raw[q] = load_stream16(p.x + row * p.cols + col);
  }
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int q = 0; q < kActPasses; ++q) {
    const int64_t row = r0 + 16 * q + rsub;
    const bool ok = col_ok && row < p.rows;
    // groups never straddle a validity boundary: a 16-lane row is one tile
    // row, and cols is a multiple of G
    const uint32_t mag = lanes_max_u32<kLanes>(bf16x8_max_mag(raw[q]));
    const float amax = __uint_as_float(mag << 16);
    const GroupQuot d = group_quot_setup(amax);
    const bool nonzero = amax > 0.0f;
    uint2 c;
    c.x = nonzero ? act_pack4(raw[q].x, raw[q].y, d) : 0u;
    c.y = nonzero ? act_pack4(raw[q].z, raw[q].w, d) : 0u;
    if (ok) {
      store_stream8(p.codes + row * p.cols + col, c);
      if (chunk % kLanes == 0) p.scales[row * p.groups_per_row + col / G] = amax / 448.0f;
    }
    if constexpr (kTranspose) {
      const int lr = 16 * q + rsub;
      *reinterpret_cast<uint2*>(&tile[lr * 32 + ((2 * chunk) ^ act_swz<kRows>(q))]) = c;
    }
  }

  if constexpr (kTranspose) {
    __syncthreads();
    constexpr int kTasks = kActRowBlocks * 32;
    for (int task = t; task < kTasks; task += kBlockThreads) {
      const int rb = task % kActRowBlocks, cb = task / kActRowBlocks;
      const int dcol = cb ^ act_swz<kRows>(rb);
      uint32_t d[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) d[i] = tile[(16 * rb + i) * 32 + dcol];
      // out[j][b]: column 4*cb + j, rows 16*rb + 4*b .. +3 (byte 0 = first row)
      uint32_t out[4][4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t a0 = d[4 * b], a1 = d[4 * b + 1], a2 = d[4 * b + 2], a3 = d[4 * b + 3];
        // v_perm_b32 picks bytes of {S0:S1}, selectors 0-3 from S1, 4-7 from S0
        const uint32_t x0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // a0.0 a1.0 a0.1 a1.1
        const uint32_t x1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // a0.2 a1.2 a0.3 a1.3
        const uint32_t y0 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
        const uint32_t y1 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
        out[0][b] = __builtin_amdgcn_perm(y0, x0, 0x05040100u);
        out[1][b] = __builtin_amdgcn_perm(y0, x0, 0x07060302u);
        out[2][b] = __builtin_amdgcn_perm(y1, x1, 0x05040100u);
        out[3][b] = __builtin_amdgcn_perm(y1, x1, 0x07060302u);
      }
      const int64_t row = r0 + 16 * rb;
      if (row >= p.rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = c0 + 4 * cb + j;
        if (c >= p.cols) continue;
        // dst is aligned to the largest of 16, 8, 4 dividing rows (codes_t is
        // 16-byte aligned, row a multiple of 16)
        uint8_t* dst = p.codes_t + c * p.rows + row;
        const bool whole = row + 16 <= p.rows;
        if (whole && p.t_store == 16) {
          store_stream16(dst, make_uint4(out[j][0], out[j][1], out[j][2], out[j][3]));
        } else if (whole && p.t_store == 8) {
          store_stream8(dst, make_uint2(out[j][0], out[j][1]));
          store_stream8(dst + 8, make_uint2(out[j][2], out[j][3]));
        } else if (whole && p.t_store == 4) {
#pragma unroll
          for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(dst + 4 * i) = out[j][i];
        } else {
          for (int i = 0; i < 16 && row + i < p.rows; ++i)
            dst[i] = (uint8_t)(out[j][i >> 2] >> (8 * (i & 3)));
        }
      }
    }
  }
}

template <int G, int kRows>
const void* act_fn(bool transpose) {
  return transpose ? reinterpret_cast<const void*>(&quantize_act_kernel<G, true, kRows>)
                   : reinterpret_cast<const void*>(&quantize_act_kernel<G, false, kRows>);
}

template <int kRows>
const void* act_kernel_rows(int32_t g, bool transpose) {
  switch (g) {
    case 16: return act_fn<16, kRows>(transpose);
    case 32: return act_fn<32, kRows>(transpose);
    case 64: return act_fn<64, kRows>(transpose);
    default: return act_fn<128, kRows>(transpose);
  }
}

}  // namespace

extern "C" {

coat_status_t coat_fp8_quantize_act(const uint16_t* x, int64_t rows, int64_t cols,
                                    int32_t group_size, uint8_t* codes, float* scales,
                                    uint8_t* codes_t, hipStream_t stream) {
  if (rows < 0 || cols < 0) return COAT_ERR_INVALID_VALUE;
  if (!valid_group_size(group_size)) return COAT_ERR_GROUP_SIZE;
  if (cols % group_size != 0) return COAT_ERR_INVALID_VALUE;
  if (rows == 0 || cols == 0) return COAT_OK;
  if (!x || !codes || !scales) return COAT_ERR_NULL_POINTER;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) ||
      (codes_t && !aligned(codes_t, 16)))
    return COAT_ERR_MISALIGNED;
  ActParams p;
  memset(&p, 0, sizeof(p));
  p.x = x;
  p.codes = codes;
  p.scales = scales;
  p.codes_t = codes_t;
  p.rows = rows;
  p.cols = cols;
  p.col_tiles = (cols + kActTileCols - 1) / kActTileCols;
  p.groups_per_row = cols / group_size;
  p.t_store = rows % 16 == 0 ? 16 : rows % 8 == 0 ? 8 : rows % 4 == 0 ? 4 : 1;
  const int64_t row_tiles = (rows + 127) / 128;   // in 128-row tiles
  if (row_tiles > 0x7FFFFFFF / p.col_tiles) return COAT_ERR_INVALID_VALUE;
  int cus = 0;
  hipError_t e = current_cu_count(&cus);
  if (e != hipSuccess) return hip_fail(e);
  const bool short_tiles = row_tiles * p.col_tiles <= 2 * (int64_t)cus;
  const bool transpose = codes_t != nullptr;
  const void* fn = short_tiles ? act_kernel_rows<64>(group_size, transpose)
                               : act_kernel_rows<128>(group_size, transpose);
  const int64_t blocks = (short_tiles ? (rows + 63) / 64 : row_tiles) * p.col_tiles;
  void* args[] = {&p};
  e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kBlockThreads), args, 0, stream);
  return e == hipSuccess ? COAT_OK : hip_fail(e);
}

}  // extern "C"
