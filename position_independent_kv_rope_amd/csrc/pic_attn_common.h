// Shared pieces of the attention kernels (pic_attn.hip: contiguous spliced K/V;
// pic_attn_paged.hip: the shared-chunk pool; pic_decode.hip: one decode step over the
// pool): tile constants, the MFMA operand layouts in LDS, the lane-pair reductions,
// the per-chunk angle table, the key-block record, the split-KV merge and the
// workspace layout of split partials.
#pragma once

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "pic_device.h"
#include "pic_internal.h"

namespace pic {
namespace {

constexpr int kM = PIC_ATTN_TILE_M;  // query vectors per tile
constexpr int kKB = 64;              // keys per staged block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bool wave_any(bool p) { return __any((int)p); }

// max / sum of a value over the lane pair (l, l ^ 32), in the VALU (v_permlane32_swap)
__device__ __forceinline__ float pair_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// The lane id, produced afresh at each call (an opaque instruction pair the compiler
// cannot merge with another), so values derived from it on a rarely taken path are
// recomputed there instead of being held across the main loop: in a kernel at the
// register limit such values get spilled, and reloading a spill is a vector memory load
// whose wait also waits for every direct load issued before it.
__device__ __forceinline__ int fresh_lane() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// ================================ bf16 kernel ==================================

constexpr int kBfWaves = 4;
constexpr int kBfThreads = 64 * kBfWaves;
static_assert(kM == 32 * kBfWaves, "one 32-query MFMA column block per wave");

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// Key (0..31 within a 32-key S^T tile t of the 64-key block) at C row r: rows held by
// lane group g in accumulator slots 8h..8h+7 become keys 16(2t+h) + 8g + 0..7.
__device__ __forceinline__ int perm_key(int t, int r) {
  const int a = r >> 3, g = (r >> 2) & 1, b = r & 3;
  return 16 * (2 * t + (a >> 1)) + 8 * g + 4 * (a & 1) + b;
}

// LDS layouts: a staged block is 64 key rows of D bf16, rows unpadded, 16-byte chunks
// XOR-swizzled per row so that the reads of one LDS cycle hit distinct banks.
// K rows are read 16 at a time (rows {0..3, 8..11, 16..19, 24..27} + const, one chunk
// each): the swizzle takes 16 distinct values over such a set.  V rows are read by the
// transposing loads 4 consecutive rows at a time, two lane groups on adjacent chunk
// pairs: XOR of chunk bits 2-3 by (row & 3) puts the four rows on four distinct
// 64-byte bank groups.
template <int kCPR>
__device__ __forceinline__ int swz_k(int r) {
  return ((r & 3) | (((r >> 3) & 3) << 2)) & (kCPR - 1);
}
template <int kCPR>
__device__ __forceinline__ int swz_v(int r) {
  return (4 * (r & 3)) & (kCPR - 1);
}

// fp32 kernels: 8 waves x 16 queries
constexpr int kF32Waves = 8;
constexpr int kF32Threads = 64 * kF32Waves;
static_assert(kM == 16 * kF32Waves, "one 16-query MFMA column block per wave");

constexpr int kPoolBlockRows = 16;

// cos/sin(delta_c * theta_i) for every chunk c and pair i of the plan.
__global__ __launch_bounds__(256) void paged_angles_kernel(float2 *__restrict__ angles,
                                                           const int32_t *__restrict__ segs,
                                                           int n_chunks, int n_pairs,
                                                           ThetaTable theta) {
  const int64_t total = (int64_t)n_chunks * n_pairs;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * 256) {
    const int c = (int)(u / n_pairs), i = (int)(u - (int64_t)c * n_pairs);
    angles[u] = delta_cos_sin(segs[8 * c + 4], theta.hi[i], theta.lo[i]);
  }
}

// Everything the attention kernel needs to stage and mask one 64-key block, resolved
// once per launch so that the kernel reads a single 32-byte record per block (one
// scalar load) instead of walking segment -> chunk -> block table with dependent loads.
struct KeyBlockRec {
  int32_t frame;     // global chunk index c (its angle row), or -1: the request's fresh rows
  int32_t row;       // fresh: first fresh row of the block; pool: first local key t0
  int32_t base_pos;  // pool: global position of local key t0
  int32_t vis;       // pool: visible local keys [s0, nv) of the block as s0 | nv << 8
  int32_t off[4];    // pool: byte offset of each 16-row pool block, -1: reads zeros
};
static_assert(sizeof(KeyBlockRec) == 32, "one s_load_dwordx8 per record");
static_assert(kKB == 4 * kPoolBlockRows, "a key block spans four pool blocks");

}  // namespace
}  // namespace pic

namespace pic {
namespace {

// ================================ merge ========================================

// Combine the split partials of each (tile, kv head) with their log-sum-exp weights:
// one thread per (merge entry, query vector, 8 output dims: 16-byte partial loads), a
// single pass over the slots with an online maximum.  The bf16 kernels store partial O in bf16 (one rounding
// of an unnormalised sum, which the merge weights by exp(m) and divides by the summed
// l), the fp32 kernel in fp32; both sit at the start of the same fp32-sized region.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(
    T *__restrict__ out, const AttnTile *__restrict__ tiles, const MergeEntry *__restrict__ merges,
    const float *__restrict__ ws_o, const float *__restrict__ ws_ml, int h_q, int h_kv,
    int tile_rows, int n_merge) {
  constexpr int kV = 8;  // output dims per thread
  constexpr int kC = D / kV;
  typedef __attribute__((__vector_size__(kV * sizeof(float)))) float f32x8;
  const int group = h_q / h_kv;
  const int64_t total = (int64_t)n_merge * kM * kC;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * 256) {
    const int e = (int)(u / (kM * kC));
    const int rem = (int)(u - (int64_t)e * (kM * kC));
    const int m = rem / kC, c = rem - m * kC;
    const MergeEntry me = merges[e];
    const AttnTile tile = tiles[me.tile];
    const int row_local = m % tile_rows;
    if (row_local >= tile.n_rows) continue;
    const int head = me.kv_head * group + m / tile_rows;
    float mmax = kNegInf, den = 0.f;
    f32x8 num = {};
#pragma unroll 4
    for (int s = 0; s < me.n_slots; ++s) {
      const int64_t at = (int64_t)(me.slot_base + s) * kM + m;
      const float2 ml = *reinterpret_cast<const float2 *>(ws_ml + at * 2);
      f32x8 os;
      if constexpr (std::is_same<T, __bf16>::value) {
        const bf16x8 ob =
            *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const __bf16 *>(ws_o) + at * D + kV * c);
#pragma unroll
        for (int i = 0; i < kV; ++i) os[i] = (float)ob[i];
      } else {
        os = *reinterpret_cast<const f32x8 *>(ws_o + at * D + kV * c);
      }
      const float ms = ml.x, ls = ml.y;
      if (ms == kNegInf) continue;
      if (ms > mmax) {
        const float r = __builtin_amdgcn_exp2f(mmax - ms);  // 0 when mmax is -inf
        den *= r;
        num *= r;
        mmax = ms;
      }
      const float w = __builtin_amdgcn_exp2f(ms - mmax);
      den += w * ls;
      num += w * os;
    }
    const float inv = 1.f / den;
    T *op = out + ((int64_t)(tile.row_begin + row_local) * h_q + head) * D + kV * c;
    if constexpr (std::is_same<T, __bf16>::value) {
      bf16x8 o;
#pragma unroll
      for (int i = 0; i < kV; ++i) o[i] = (__bf16)(num[i] * inv);
      *reinterpret_cast<bf16x8 *>(op) = o;
    } else {
      *reinterpret_cast<f32x8 *>(op) = num * inv;
    }
  }
}

// The same merge with four adjacent lanes per output, for plans whose merges average
// many slots (tens on a 32k-token request, where one lane per output waits for one load
// latency per few slots): lane j of the four folds slots j, j + 4, ... with all of its
// loads issued before its first fold, then the four partial states are combined across
// the lanes and lane 0 stores.  With a few slots per merge the one-lane kernel is as
// fast and launches a quarter of the workgroups, so it stays the default.
constexpr int kMergeWideFrom = 16;  // mean slots per merge from which the wide kernel runs

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel_x4(
    T *__restrict__ out, const AttnTile *__restrict__ tiles, const MergeEntry *__restrict__ merges,
    const float *__restrict__ ws_o, const float *__restrict__ ws_ml, int h_q, int h_kv,
    int tile_rows, int n_merge) {
  constexpr int kV = 8;
  constexpr int kC = D / kV;
  constexpr int kLanes = 4, kBatch = 4;
  typedef __attribute__((__vector_size__(kV * sizeof(float)))) float f32x8;
  const int group = h_q / h_kv;
  // the four lanes of a group run the same iterations (total and the grid stride are
  // multiples of four), so the exchange below sees all of them
  const int64_t total = (int64_t)n_merge * kM * kC * kLanes;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * 256) {
    const int j = (int)(u % kLanes);
    const int64_t w = u / kLanes;
    const int e = (int)(w / (kM * kC));
    const int rem = (int)(w - (int64_t)e * (kM * kC));
    const int m = rem / kC, c = rem - m * kC;
    const MergeEntry me = merges[e];
    const AttnTile tile = tiles[me.tile];
    const int row_local = m % tile_rows;
    if (row_local >= tile.n_rows) continue;  // the same for the four lanes
    const int head = me.kv_head * group + m / tile_rows;
    float mmax = kNegInf, den = 0.f;
    f32x8 num = {};
    auto fold = [&](float ms, float ls, const f32x8 &os) {
      if (ms == kNegInf) return;
      if (ms > mmax) {
        const float r = __builtin_amdgcn_exp2f(mmax - ms);  // 0 when mmax is -inf
        den *= r;
        num *= r;
        mmax = ms;
      }
      const float wt = __builtin_amdgcn_exp2f(ms - mmax);
      den += wt * ls;
      num += wt * os;
    };
    for (int s0 = j; s0 < me.n_slots; s0 += kLanes * kBatch) {
      float2 ml[kBatch];
      f32x8 os[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int sl = s0 + b * kLanes;
        ml[b] = make_float2(kNegInf, 0.f);
        os[b] = f32x8{};
        if (sl < me.n_slots) {
          const int64_t at = (int64_t)(me.slot_base + sl) * kM + m;
          ml[b] = *reinterpret_cast<const float2 *>(ws_ml + at * 2);
          if constexpr (std::is_same<T, __bf16>::value) {
            const bf16x8 ob = *reinterpret_cast<const bf16x8 *>(
                reinterpret_cast<const __bf16 *>(ws_o) + at * D + kV * c);
#pragma unroll
            for (int i = 0; i < kV; ++i) os[b][i] = (float)ob[i];
          } else {
            os[b] = *reinterpret_cast<const f32x8 *>(ws_o + at * D + kV * c);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) fold(ml[b].x, ml[b].y, os[b]);
    }
#pragma unroll
    for (int x = 1; x < kLanes; x <<= 1) {
      const float om = __shfl_xor(mmax, x), ol = __shfl_xor(den, x);
      f32x8 on;
#pragma unroll
      for (int i = 0; i < kV; ++i) on[i] = __shfl_xor(num[i], x);
      fold(om, ol, on);
    }
    if (j != 0) continue;
    const float inv = 1.f / den;
    T *op = out + ((int64_t)(tile.row_begin + row_local) * h_q + head) * D + kV * c;
    if constexpr (std::is_same<T, __bf16>::value) {
      bf16x8 o;
#pragma unroll
      for (int i = 0; i < kV; ++i) o[i] = (__bf16)(num[i] * inv);
      *reinterpret_cast<bf16x8 *>(op) = o;
    } else {
      *reinterpret_cast<f32x8 *>(op) = num * inv;
    }
  }
}

// Launch the merge of a plan's split partials (nothing when the plan has none).
template <typename T, int D>
int launch_merge(const PlanHeader &h, const AttnTile *tiles, const MergeEntry *merges, void *out,
                 const float *ws_o, const float *ws_ml, hipStream_t s) {
  if (h[PIC_H_N_MERGE] == 0) return PIC_OK;
  const bool wide = h[PIC_H_N_PARTIALS] >= (int64_t)kMergeWideFrom * h[PIC_H_N_MERGE];
  const int64_t threads = (int64_t)h[PIC_H_N_MERGE] * kM * (D / 8) * (wide ? 4 : 1);
  const unsigned blocks = (unsigned)std::min<int64_t>((threads + 255) / 256, 1 << 20);
  if (wide)
    hipLaunchKernelGGL((merge_kernel_x4<T, D>), dim3(blocks), dim3(256), 0, s,
                       static_cast<T *>(out), tiles, merges, ws_o, ws_ml, h[PIC_H_H_Q],
                       h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], h[PIC_H_N_MERGE]);
  else
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3(blocks), dim3(256), 0, s,
                       static_cast<T *>(out), tiles, merges, ws_o, ws_ml, h[PIC_H_H_Q],
                       h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], h[PIC_H_N_MERGE]);
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}

// Workspace layout: partial O [slots][kM][D], partial (m, l) [slots][kM][2], then for
// paged plans the angle table [n_chunks][D/2] float2 and the key-block records
// [n_kblocks] (sections 16-byte aligned).
size_t partial_bytes(const PlanHeader &h, int head_dim) {
  return (size_t)h[PIC_H_N_PARTIALS] * kM * ((size_t)head_dim + 2) * sizeof(float);
}
size_t angle_offset(const PlanHeader &h, int head_dim) {
  return (partial_bytes(h, head_dim) + 15) / 16 * 16;
}
size_t keyblock_offset(const PlanHeader &h, int head_dim) {
  return angle_offset(h, head_dim) +
         ((size_t)h[PIC_H_N_CHUNKS] * (head_dim / 2) * sizeof(float2) + 15) / 16 * 16;
}

}  // namespace
}  // namespace pic
