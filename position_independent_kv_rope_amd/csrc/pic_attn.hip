// Selective attention of the recomputed rows (pic_selective_attn).
//
// EPIC walkthrough, link_legolink Step 3: the recomputed rows' Q, rotated at their
// global positions, attend over the spliced K/V with a causal mask.  For a row at
// position p the visible keys are j <= p, which is the offset mask of "KV cache 从零
// 实现" (allowed[i, j] = [j <= P + i] for a run of rows starting at P).  GQA maps
// query head h to KV head h / G.
//
// Work decomposition (the host planner builds it): an attention tile is
// PIC_ATTN_TILE_M = 64 (row, head) pairs -- 64/G consecutive recomputed rows of one
// request times the G query heads that share one KV head -- so every K/V element
// staged in LDS feeds 64 query vectors.  An item is (tile, kv head, key range); long
// tiles are split along keys and a merge kernel combines the partial results with
// their log-sum-exp weights.
//
// Inside a workgroup (4 waves) each wave owns 16 of the 64 query vectors.  Per block
// of 64 keys the workgroup stages K (row-major) and V (transposed, key-contiguous)
// into LDS, then each wave computes S^T = K Q^T with MFMA (16 keys x 16 queries per
// instruction), runs the online softmax in the exp2 domain with the running max kept
// per query column (the C layout puts one query per lane column, so the row statistics
// need only two cross-lane exchanges), and accumulates O^T += V^T P^T with MFMA.  The
// keys of a 32-key group are permuted between the two S^T instructions so that each
// lane's softmax probabilities are exactly the 8 consecutive keys its PV operand needs.
// bf16 uses v_mfma_f32_16x16x32_bf16 (fp32 accumulate); fp32 uses v_mfma_f32_16x16x4_f32.
#include <cmath>
#include <type_traits>

#include "pic_device.h"
#include "pic_internal.h"

namespace pic {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kKB = 64;  // keys per staged block
constexpr int kM = PIC_ATTN_TILE_M;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

static_assert(kM == 16 * kWaves, "one 16-query MFMA column block per wave");

template <typename T>
struct Cfg;
template <>
struct Cfg<__bf16> {
  static constexpr int kPad = 8;  // elements of padding per LDS row (16 bytes)
};
template <>
struct Cfg<float> {
  static constexpr int kPad = 4;
};

// Key (within a 64-key block) held in C-tile slot i of lane group grp of sub-block sb.
template <typename T>
__device__ __forceinline__ int key_of(int sb, int grp, int i) {
  if constexpr (std::is_same<T, __bf16>::value)
    return 32 * (sb >> 1) + 8 * grp + 4 * (sb & 1) + i;
  else
    return 16 * sb + 4 * grp + i;
}

__device__ __forceinline__ float wave_max_cols(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum_cols(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(
    const T *__restrict__ q, const T *__restrict__ kbuf, const T *__restrict__ vbuf,
    T *__restrict__ out, const int32_t *__restrict__ rows, const AttnTile *__restrict__ tiles,
    const AttnItem *__restrict__ items, float *__restrict__ ws_o, float *__restrict__ ws_ml,
    int h_q, int h_kv, int tile_rows, float scale_log2) {
  constexpr int kPad = Cfg<T>::kPad;
  constexpr int kKs = D + kPad;    // K row stride in LDS (elements)
  constexpr int kVs = kKB + kPad;  // V^T row stride in LDS (elements)
  constexpr int kEPU = 16 / sizeof(T);  // elements per 16-byte unit
  constexpr int kUPR = D / kEPU;        // 16-byte units per key row of one head
  constexpr bool kBf16 = std::is_same<T, __bf16>::value;
  constexpr int kDB = D / 16;           // 16-wide output d blocks
  constexpr int kQOps = kBf16 ? D / 32 : D / 4;

  __shared__ __attribute__((aligned(16))) T ks[kKB * kKs];
  __shared__ __attribute__((aligned(16))) T vt[D * kVs];

  const AttnItem it = items[blockIdx.x];
  const AttnTile tile = tiles[it.tile];
  const int g = it.kv_head;
  const int group = h_q / h_kv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // query column of this lane in C tiles
  const int grp = lane >> 4;  // lane group 0..3

  // ---- the query vector of this lane's column ----
  const int m = 16 * wave + col;
  const int row_local = m % tile_rows;
  const int head = g * group + m / tile_rows;
  const bool valid = row_local < tile.n_rows;
  const int row = tile.row_begin + (valid ? row_local : 0);
  const int pos = valid ? rows[row] : -1;

  typedef typename std::conditional<kBf16, bf16x8, float>::type Op;
  Op qop[kQOps];
  {
    const T *qp = q + ((int64_t)row * h_q + head) * D;
#pragma unroll
    for (int s = 0; s < kQOps; ++s) {
      if constexpr (kBf16) {
        qop[s] = valid ? *reinterpret_cast<const bf16x8 *>(qp + 32 * s + 8 * grp) : bf16x8{};
      } else {
        qop[s] = valid ? qp[4 * s + grp] : 0.0f;
      }
    }
  }

  // lowest position among the wave's valid columns (masking is skipped below it)
  int pos_min = valid ? pos : 0x7fffffff;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) pos_min = min(pos_min, __shfl_xor(pos_min, o));

  f32x4 acc[kDB];
#pragma unroll
  for (int d = 0; d < kDB; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;  // running max of scaled scores (log2 domain), per column
  float l_lane = 0.f;     // this lane's share of the running denominator

  const int key_begin = it.key_begin;
  const int key_end = it.key_end;  // exclusive, <= p_last + 1
  const int key_last = key_end - 1;
  const int64_t head_stride = (int64_t)h_kv * D;
  const T *kbase = kbuf + (int64_t)tile.tok_base * head_stride + (int64_t)g * D;
  const T *vbase = vbuf + (int64_t)tile.tok_base * head_stride + (int64_t)g * D;

  for (int kb0 = key_begin; kb0 < key_end; kb0 += kKB) {
    __syncthreads();
    // ---- stage K (row-major) ----
    for (int u = threadIdx.x; u < kKB * kUPR; u += kThreads) {
      const int key = u / kUPR, c = u - key * kUPR;
      const int kk = min(kb0 + key, key_last);
      *reinterpret_cast<u32x4 *>(&ks[key * kKs + c * kEPU]) =
          *reinterpret_cast<const u32x4 *>(kbase + (int64_t)kk * head_stride + c * kEPU);
    }
    // ---- stage V transposed: 4 keys x one 16-byte unit per work item ----
    for (int u = threadIdx.x; u < (kKB / 4) * kUPR; u += kThreads) {
      const int quad = u / kUPR, c = u - quad * kUPR;
      T e[4][kEPU];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = min(kb0 + 4 * quad + r, key_last);
        const u32x4 raw = *reinterpret_cast<const u32x4 *>(vbase + (int64_t)kk * head_stride + c * kEPU);
        __builtin_memcpy(e[r], &raw, 16);
      }
#pragma unroll
      for (int j = 0; j < kEPU; ++j) {
        T four[4] = {e[0][j], e[1][j], e[2][j], e[3][j]};
        if constexpr (kBf16) {
          uint64_t w;
          __builtin_memcpy(&w, four, 8);
          *reinterpret_cast<uint64_t *>(&vt[(c * kEPU + j) * kVs + 4 * quad]) = w;
        } else {
          u32x4 w;
          __builtin_memcpy(&w, four, 16);
          *reinterpret_cast<u32x4 *>(&vt[(c * kEPU + j) * kVs + 4 * quad]) = w;
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for the 4 sub-blocks of 16 keys ----
    f32x4 sc[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      sc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int krow = key_of<T>(sb, col >> 2, col & 3);  // A row = C row = col here
#pragma unroll
      for (int s = 0; s < kQOps; ++s) {
        if constexpr (kBf16) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&ks[krow * kKs + 32 * s + 8 * grp]);
          sc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[s], sc[sb], 0, 0, 0);
        } else {
          const float a = ks[krow * kKs + 4 * s + grp];
          sc[sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qop[s], sc[sb], 0, 0, 0);
        }
      }
    }

    // ---- mask (only blocks that reach past some column's position or the range end) ----
    if (kb0 + kKB - 1 > min(pos_min, key_last)) {
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb0 + key_of<T>(sb, grp, i);
          if (key > pos || key > key_last) sc[sb][i] = kNegInf;
        }
    }

    // ---- online softmax (exp2 domain) ----
    float mx = kNegInf;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[sb][i]);
    mx = wave_max_cols(mx);
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const bool none = m_new == kNegInf;
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float base = none ? 0.f : m_new;
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[sb][i], scale_log2, -base));
        sc[sb][i] = p;
        psum += p;
      }
    l_lane = l_lane * alpha + psum;
#pragma unroll
    for (int d = 0; d < kDB; ++d) acc[d] *= alpha;

    // ---- O^T += V^T P^T ----
    if constexpr (kBf16) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = (__bf16)sc[2 * h][i];
          pb[4 + i] = (__bf16)sc[2 * h + 1][i];
        }
#pragma unroll
        for (int d = 0; d < kDB; ++d) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&vt[(16 * d + col) * kVs + 32 * h + 8 * grp]);
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[d], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int d = 0; d < kDB; ++d) {
            const float a = vt[(16 * d + col) * kVs + 16 * sb + 4 * grp + i];
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sc[sb][i], acc[d], 0, 0, 0);
          }
    }
  }

  // ---- epilogue ----
  const float l_row = wave_sum_cols(l_lane);
  if (!valid) return;
  if (it.slot < 0) {
    const float inv = 1.f / l_row;
    T *op = out + ((int64_t)row * h_q + head) * D;
#pragma unroll
    for (int d = 0; d < kDB; ++d) {
      if constexpr (kBf16) {
        bf16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (__bf16)(acc[d][i] * inv);
        *reinterpret_cast<bf16x4 *>(op + 16 * d + 4 * grp) = o;
      } else {
        *reinterpret_cast<f32x4 *>(op + 16 * d + 4 * grp) = acc[d] * inv;
      }
    }
  } else {
    float *wo = ws_o + ((int64_t)it.slot * kM + m) * D;
#pragma unroll
    for (int d = 0; d < kDB; ++d) *reinterpret_cast<f32x4 *>(wo + 16 * d + 4 * grp) = acc[d];
    if (grp == 0) {
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 0] = m_run;
      ws_ml[((int64_t)it.slot * kM + m) * 2 + 1] = l_row;
    }
  }
}

// Combine the split partials of one (tile, kv head) with their log-sum-exp weights.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(
    T *__restrict__ out, const int32_t *__restrict__ rows, const AttnTile *__restrict__ tiles,
    const MergeEntry *__restrict__ merges, const float *__restrict__ ws_o,
    const float *__restrict__ ws_ml, int h_q, int h_kv, int tile_rows) {
  (void)rows;
  const MergeEntry me = merges[blockIdx.x];
  const AttnTile tile = tiles[me.tile];
  const int group = h_q / h_kv;
  constexpr int kC = D / 4;  // 4-wide chunks per query vector
  for (int u = threadIdx.x; u < kM * kC; u += kThreads) {
    const int m = u / kC, c = u - m * kC;
    const int row_local = m % tile_rows;
    if (row_local >= tile.n_rows) continue;
    const int head = me.kv_head * group + m / tile_rows;
    float mmax = kNegInf;
    for (int s = 0; s < me.n_slots; ++s)
      mmax = fmaxf(mmax, ws_ml[((int64_t)(me.slot_base + s) * kM + m) * 2]);
    float den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < me.n_slots; ++s) {
      const int64_t at = (int64_t)(me.slot_base + s) * kM + m;
      const float ms = ws_ml[at * 2];
      if (ms == kNegInf) continue;
      const float w = __builtin_amdgcn_exp2f(ms - mmax);
      den += w * ws_ml[at * 2 + 1];
      num += w * *reinterpret_cast<const f32x4 *>(ws_o + at * D + 4 * c);
    }
    const float inv = 1.f / den;
    T *op = out + ((int64_t)(tile.row_begin + row_local) * h_q + head) * D + 4 * c;
    if constexpr (std::is_same<T, __bf16>::value) {
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (__bf16)(num[i] * inv);
      *reinterpret_cast<bf16x4 *>(op) = o;
    } else {
      *reinterpret_cast<f32x4 *>(op) = num * inv;
    }
  }
}

template <typename T, int D>
int launch_attn(const PlanHeader &h, const int32_t *plan_dev, const void *q, const void *k,
                const void *v, void *out, float scale, void *workspace, hipStream_t s) {
  const int32_t *rows = plan_dev + h[PIC_H_O_ROWS];
  const AttnTile *tiles = reinterpret_cast<const AttnTile *>(plan_dev + h[PIC_H_O_ATTN_TILES]);
  const AttnItem *items = reinterpret_cast<const AttnItem *>(plan_dev + h[PIC_H_O_ATTN_ITEMS]);
  const MergeEntry *merges = reinterpret_cast<const MergeEntry *>(plan_dev + h[PIC_H_O_MERGE]);
  float *ws_o = static_cast<float *>(workspace);
  float *ws_ml = ws_o ? ws_o + (int64_t)h[PIC_H_N_PARTIALS] * kM * D : nullptr;
  const float scale_log2 = scale * kLog2e;
  hipLaunchKernelGGL((attn_kernel<T, D>), dim3(h[PIC_H_N_ATTN_ITEMS]), dim3(kThreads), 0, s,
                     static_cast<const T *>(q), static_cast<const T *>(k),
                     static_cast<const T *>(v), static_cast<T *>(out), rows, tiles, items, ws_o,
                     ws_ml, h[PIC_H_H_Q], h[PIC_H_H_KV], h[PIC_H_TILE_ROWS], scale_log2);
  PIC_LAUNCH_CHECK();
  if (h[PIC_H_N_MERGE] > 0) {
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3(h[PIC_H_N_MERGE]), dim3(kThreads), 0, s,
                       static_cast<T *>(out), rows, tiles, merges, ws_o, ws_ml, h[PIC_H_H_Q],
                       h[PIC_H_H_KV], h[PIC_H_TILE_ROWS]);
    PIC_LAUNCH_CHECK();
  }
  return PIC_OK;
}

}  // namespace
}  // namespace pic

extern "C" size_t pic_attn_workspace_bytes(const int32_t *plan_host, int32_t head_dim) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || head_dim <= 0) return 0;
  return (size_t)h[PIC_H_N_PARTIALS] * kM * ((size_t)head_dim + 2) * sizeof(float);
}

extern "C" int pic_selective_attn(const int32_t *plan_host, const int32_t *plan_dev,
                                  const void *q, const void *k, const void *v, void *out,
                                  int32_t dtype, int32_t head_dim, float scale, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid()) return PIC_EINVAL;
  if (dtype != PIC_BF16 && dtype != PIC_F32) return PIC_EINVAL;
  if (!(scale > 0.f) || !std::isfinite(scale) || head_dim <= 0) return PIC_EINVAL;
  if (h[PIC_H_N_ATTN_ITEMS] == 0) return PIC_OK;
  if (!plan_dev || !q || !k || !v || !out) return PIC_EINVAL;
  const size_t need = pic_attn_workspace_bytes(plan_host, head_dim);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PIC_ENOSPC;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PIC_BF16) {
    switch (head_dim) {
      case 64: return launch_attn<__bf16, 64>(h, plan_dev, q, k, v, out, scale, workspace, s);
      case 128: return launch_attn<__bf16, 128>(h, plan_dev, q, k, v, out, scale, workspace, s);
      default: return PIC_EUNSUPPORTED;
    }
  }
  switch (head_dim) {
    case 16: return launch_attn<float, 16>(h, plan_dev, q, k, v, out, scale, workspace, s);
    case 32: return launch_attn<float, 32>(h, plan_dev, q, k, v, out, scale, workspace, s);
    case 64: return launch_attn<float, 64>(h, plan_dev, q, k, v, out, scale, workspace, s);
    case 128: return launch_attn<float, 128>(h, plan_dev, q, k, v, out, scale, workspace, s);
    default: return PIC_EUNSUPPORTED;
  }
}
