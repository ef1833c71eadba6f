// The per-layer part of the link that surrounds the attention (pic_qkv_rope,
// pic_out_proj) and the multi-layer link itself (pic_link).
//
// EPIC walkthrough, link_legolink Step 3 runs over the model's layers: in each layer
// the recomputed rows' Q, K and V are computed from their hidden states with RoPE at
// their global positions (compute_qkv), the fresh K/V replace the cached rows, the
// rows attend over the spliced K/V, and the attention output becomes the rows' input
// to the next layer.  The layer here closes that loop with the plainest block: an
// output projection added to the hidden state (x <- x + O W_o^T).
//
// Both projections are NT GEMMs, C[m][n] = sum_k A[m][k] W[n][k] (activations row-major,
// weights in the nn.Linear layout: one row per output feature), on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  A workgroup computes a 128 x 128
// tile with 4 waves (2 x 2, 64 x 64 each); K is staged 64 at a time (128-byte rows) by
// direct buffer->LDS loads into a double-buffered, XOR-swizzled LDS tile, so staging
// costs no registers and rows past M read as zero through the buffer range.  The
// epilogue goes through LDS: the fp32 tile is written there, then each thread takes
// one token row and rotates its (Q or K) feature pairs with cos/sin of p_r * theta_i
// from a per-row table (same double-float angle as the rope kernels) before storing
// bf16 heads, or adds the tile to the residual stream.
#include <algorithm>
#include <cmath>

#include "pic_device.h"
#include "pic_internal.h"

namespace pic {
namespace {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kGT = 128;                 // tile rows (tokens) and columns (features)
constexpr int kGK = 64;                  // k per stage
constexpr int kGThreads = 256;           // 4 waves
constexpr int kGRowB = kGK * 2;          // bytes of one staged row
constexpr int kGStageB = kGT * kGRowB;   // one operand, one stage: 16 KiB
constexpr int kGRounds = kGStageB / (1024 * 4);  // direct loads per wave per operand
constexpr int kGCStride = kGT + 4;       // floats per row of the epilogue tile
constexpr int kGLdsBytes =
    (4 * kGStageB > kGT * kGCStride * 4) ? 4 * kGStageB : kGT * kGCStride * 4;

enum { kEpiQkvRope = 0, kEpiResidual = 1 };

// 16-byte chunk swizzle of a 128-byte staged row: the 16 rows one LDS cycle of a
// 128-bit read touches (same chunk index) land on 16 distinct bank groups.
__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

struct QkvOut {
  __bf16 *q, *k, *v;
  const float2 *cs;  // [M][D/2] cos/sin of p_r * theta_i
  int h_q, h_kv;
};

// Output tile of a workgroup.  Consecutive workgroups go round-robin to the 8 XCDs
// (each with its own L2), so workgroup b works on position (b % 8) * per + b / 8 of
// the tile sequence: every XCD takes one contiguous stretch.  The sequence walks groups
// of kGroupM row tiles column by column, so the ~64 tiles an XCD runs at once form an
// 8 x 8 block that shares its A and W tiles in that XCD's L2 as they stream through K.
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ bool gemm_tile(int mt, int nt, int &tm, int &tn) {
  const int total = mt * nt;
  const int per = (total + kXcds - 1) / kXcds;
  const int u = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (u >= total) return false;
  const int g = u / (kGroupM * nt);
  const int gm = min(kGroupM, mt - g * kGroupM);
  const int w = u - g * kGroupM * nt;
  tm = g * kGroupM + w % gm;
  tn = w / gm;
  return true;
}

inline unsigned gemm_grid(int mt, int nt) {
  return (unsigned)(((int64_t)mt * nt + kXcds - 1) / kXcds * kXcds);
}

template <int kEpi, int D, bool kHalf>
__device__ __forceinline__ void gemm_nt_body(const __bf16 *__restrict__ A,
                                             const __bf16 *__restrict__ W, int M, int K, int N,
                                             int tm, int tn, QkvOut qo,
                                             __bf16 *__restrict__ x) {
  __shared__ __attribute__((aligned(1024))) char lds[kGLdsBytes];
  const int m0 = tm * kGT, n0 = tn * kGT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int n = lane & 31, grp = lane >> 5;
  const int row_bytes = K * 2;

  // ---- staging: 128 rows x 128 bytes of A and of W per stage ----
  const int rows_a = min(M - m0, kGT);
  int voff[kGRounds];
#pragma unroll
  for (int r = 0; r < kGRounds; ++r) {
    const int R = 8 * (4 * r + wave) + (lane >> 3);  // staged row this lane fills
    voff[r] = R * row_bytes + 16 * ((lane & 7) ^ gswz(R));
  }
  auto issue = [&](int j, int buf) {
    // rows past M: offsets beyond the resource's records read zero
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + (int64_t)m0 * K), 0, rows_a * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(W + (int64_t)n0 * K), 0, kGT * row_bytes, 0x00020000);
    const int kb = j * kGRowB;
#pragma unroll
    for (int r = 0; r < kGRounds; ++r) {
      const int dst = buf * 2 * kGStageB + (4 * r + wave) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(lds + dst), 16, voff[r] + kb, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(lds + dst + kGStageB), 16,
                                               voff[r] + kb, 0, 0, 0);
    }
  };

  // ---- LDS read offsets of this lane's operand rows ----
  int aoff[2], boff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ra = wm * 64 + 32 * i + n, rb = wn * 64 + 32 * i + n;
    aoff[i] = ra * kGRowB;
    boff[i] = kGStageB + rb * kGRowB;
  }
  int sa[2], sb[2];  // swizzle of each operand row
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    sa[i] = gswz(wm * 64 + 32 * i + n);
    sb[i] = gswz(wn * 64 + 32 * i + n);
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int n_stages = K / kGK;
  issue(0, 0);
  for (int j = 0; j < n_stages; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_stages) {
      issue(j + 1, buf ^ 1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kGRounds) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_barrier" ::: "memory");
    const char *base = lds + buf * 2 * kGStageB;
#pragma unroll
    for (int s = 0; s < kGK / 16; ++s) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8 *>(base + aoff[i] + 16 * ((2 * s + grp) ^ sa[i]));
        b[i] = *reinterpret_cast<const bf16x8 *>(base + boff[i] + 16 * ((2 * s + grp) ^ sb[i]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[jj], acc[i][jj], 0, 0, 0);
    }
    asm volatile("s_barrier" ::: "memory");  // buffer buf is refilled next
  }

  // ---- epilogue through LDS: C[m][n] fp32, row stride kGCStride ----
  float *ct = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ml = wm * 64 + 32 * i + 8 * (e >> 2) + 4 * grp + (e & 3);
        const int nl = wn * 64 + 32 * jj + n;
        ct[ml * kGCStride + nl] = acc[i][jj][e];
      }
  __syncthreads();

  const int ml = threadIdx.x >> 1, part = threadIdx.x & 1;
  const int m = m0 + ml;
  if (m >= M) return;
  const float *crow = ct + ml * kGCStride;
  if constexpr (kEpi == kEpiResidual) {
    // x[m][n0 + f] += C[m][f] for this thread's 64 features
    __bf16 *xr = x + (int64_t)m * N + n0 + 64 * part;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      bf16x8 v = *reinterpret_cast<const bf16x8 *>(xr + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (__bf16)((float)v[e] + crow[64 * part + 8 * c + e]);
      *reinterpret_cast<bf16x8 *>(xr + 8 * c) = v;
    }
  } else {
    constexpr int kHeads = kGT / D;  // whole heads per tile
    const int head0 = n0 / D;
    int region, h0, hcount;
    __bf16 *dst;
    if (head0 < qo.h_q) {
      region = 0, h0 = head0, hcount = qo.h_q, dst = qo.q;
    } else if (head0 < qo.h_q + qo.h_kv) {
      region = 1, h0 = head0 - qo.h_q, hcount = qo.h_kv, dst = qo.k;
    } else {
      region = 2, h0 = head0 - qo.h_q - qo.h_kv, hcount = qo.h_kv, dst = qo.v;
    }
    __bf16 *out = dst + ((int64_t)m * hcount + h0) * D;  // kHeads consecutive heads
    if (region == 2) {  // V: no rotation
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)crow[64 * part + 8 * c + e];
        *reinterpret_cast<bf16x8 *>(out + 64 * part + 8 * c) = v;
      }
      return;
    }
    // Q or K: the tile's kHeads * D/2 = 64 pairs; this thread rotates pairs
    // [32 * part, 32 * part + 32), eight at a time
    const float2 *cs = qo.cs + (int64_t)m * (D / 2);
#pragma unroll
    for (int g8 = 0; g8 < 4; ++g8) {
      const int p0 = 32 * part + 8 * g8;  // first pair of this group
      const int hh = p0 / (D / 2), i0 = p0 % (D / 2);
      float2 c8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) c8[e] = cs[i0 + e];
      if constexpr (!kHalf) {  // pairs (2i, 2i+1): 16 consecutive features
        const float *src = crow + hh * D + 2 * i0;
        bf16x8 lo, hi;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = src[2 * e], b = src[2 * e + 1];
          const float ra = a * c8[e].x - b * c8[e].y, rb = a * c8[e].y + b * c8[e].x;
          if (e < 4) {
            lo[2 * e] = (__bf16)ra;
            lo[2 * e + 1] = (__bf16)rb;
          } else {
            hi[2 * (e - 4)] = (__bf16)ra;
            hi[2 * (e - 4) + 1] = (__bf16)rb;
          }
        }
        *reinterpret_cast<bf16x8 *>(out + hh * D + 2 * i0) = lo;
        *reinterpret_cast<bf16x8 *>(out + hh * D + 2 * i0 + 8) = hi;
      } else {  // pairs (i, i + D/2)
        const float *src = crow + hh * D + i0;
        bf16x8 lo, hi;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = src[e], b = src[e + D / 2];
          lo[e] = (__bf16)(a * c8[e].x - b * c8[e].y);
          hi[e] = (__bf16)(a * c8[e].y + b * c8[e].x);
        }
        *reinterpret_cast<bf16x8 *>(out + hh * D + i0) = lo;
        *reinterpret_cast<bf16x8 *>(out + hh * D + i0 + D / 2) = hi;
      }
      (void)kHeads;
    }
  }
}

template <int D, bool kHalf>
__global__ __launch_bounds__(kGThreads, 2) void qkv_rope_gemm_kernel(const __bf16 *__restrict__ x,
                                                                     const __bf16 *__restrict__ w,
                                                                     int M, int K, int N, QkvOut qo) {
  int tm, tn;
  if (!gemm_tile((M + kGT - 1) / kGT, N / kGT, tm, tn)) return;
  gemm_nt_body<kEpiQkvRope, D, kHalf>(x, w, M, K, N, tm, tn, qo, nullptr);
}

template <int D>
__global__ __launch_bounds__(kGThreads, 2) void out_proj_gemm_kernel(const __bf16 *__restrict__ o,
                                                                     const __bf16 *__restrict__ w,
                                                                     int M, int K, int N,
                                                                     __bf16 *__restrict__ x) {
  int tm, tn;
  if (!gemm_tile((M + kGT - 1) / kGT, N / kGT, tm, tn)) return;
  gemm_nt_body<kEpiResidual, D, false>(o, w, M, K, N, tm, tn, QkvOut{}, x);
}

// cos/sin of p_r * theta_i for every recomputed row r and pair i
__global__ __launch_bounds__(256) void row_angles_kernel(float2 *__restrict__ cs,
                                                         const int32_t *__restrict__ rows,
                                                         int n_rows, int n_pairs,
                                                         ThetaTable theta) {
  const int64_t total = (int64_t)n_rows * n_pairs;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * 256) {
    const int r = (int)(u / n_pairs), i = (int)(u - (int64_t)r * n_pairs);
    cs[u] = delta_cos_sin(rows[r], theta.hi[i], theta.lo[i]);
  }
}

size_t angle_table_bytes(const PlanHeader &h, int head_dim) {
  return ((size_t)h[PIC_H_N_ROWS] * (head_dim / 2) * sizeof(float2) + 255) / 256 * 256;
}

// shape checks shared by the two projections
int check_gemm(const PlanHeader &h, int32_t dtype, int32_t d_model, int32_t head_dim) {
  if (dtype != PIC_BF16 && dtype != PIC_F32) return PIC_EINVAL;
  if (d_model <= 0 || head_dim <= 0 || head_dim % 2) return PIC_EINVAL;
  if (dtype != PIC_BF16) return PIC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PIC_EUNSUPPORTED;
  if (d_model % kGK) return PIC_EUNSUPPORTED;
  if ((int64_t)kGT * d_model * 2 > 0x7fff0000LL) return PIC_EUNSUPPORTED;
  (void)h;
  return PIC_OK;
}

template <int D, bool kHalf>
int launch_qkv(const PlanHeader &h, const int32_t *plan_dev, const void *x, const void *w,
               void *q, void *kf, void *vf, int d_model, double rope_base, void *workspace,
               hipStream_t s) {
  const int M = h[PIC_H_N_ROWS];
  float2 *cs = static_cast<float2 *>(workspace);
  {
    const int64_t total = (int64_t)M * (D / 2);
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65535);
    hipLaunchKernelGGL(row_angles_kernel, dim3(blocks), dim3(256), 0, s, cs,
                       plan_dev + h[PIC_H_O_ROWS], M, D / 2, make_theta(D, rope_base));
    PIC_LAUNCH_CHECK();
  }
  const int n_out = (h[PIC_H_H_Q] + 2 * h[PIC_H_H_KV]) * D;
  QkvOut qo{static_cast<__bf16 *>(q), static_cast<__bf16 *>(kf), static_cast<__bf16 *>(vf), cs,
            h[PIC_H_H_Q], h[PIC_H_H_KV]};
  hipLaunchKernelGGL((qkv_rope_gemm_kernel<D, kHalf>), dim3(gemm_grid((M + kGT - 1) / kGT, n_out / kGT)),
                     dim3(kGThreads), 0, s, static_cast<const __bf16 *>(x),
                     static_cast<const __bf16 *>(w), M, d_model, n_out, qo);
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}

}  // namespace
}  // namespace pic

extern "C" size_t pic_qkv_workspace_bytes(const int32_t *plan_host, int32_t head_dim) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || head_dim <= 0) return 0;
  return angle_table_bytes(h, head_dim);
}

extern "C" int pic_qkv_rope(const int32_t *plan_host, const int32_t *plan_dev, const void *x,
                            const void *w_qkv, void *q, void *k_fresh, void *v_fresh,
                            int32_t dtype, int32_t d_model, int32_t head_dim,
                            int32_t rope_layout, double rope_base, void *workspace,
                            size_t workspace_bytes, void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid()) return PIC_EINVAL;
  if (rope_layout != PIC_ROPE_ADJACENT && rope_layout != PIC_ROPE_HALF) return PIC_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return PIC_EINVAL;
  const int st = check_gemm(h, dtype, d_model, head_dim);
  if (st != PIC_OK) return st;
  // every Q/K/V region must be whole 128-feature tiles; positions exact in fp32
  if ((h[PIC_H_H_Q] * head_dim) % kGT || (h[PIC_H_H_KV] * head_dim) % kGT) return PIC_EUNSUPPORTED;
  if (h[PIC_H_MAX_TOKENS] > (1 << 24)) return PIC_EUNSUPPORTED;
  if (h[PIC_H_N_ROWS] == 0) return PIC_OK;
  if (!plan_dev || !x || !w_qkv || !q || !k_fresh || !v_fresh || !workspace) return PIC_EINVAL;
  if (workspace_bytes < angle_table_bytes(h, head_dim)) return PIC_ENOSPC;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool half = rope_layout == PIC_ROPE_HALF;
  if (head_dim == 128)
    return half ? launch_qkv<128, true>(h, plan_dev, x, w_qkv, q, k_fresh, v_fresh, d_model, rope_base, workspace, s)
                : launch_qkv<128, false>(h, plan_dev, x, w_qkv, q, k_fresh, v_fresh, d_model, rope_base, workspace, s);
  return half ? launch_qkv<64, true>(h, plan_dev, x, w_qkv, q, k_fresh, v_fresh, d_model, rope_base, workspace, s)
              : launch_qkv<64, false>(h, plan_dev, x, w_qkv, q, k_fresh, v_fresh, d_model, rope_base, workspace, s);
}

extern "C" int pic_out_proj(const int32_t *plan_host, const void *o, const void *w_o, void *x,
                            int32_t dtype, int32_t d_model, int32_t head_dim, void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid()) return PIC_EINVAL;
  const int st = check_gemm(h, dtype, d_model, head_dim);
  if (st != PIC_OK) return st;
  const int k_in = h[PIC_H_H_Q] * head_dim;  // the GEMM's reduction length
  if (d_model % kGT || k_in % kGK || (int64_t)kGT * k_in * 2 > 0x7fff0000LL) return PIC_EUNSUPPORTED;
  const int M = h[PIC_H_N_ROWS];
  if (M == 0) return PIC_OK;
  if (!o || !w_o || !x) return PIC_EINVAL;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128)
    hipLaunchKernelGGL((out_proj_gemm_kernel<128>), dim3(gemm_grid((M + kGT - 1) / kGT, d_model / kGT)),
                       dim3(kGThreads), 0, s, static_cast<const __bf16 *>(o),
                       static_cast<const __bf16 *>(w_o), M, k_in, d_model, static_cast<__bf16 *>(x));
  else
    hipLaunchKernelGGL((out_proj_gemm_kernel<64>), dim3(gemm_grid((M + kGT - 1) / kGT, d_model / kGT)),
                       dim3(kGThreads), 0, s, static_cast<const __bf16 *>(o),
                       static_cast<const __bf16 *>(w_o), M, k_in, d_model, static_cast<__bf16 *>(x));
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}

extern "C" size_t pic_link_workspace_bytes(const int32_t *plan_host, int32_t head_dim) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || head_dim <= 0 || h[PIC_H_PAGED]) return 0;
  const size_t attn = (pic_attn_workspace_bytes(plan_host, head_dim) + 255) / 256 * 256;
  return attn + angle_table_bytes(h, head_dim);
}

extern "C" int pic_link(const int32_t *plan_host, const int32_t *plan_dev, int32_t n_layers,
                        void *x, const void *const *w_qkv, const void *const *w_o,
                        void *const *k_cache, void *const *v_cache, void *q, void *k_fresh,
                        void *v_fresh, void *o, int32_t dtype, int32_t d_model, int32_t head_dim,
                        int32_t rope_layout, double rope_base, float scale, void *workspace,
                        size_t workspace_bytes, void *stream) {
  using namespace pic;
  // every check of the per-layer calls, before anything is launched
  const PlanHeader h{plan_host};
  if (!h.valid() || h[PIC_H_PAGED] || n_layers < 0) return PIC_EINVAL;
  if (rope_layout != PIC_ROPE_ADJACENT && rope_layout != PIC_ROPE_HALF) return PIC_EINVAL;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return PIC_EINVAL;
  if (!resolve_scale(scale, head_dim)) return PIC_EINVAL;
  int st = check_gemm(h, dtype, d_model, head_dim);
  if (st != PIC_OK) return st;
  if (d_model % kGT || (h[PIC_H_H_Q] * head_dim) % kGT || (h[PIC_H_H_KV] * head_dim) % kGT ||
      (int64_t)kGT * h[PIC_H_H_Q] * head_dim * 2 > 0x7fff0000LL ||
      (int64_t)h[PIC_H_MAX_TOKENS] * h[PIC_H_H_KV] * head_dim * 2 > 0x7fff0000LL ||
      h[PIC_H_MAX_TOKENS] > (1 << 24))
    return PIC_EUNSUPPORTED;
  if (n_layers == 0) return PIC_OK;
  if (!w_qkv || !w_o || !k_cache || !v_cache) return PIC_EINVAL;
  for (int l = 0; l < n_layers; ++l)
    if (!w_qkv[l] || !w_o[l] || !k_cache[l] || !v_cache[l]) return PIC_EINVAL;
  if (!plan_dev) return PIC_EINVAL;
  if (h[PIC_H_N_ROWS] > 0 && (!x || !q || !k_fresh || !v_fresh || !o)) return PIC_EINVAL;
  const size_t need = pic_link_workspace_bytes(plan_host, head_dim);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PIC_ENOSPC;
  const size_t attn_ws = (pic_attn_workspace_bytes(plan_host, head_dim) + 255) / 256 * 256;
  char *ws = static_cast<char *>(workspace);
  for (int l = 0; l < n_layers && st == PIC_OK; ++l) {
    st = pic_qkv_rope(plan_host, plan_dev, x, w_qkv[l], q, k_fresh, v_fresh, dtype, d_model,
                      head_dim, rope_layout, rope_base, ws + attn_ws, workspace_bytes - attn_ws,
                      stream);
    if (st == PIC_OK)  // the layer's rotation and splice as one launch
      st = pic_rope_splice(plan_host, plan_dev, k_cache[l], v_cache[l], k_fresh, v_fresh, dtype,
                           head_dim, rope_layout, rope_base, PIC_ROPE_BY_DELTA, stream);
    if (st == PIC_OK)
      st = pic_selective_attn(plan_host, plan_dev, q, k_cache[l], v_cache[l], o, dtype, head_dim,
                              scale, attn_ws ? ws : nullptr, attn_ws, stream);
    if (st == PIC_OK) st = pic_out_proj(plan_host, o, w_o[l], x, dtype, d_model, head_dim, stream);
  }
  return st;
}
