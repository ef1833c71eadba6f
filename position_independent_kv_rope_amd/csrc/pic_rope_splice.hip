// Rotary correction of cached K (pic_rope_delta), RoPE of a position-free cache at the
// target positions (pic_rope_apply) and the row splice (pic_splice).
//
// Scheme B of the same article (section 3.2) caches K before RoPE and applies RoPE at
// the target positions on a hit; pic_rope_apply is that path, with one angle per
// (row, pair) instead of one per pair.
//
// Rotary correction follows the 10100.com article on RoPE and prefix caching, section
// 3.3 (scheme C): a cached K row carrying RoPE at position p is moved to p + delta by
// one rotation R(delta) of every dimension pair, using that rotations add up; the
// article notes that production code applies the delta rotation directly in one
// kernel instead of stacking two RoPE applications.  Section 2.2 and footnote 3 fix
// the pairs and frequencies theta_i = base^(-2i/D).
//
// Both kernels stream HBM: every element is read once and written once, with 16-byte
// coalesced accesses.  The rotation angle is constant per (chunk, pair), so each
// workgroup evaluates cos/sin of delta * theta_i once into LDS and then streams its
// tile of rows.  The angle is carried as a double-float in fp32: theta_i arrives from
// the host as an fp32 hi/lo pair of the fp64 value, the product delta * theta_hi is
// made exact with an FMA (its rounding error recovered as a second term), and the
// reduction modulo 2*pi uses a three-part Cody-Waite constant whose first product is
// exact, so the reduced angle is accurate to a few 1e-7 rad even at delta ~ 1e5.
#include <cmath>

#include "pic_device.h"
#include "pic_internal.h"

namespace pic {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeUnroll = 4;
// 8 consecutive elements <-> 8 floats.
__device__ __forceinline__ void load8(const __bf16 *p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
}
__device__ __forceinline__ void store8(__bf16 *p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (__bf16)x[j];
  *reinterpret_cast<bf16x8 *>(p) = v;
}
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a[j];
    x[4 + j] = b[j];
  }
}
__device__ __forceinline__ void store8(float *p, const float (&x)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = x[j];
    b[j] = x[4 + j];
  }
  *reinterpret_cast<f32x4 *>(p) = a;
  *reinterpret_cast<f32x4 *>(p + 4) = b;
}

// One workgroup per rope tile (<= PIC_ROPE_TILE_ROWS rows of one chunk).
// kAbs == false (rotation by delta): one angle delta * theta_i per pair for the whole
//   tile; tiles with delta 0 return at once.
// kAbs == true (RoPE at the target position): angle (pos0 + r) * theta_i for row r.
// The angles go to LDS (dynamic: n_pairs or n_rows * n_pairs float2) once per tile.
// kHalf == false: pairs (2i, 2i+1); a unit is 8 consecutive elements = 4 pairs.
// kHalf == true:  pairs (i, i+D/2); a unit is elements [8j, 8j+8) and [D/2+8j, D/2+8j+8).
template <typename T, bool kHalf, bool kAbs>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(
    T *__restrict__ k, const RopeTile *__restrict__ tiles, int h_kv, int head_dim,
    ThetaTable theta) {
  extern __shared__ float2 cs[];
  const RopeTile t = tiles[blockIdx.x];
  if (!kAbs && t.delta == 0) return;
  const int n_pairs = head_dim >> 1;
  if (kAbs) {
    for (int e = threadIdx.x; e < t.n_rows * n_pairs; e += kRopeThreads) {
      const int r = e / n_pairs, i = e - r * n_pairs;
      cs[e] = delta_cos_sin(t.pos0 + r, theta.hi[i], theta.lo[i]);
    }
  } else {
    for (int i = threadIdx.x; i < n_pairs; i += kRopeThreads)
      cs[i] = delta_cos_sin(t.delta, theta.hi[i], theta.lo[i]);
  }
  __syncthreads();

  const int units_per_head = kHalf ? (head_dim >> 4) : (head_dim >> 3);
  const int units_per_row = units_per_head * h_kv;
  const int total = t.n_rows * units_per_row;
  const int64_t row_elems = (int64_t)h_kv * head_dim;
  T *base = k + (int64_t)t.tok_begin * row_elems;

  for (int u0 = threadIdx.x; u0 < total; u0 += kRopeThreads * kRopeUnroll) {
    float a[kRopeUnroll][8], b[kRopeUnroll][8];
    T *pa[kRopeUnroll];
    int cso[kRopeUnroll];  // this unit's first angle in cs
    bool live[kRopeUnroll];
#pragma unroll
    for (int q = 0; q < kRopeUnroll; ++q) {
      const int u = u0 + q * kRopeThreads;
      live[q] = u < total;
      const int uu = live[q] ? u : 0;
      const int row = uu / units_per_row;
      const int rem = uu - row * units_per_row;
      const int head = rem / units_per_head;
      const int j = rem - head * units_per_head;
      cso[q] = (kAbs ? row * n_pairs : 0) + (kHalf ? 8 * j : 4 * j);
      pa[q] = base + row * row_elems + head * head_dim + 8 * j;
      if (live[q]) {
        load8(pa[q], a[q]);
        if (kHalf) load8(pa[q] + n_pairs, b[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < kRopeUnroll; ++q) {
      if (!live[q]) continue;
      if (kHalf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float2 c = cs[cso[q] + i];
          const float x0 = a[q][i], x1 = b[q][i];
          a[q][i] = x0 * c.x - x1 * c.y;
          b[q][i] = x0 * c.y + x1 * c.x;
        }
        store8(pa[q], a[q]);
        store8(pa[q] + n_pairs, b[q]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float2 c = cs[cso[q] + i];
          const float x0 = a[q][2 * i], x1 = a[q][2 * i + 1];
          a[q][2 * i] = x0 * c.x - x1 * c.y;
          a[q][2 * i + 1] = x0 * c.y + x1 * c.x;
        }
        store8(pa[q], a[q]);
      }
    }
  }
}

// Row scatter of the fresh K/V: 16-byte units, both buffers in one pass.
__global__ __launch_bounds__(256) void splice_kernel(u32x4 *__restrict__ k, u32x4 *__restrict__ v,
                                                     const u32x4 *__restrict__ kf,
                                                     const u32x4 *__restrict__ vf,
                                                     const int32_t *__restrict__ row_tok,
                                                     int64_t total, int units_per_row) {
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * 256) {
    const int64_t r = u / units_per_row;
    const int64_t c = u - r * units_per_row;
    const int64_t dst = (int64_t)row_tok[r] * units_per_row + c;
    const u32x4 a = kf[u];
    const u32x4 b = vf[u];
    k[dst] = a;
    v[dst] = b;
  }
}

template <typename T, bool kAbs>
int launch_rope(const PlanHeader &h, const int32_t *plan_dev, void *k, int head_dim, int layout,
                const ThetaTable &theta, hipStream_t s) {
  const RopeTile *tiles = reinterpret_cast<const RopeTile *>(plan_dev + h[PIC_H_O_ROPE_TILES]);
  const dim3 grid(h[PIC_H_N_ROPE_TILES]);
  const size_t lds = (kAbs ? PIC_ROPE_TILE_ROWS : 1) * (size_t)(head_dim / 2) * sizeof(float2);
  if (layout == PIC_ROPE_HALF)
    hipLaunchKernelGGL((rope_kernel<T, true, kAbs>), grid, dim3(kRopeThreads), lds, s,
                       static_cast<T *>(k), tiles, h[PIC_H_H_KV], head_dim, theta);
  else
    hipLaunchKernelGGL((rope_kernel<T, false, kAbs>), grid, dim3(kRopeThreads), lds, s,
                       static_cast<T *>(k), tiles, h[PIC_H_H_KV], head_dim, theta);
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}

// Shared argument checks and dispatch of pic_rope_delta / pic_rope_apply.
template <bool kAbs>
int rope_entry(const int32_t *plan_host, const int32_t *plan_dev, void *k, int32_t dtype,
               int32_t head_dim, int32_t rope_layout, double rope_base, void *stream) {
  const PlanHeader h{plan_host};
  if (!h.valid()) return PIC_EINVAL;
  if (dtype != PIC_BF16 && dtype != PIC_F32) return PIC_EINVAL;
  if (rope_layout != PIC_ROPE_ADJACENT && rope_layout != PIC_ROPE_HALF) return PIC_EINVAL;
  if (head_dim <= 0 || head_dim % 2 != 0 || !(rope_base > 0.0) || !std::isfinite(rope_base))
    return PIC_EINVAL;
  const int unit = rope_layout == PIC_ROPE_HALF ? 16 : 8;
  if (head_dim % unit != 0 || head_dim > 2 * kMaxPairs) return PIC_EUNSUPPORTED;
  if (h[PIC_H_N_ROPE_TILES] == 0) return PIC_OK;
  if (plan_dev == nullptr || k == nullptr) return PIC_EINVAL;
  if (kAbs) {  // positions are formed in fp32 exactly, which holds below 2^24
    const RopeTile *tl = reinterpret_cast<const RopeTile *>(plan_host + h[PIC_H_O_ROPE_TILES]);
    for (int32_t i = 0; i < h[PIC_H_N_ROPE_TILES]; ++i)
      if ((int64_t)tl[i].pos0 + tl[i].n_rows > (int64_t(1) << 24)) return PIC_EUNSUPPORTED;
  }

  const ThetaTable theta = make_theta(head_dim, rope_base);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PIC_BF16)
    return launch_rope<__bf16, kAbs>(h, plan_dev, k, head_dim, rope_layout, theta, s);
  return launch_rope<float, kAbs>(h, plan_dev, k, head_dim, rope_layout, theta, s);
}

}  // namespace
}  // namespace pic

extern "C" int pic_rope_delta(const int32_t *plan_host, const int32_t *plan_dev, void *k,
                              int32_t dtype, int32_t head_dim, int32_t rope_layout,
                              double rope_base, void *stream) {
  return pic::rope_entry<false>(plan_host, plan_dev, k, dtype, head_dim, rope_layout, rope_base,
                                stream);
}

extern "C" int pic_rope_apply(const int32_t *plan_host, const int32_t *plan_dev, void *k,
                              int32_t dtype, int32_t head_dim, int32_t rope_layout,
                              double rope_base, void *stream) {
  return pic::rope_entry<true>(plan_host, plan_dev, k, dtype, head_dim, rope_layout, rope_base,
                               stream);
}

extern "C" int pic_splice(const int32_t *plan_host, const int32_t *plan_dev, void *k, void *v,
                          const void *k_fresh, const void *v_fresh, int32_t dtype,
                          int32_t head_dim, void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid()) return PIC_EINVAL;
  const size_t es = dtype_size(dtype);
  if (es == 0 || head_dim <= 0) return PIC_EINVAL;
  if (head_dim % 8 != 0) return PIC_EUNSUPPORTED;
  const int64_t n_rows = h[PIC_H_N_ROWS];
  if (n_rows == 0) return PIC_OK;
  if (!plan_dev || !k || !v || !k_fresh || !v_fresh) return PIC_EINVAL;
  const int64_t row_bytes = (int64_t)h[PIC_H_H_KV] * head_dim * (int64_t)es;
  const int units_per_row = (int)(row_bytes / 16);
  const int64_t total = n_rows * units_per_row;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(splice_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4 *>(k),
                     static_cast<u32x4 *>(v), static_cast<const u32x4 *>(k_fresh),
                     static_cast<const u32x4 *>(v_fresh), plan_dev + h[PIC_H_O_ROW_TOK], total,
                     units_per_row);
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}
