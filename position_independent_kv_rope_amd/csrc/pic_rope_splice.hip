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
#include <type_traits>

#include "pic_device.h"
#include "pic_internal.h"

namespace pic {
namespace {

constexpr int kRopeThreads = 256;
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

// 8 consecutive elements of T as loaded (16 bytes of bf16, 32 bytes of fp32).
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;
template <typename T>
using Raw8 = typename std::conditional<sizeof(T) == 2, bf16x8, f32x8>::type;

// One rope tile (<= PIC_ROPE_TILE_ROWS rows of one chunk), run by one workgroup.
// kAbs == false (rotation by delta): one angle delta * theta_i per pair for the whole
//   tile (callers skip tiles with delta 0).
// kAbs == true (RoPE at the target position): angle (pos0 + r) * theta_i for row r.
// kHalf == false: pairs (2i, 2i+1); a unit is 8 consecutive elements = 4 pairs.
// kHalf == true:  pairs (i, i+D/2); a unit is elements [8j, 8j+8) and [D/2+8j, D/2+8j+8).
// Every thread first issues the loads of all its units of the round (up to 16 16-byte
// loads: a whole bf16 tile of 32 rows x 1024 elements is one round), then the angles
// are evaluated into LDS (cs: n_pairs or n_rows * n_pairs float2) while those loads
// are in flight; the barrier waits on the LDS writes only.  So every workgroup keeps its
// whole tile in flight at once, which matters when the launch is one wave of
// workgroups (a 32k-token request is ~1,000 tiles).
template <typename T, bool kHalf, bool kAbs>
__device__ __forceinline__ void rope_tile(T *__restrict__ k, const RopeTile &t, int h_kv,
                                          int head_dim, const ThetaTable &theta, float2 *cs,
                                          int head0, int n_heads) {
  constexpr int kLoadsPerUnit = (kHalf ? 2 : 1) * (int)sizeof(T) / 2;  // 16-byte loads
  constexpr int kU = 16 / kLoadsPerUnit;                                 // units per round
  const int n_pairs = head_dim >> 1;
  const int units_per_head = kHalf ? (head_dim >> 4) : (head_dim >> 3);
  const int units_per_row = units_per_head * n_heads;  // this workgroup's heads of a row
  const int total = t.n_rows * units_per_row;
  const int64_t row_elems = (int64_t)h_kv * head_dim;
  T *base = k + (int64_t)t.tok_begin * row_elems + (int64_t)head0 * head_dim;

  // a unit's place in the tile: element offset from base and first angle in cs
  auto place = [&](int u, int &off, int &cso) {
    const int row = u / units_per_row;
    const int rem = u - row * units_per_row;
    const int head = rem / units_per_head;
    const int j = rem - head * units_per_head;
    cso = (kAbs ? row * n_pairs : 0) + (kHalf ? 8 * j : 4 * j);
    off = row * (int)row_elems + head * head_dim + 8 * j;
  };
  // this thread's theta values, read before the tile's loads are issued (vector memory
  // completes in order: a wait for them must not wait for the tile)
  // (unconditional loads, clamped indices: no branch splits the loads into blocks, so
  // the wait for theta below counts only the two theta loads)
  // Rotation by delta: thread i < n_pairs evaluates pair i.  RoPE at the position: entry
  // e = tid + 256 m is pair e % n_pairs, which is tid % n_pairs when n_pairs divides 256.
  const bool pair_fixed = kRopeThreads % n_pairs == 0;
  const int ti = kAbs && pair_fixed ? (int)threadIdx.x % n_pairs : min((int)threadIdx.x, n_pairs - 1);
  float th_hi = theta.hi[ti], th_lo = theta.lo[ti];
  asm volatile("" ::: "memory");  // theta loads issued before the tile's loads
  // one round: this thread's kU units starting at u0 (the first round also evaluates the
  // angles while its loads are in flight)
  auto round_at = [&](int u0, bool first) {
    Raw8<T> ra[kU], rb[kU];  // raw 8-element vectors: converted only when rotated
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int u = min(u0 + q * kRopeThreads, total - 1);  // past the tile: reload its last unit
      int off, cso;
      place(u, off, cso);
      ra[q] = *reinterpret_cast<const Raw8<T> *>(base + off);
      if (kHalf) rb[q] = *reinterpret_cast<const Raw8<T> *>(base + off + n_pairs);
    }
    // every load is issued before the angle math (which waits for theta only)
    asm volatile("" : "+v"(th_hi), "+v"(th_lo) : : "memory");
    if (first) {
      if (kAbs && pair_fixed) {
        for (int e = threadIdx.x; e < t.n_rows * n_pairs; e += kRopeThreads)
          cs[e] = delta_cos_sin(t.pos0 + e / n_pairs, th_hi, th_lo);
      } else if (kAbs) {
        for (int e = threadIdx.x; e < t.n_rows * n_pairs; e += kRopeThreads) {
          const int r = e / n_pairs, i = e - r * n_pairs;
          cs[e] = delta_cos_sin(t.pos0 + r, theta.hi[i], theta.lo[i]);
        }
      } else if ((int)threadIdx.x < n_pairs) {
        cs[threadIdx.x] = delta_cos_sin(t.delta, th_hi, th_lo);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this thread's LDS writes done
      __builtin_amdgcn_s_barrier();         // (the tile's loads stay in flight)
    }
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int u = u0 + q * kRopeThreads;
      if (u >= total) continue;
      int off, cso;
      place(u, off, cso);
      T *pa = base + off;
      float a[8], b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = (float)ra[q][j];
      if (kHalf) {
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = (float)rb[q][j];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float2 c = cs[cso + i];
          const float x0 = a[i], x1 = b[i];
          a[i] = x0 * c.x - x1 * c.y;
          b[i] = x0 * c.y + x1 * c.x;
        }
        store8(pa, a);
        store8(pa + n_pairs, b);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float2 c = cs[cso + i];
          const float x0 = a[2 * i], x1 = a[2 * i + 1];
          a[2 * i] = x0 * c.x - x1 * c.y;
          a[2 * i + 1] = x0 * c.y + x1 * c.x;
        }
        store8(pa, a);
      }
    }
  };
  round_at(threadIdx.x, true);  // a bf16 tile of <= 32 rows is this one round
  for (int u0 = threadIdx.x + kRopeThreads * kU; u0 < total; u0 += kRopeThreads * kU)
    round_at(u0, false);
}

template <typename T, bool kHalf, bool kAbs>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(
    T *__restrict__ k, const RopeTile *__restrict__ tiles, int h_kv, int head_dim, int split,
    ThetaTable theta) {
  extern __shared__ float2 cs[];
  const int tile = blockIdx.x / split, part = blockIdx.x - tile * split;
  const RopeTile t = tiles[tile];
  if (!kAbs && t.delta == 0) return;
  const int hp = h_kv / split;
  rope_tile<T, kHalf, kAbs>(k, t, h_kv, head_dim, theta, cs, part * hp, hp);
}

// Row scatter of the fresh K/V in 16-byte units, both buffers in one pass: one
// workgroup copies the kSpliceUnroll * 256 consecutive units starting at u0 (unit u is
// chunk u % units_per_row of fresh row u / units_per_row), all loads before the stores.
constexpr int kSpliceThreads = 256;
constexpr int kSpliceUnroll = 4;
constexpr int64_t kSpliceBlockUnits = kSpliceThreads * kSpliceUnroll;
__device__ __forceinline__ void splice_block(u32x4 *__restrict__ k, u32x4 *__restrict__ v,
                                             const u32x4 *__restrict__ kf,
                                             const u32x4 *__restrict__ vf,
                                             const int32_t *__restrict__ row_tok, int64_t u0,
                                             int64_t total, int units_per_row) {
  u32x4 a[kSpliceUnroll], b[kSpliceUnroll];
  int64_t dst[kSpliceUnroll];
#pragma unroll
  for (int q = 0; q < kSpliceUnroll; ++q) {
    const int64_t u = u0 + q * kSpliceThreads + threadIdx.x;
    dst[q] = -1;
    if (u < total) {
      const int64_t r = u / units_per_row;
      dst[q] = (int64_t)row_tok[r] * units_per_row + (u - r * units_per_row);
      a[q] = kf[u];
      b[q] = vf[u];
    }
  }
#pragma unroll
  for (int q = 0; q < kSpliceUnroll; ++q)
    if (dst[q] >= 0) {
      k[dst[q]] = a[q];
      v[dst[q]] = b[q];
    }
}

__global__ __launch_bounds__(kSpliceThreads) void splice_kernel(
    u32x4 *__restrict__ k, u32x4 *__restrict__ v, const u32x4 *__restrict__ kf,
    const u32x4 *__restrict__ vf, const int32_t *__restrict__ row_tok, int64_t total,
    int units_per_row) {
  for (int64_t u0 = (int64_t)blockIdx.x * kSpliceBlockUnits; u0 < total;
       u0 += (int64_t)gridDim.x * kSpliceBlockUnits)
    splice_block(k, v, kf, vf, row_tok, u0, total, units_per_row);
}

// Rotation and splice in one launch.  The rotation never touches a recomputed row
// (rope tiles start after each chunk's recomputed head, and query rows belong to no
// chunk), so the two parts write disjoint rows and need no ordering: workgroups
// [0, n_splice) copy fresh rows, the rest take one rope tile each.
template <typename T, bool kHalf, bool kAbs>
__global__ __launch_bounds__(kRopeThreads) void rope_splice_kernel(
    T *__restrict__ k, T *__restrict__ v, const u32x4 *__restrict__ kf,
    const u32x4 *__restrict__ vf, const int32_t *__restrict__ row_tok, int64_t total,
    int units_per_row, int n_splice, const RopeTile *__restrict__ tiles, int h_kv,
    int head_dim, int split, ThetaTable theta) {
  static_assert(kRopeThreads == kSpliceThreads, "one workgroup size for both parts");
  extern __shared__ float2 cs[];
  if ((int)blockIdx.x < n_splice) {
    splice_block(reinterpret_cast<u32x4 *>(k), reinterpret_cast<u32x4 *>(v), kf, vf, row_tok,
                 (int64_t)blockIdx.x * kSpliceBlockUnits, total, units_per_row);
    return;
  }
  const int idx = (int)blockIdx.x - n_splice;
  const int tile = idx / split, part = idx - tile * split;
  const RopeTile t = tiles[tile];
  if (!kAbs && t.delta == 0) return;
  const int hp = h_kv / split;
  rope_tile<T, kHalf, kAbs>(k, t, h_kv, head_dim, theta, cs, part * hp, hp);
}

// Workgroups per rope tile.  Large launches share a tile's KV heads out over `split`
// workgroups (a power of two dividing h_kv) until the launch holds kRopeSplitBlocks of
// them: more, shorter workgroups keep the HBM stream busier towards the end of the
// launch (4 x 50k tokens, 6,135 tiles: 131 -> 125 us).  Launches of fewer than
// kRopeSplitFrom tiles keep one workgroup per tile: there every extra workgroup costs
// more in dispatch than it returns (32k tokens, 992 tiles: 28 us whole, 29/38/60 us in
// halves/quarters/eighths).
constexpr int64_t kRopeSplitFrom = 2048;
constexpr int64_t kRopeSplitBlocks = 8192;
int rope_split(int n_tiles, int h_kv, bool absolute) {
  int split = 1;
  // RoPE at the target position builds a per-row angle table for the whole tile, which
  // every workgroup of a split tile would build again: those tiles stay whole
  if (absolute || n_tiles < kRopeSplitFrom) return split;
  while (2 * split <= h_kv && h_kv % (2 * split) == 0 &&
         (int64_t)n_tiles * split < kRopeSplitBlocks)
    split *= 2;
  return split;
}

template <typename T, bool kAbs>
int launch_rope(const PlanHeader &h, const int32_t *plan_dev, void *k, int head_dim, int layout,
                const ThetaTable &theta, hipStream_t s) {
  const RopeTile *tiles = reinterpret_cast<const RopeTile *>(plan_dev + h[PIC_H_O_ROPE_TILES]);
  const int split = rope_split(h[PIC_H_N_ROPE_TILES], h[PIC_H_H_KV], kAbs);
  const dim3 grid(h[PIC_H_N_ROPE_TILES] * split);
  const size_t lds = (kAbs ? PIC_ROPE_TILE_ROWS : 1) * (size_t)(head_dim / 2) * sizeof(float2);
  if (layout == PIC_ROPE_HALF)
    hipLaunchKernelGGL((rope_kernel<T, true, kAbs>), grid, dim3(kRopeThreads), lds, s,
                       static_cast<T *>(k), tiles, h[PIC_H_H_KV], head_dim, split, theta);
  else
    hipLaunchKernelGGL((rope_kernel<T, false, kAbs>), grid, dim3(kRopeThreads), lds, s,
                       static_cast<T *>(k), tiles, h[PIC_H_H_KV], head_dim, split, theta);
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}

// Argument checks shared by pic_rope_delta / pic_rope_apply / pic_rope_splice; PIC_OK
// means the rotation may be launched (or has nothing to do when the plan has no tile).
template <bool kAbs>
int rope_check(const PlanHeader &h, const int32_t *plan_dev, const void *k, int32_t dtype,
               int32_t head_dim, int32_t rope_layout, double rope_base) {
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
    const int32_t *plan_host = h.w;
    const RopeTile *tl = reinterpret_cast<const RopeTile *>(plan_host + h[PIC_H_O_ROPE_TILES]);
    for (int32_t i = 0; i < h[PIC_H_N_ROPE_TILES]; ++i)
      if ((int64_t)tl[i].pos0 + tl[i].n_rows > (int64_t(1) << 24)) return PIC_EUNSUPPORTED;
  }
  return PIC_OK;
}

template <bool kAbs>
int rope_entry(const int32_t *plan_host, const int32_t *plan_dev, void *k, int32_t dtype,
               int32_t head_dim, int32_t rope_layout, double rope_base, void *stream) {
  const PlanHeader h{plan_host};
  const int st = rope_check<kAbs>(h, plan_dev, k, dtype, head_dim, rope_layout, rope_base);
  if (st != PIC_OK || h[PIC_H_N_ROPE_TILES] == 0) return st;
  const ThetaTable theta = make_theta(head_dim, rope_base);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PIC_BF16)
    return launch_rope<__bf16, kAbs>(h, plan_dev, k, head_dim, rope_layout, theta, s);
  return launch_rope<float, kAbs>(h, plan_dev, k, head_dim, rope_layout, theta, s);
}

// Argument checks of pic_splice; *total / *units_per_row describe the copy.
int splice_check(const PlanHeader &h, const int32_t *plan_dev, const void *k, const void *v,
                 const void *k_fresh, const void *v_fresh, int32_t dtype, int32_t head_dim,
                 int64_t *total, int *units_per_row) {
  *total = 0;
  if (!h.valid()) return PIC_EINVAL;
  const size_t es = dtype_size(dtype);
  if (es == 0 || head_dim <= 0) return PIC_EINVAL;
  if (head_dim % 8 != 0) return PIC_EUNSUPPORTED;
  const int64_t n_rows = h[PIC_H_N_ROWS];
  if (n_rows == 0) return PIC_OK;
  if (!plan_dev || !k || !v || !k_fresh || !v_fresh) return PIC_EINVAL;
  const int64_t row_bytes = (int64_t)h[PIC_H_H_KV] * head_dim * (int64_t)es;
  *units_per_row = (int)(row_bytes / 16);
  *total = n_rows * *units_per_row;
  return PIC_OK;
}

int launch_splice(const PlanHeader &h, const int32_t *plan_dev, void *k, void *v,
                  const void *k_fresh, const void *v_fresh, int64_t total, int units_per_row,
                  hipStream_t s) {
  const int64_t blocks =
      std::min<int64_t>((total + kSpliceBlockUnits - 1) / kSpliceBlockUnits, 8192);
  hipLaunchKernelGGL(splice_kernel, dim3((unsigned)blocks), dim3(kSpliceThreads), 0, s,
                     static_cast<u32x4 *>(k), static_cast<u32x4 *>(v),
                     static_cast<const u32x4 *>(k_fresh), static_cast<const u32x4 *>(v_fresh),
                     plan_dev + h[PIC_H_O_ROW_TOK], total, units_per_row);
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}

// Grid limit of the single launch (rope tiles + splice workgroups); larger plans run
// the two parts as two launches on the same stream.
constexpr int64_t kMaxFusedBlocks = int64_t(1) << 22;

// ---- rotation + splice from a shared paged pool into contiguous spliced buffers ----
//
// The shared-pool counterpart of the one-launch rotation + splice: the pool (chunks
// stored once, RoPE at local positions, [blocks][16][h_kv][D]) is only read; each
// request's spliced K/V are written to contiguous caller buffers [n_tokens][h_kv][D]:
// kept row t of request chunk c becomes R(delta_c) K_pool[t] (V copied), and every
// recomputed row its fresh K/V.  A paged plan's key-block records give the work: one
// workgroup per 64-row pool block of a request chunk (rows past the chunk's seam), the
// first workgroups copying the fresh rows.  Pool blocks that the chunk's block-table
// row does not list, or ids outside the pool, give zero rows.
constexpr int kPoolBlockRows = 16;
constexpr int kKeyBlockRows = 64;

template <typename T, bool kHalf>
__device__ __forceinline__ void pool_block(T *__restrict__ k, T *__restrict__ v,
                                           const T *__restrict__ pool_k,
                                           const T *__restrict__ pool_v, int c, int t0,
                                           const int32_t *__restrict__ segs,
                                           const int32_t *__restrict__ chunk_block_ptr,
                                           const int32_t *__restrict__ block_ids,
                                           const int32_t *__restrict__ req_tok_ptr, int h_kv,
                                           int head_dim, int64_t pool_blocks,
                                           const ThetaTable &theta, float2 *cs, int *bid_s) {
  constexpr int kLoadsPerUnit = (kHalf ? 2 : 1) * (int)sizeof(T) / 2;  // 16-byte loads
  constexpr int kU = 8 / kLoadsPerUnit;  // units of K (and of V) per thread per round
  const int32_t *sg = segs + 8 * c;
  const int off = sg[0], len = sg[1], seam = sg[2], pid = sg[3], delta = sg[4], req = sg[5];
  const int t_lo = max(t0, seam), t_hi = min(t0 + kKeyBlockRows, len);
  const int n_pairs = head_dim >> 1;
  if ((int)threadIdx.x < kKeyBlockRows / kPoolBlockRows) {
    const int tab0 = chunk_block_ptr[pid];
    const int ntab = max(0, chunk_block_ptr[pid + 1] - tab0);
    const int pb = t0 / kPoolBlockRows + (int)threadIdx.x;
    const int bid = pb < ntab ? block_ids[tab0 + pb] : -1;
    bid_s[threadIdx.x] = bid >= 0 && bid < pool_blocks ? bid : -1;
  }
  for (int i = threadIdx.x; i < n_pairs; i += kRopeThreads)
    cs[i] = delta_cos_sin(delta, theta.hi[i], theta.lo[i]);
  __syncthreads();
  if (t_lo >= t_hi) return;

  const int units_per_head = kHalf ? (head_dim >> 4) : (head_dim >> 3);
  const int units_per_row = units_per_head * h_kv;
  const int total = (t_hi - t_lo) * units_per_row;
  const int64_t row_elems = (int64_t)h_kv * head_dim;
  const int64_t dst0 = (int64_t)req_tok_ptr[req] + off;  // K/V row of local key 0
  // a unit's source (pool) and destination element offsets; src < 0: a zero row
  auto place = [&](int u, int64_t &src, int64_t &dst, int &cso) {
    const int i = u / units_per_row;
    const int rem = u - i * units_per_row;
    const int head = rem / units_per_head;
    const int j = rem - head * units_per_head;
    const int t = t_lo + i;
    const int bid = bid_s[(t - t0) / kPoolBlockRows];
    const int64_t in_row = (int64_t)head * head_dim + 8 * j;
    src = bid < 0 ? -1 : ((int64_t)bid * kPoolBlockRows + t % kPoolBlockRows) * row_elems + in_row;
    dst = (dst0 + t) * row_elems + in_row;
    cso = kHalf ? 8 * j : 4 * j;
  };
  for (int u0 = threadIdx.x; u0 < total; u0 += kRopeThreads * kU) {
    Raw8<T> ka[kU], kb[kU], va[kU], vb[kU];
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int u = min(u0 + q * kRopeThreads, total - 1);
      int64_t src, dst;
      int cso;
      place(u, src, dst, cso);
      ka[q] = va[q] = kb[q] = vb[q] = Raw8<T>{};
      if (src >= 0) {  // zero rows (unlisted or out-of-pool blocks) load nothing
        ka[q] = *reinterpret_cast<const Raw8<T> *>(pool_k + src);
        va[q] = *reinterpret_cast<const Raw8<T> *>(pool_v + src);
        if (kHalf) {
          kb[q] = *reinterpret_cast<const Raw8<T> *>(pool_k + src + n_pairs);
          vb[q] = *reinterpret_cast<const Raw8<T> *>(pool_v + src + n_pairs);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int u = u0 + q * kRopeThreads;
      if (u >= total) continue;
      int64_t src, dst;
      int cso;
      place(u, src, dst, cso);
      float a[8], b[8], x[8], y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = src < 0 ? 0.f : (float)ka[q][e];
        x[e] = src < 0 ? 0.f : (float)va[q][e];
        if (kHalf) {
          b[e] = src < 0 ? 0.f : (float)kb[q][e];
          y[e] = src < 0 ? 0.f : (float)vb[q][e];
        }
      }
      if (kHalf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float2 cz = cs[cso + i];
          const float x0 = a[i], x1 = b[i];
          a[i] = x0 * cz.x - x1 * cz.y;
          b[i] = x0 * cz.y + x1 * cz.x;
        }
        store8(k + dst, a);
        store8(k + dst + n_pairs, b);
        store8(v + dst, x);
        store8(v + dst + n_pairs, y);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float2 cz = cs[cso + i];
          const float x0 = a[2 * i], x1 = a[2 * i + 1];
          a[2 * i] = x0 * cz.x - x1 * cz.y;
          a[2 * i + 1] = x0 * cz.y + x1 * cz.x;
        }
        store8(k + dst, a);
        store8(v + dst, x);
      }
    }
  }
}

template <typename T, bool kHalf>
__global__ __launch_bounds__(kRopeThreads) void pool_rope_splice_kernel(
    T *__restrict__ k, T *__restrict__ v, const T *__restrict__ pool_k,
    const T *__restrict__ pool_v, const u32x4 *__restrict__ kf, const u32x4 *__restrict__ vf,
    const int32_t *__restrict__ row_tok, int64_t total, int units_per_row, int n_splice,
    const int4 *__restrict__ kblocks, const int32_t *__restrict__ segs,
    const int32_t *__restrict__ chunk_block_ptr, const int32_t *__restrict__ block_ids,
    const int32_t *__restrict__ req_tok_ptr, int h_kv, int head_dim, int64_t pool_blocks,
    ThetaTable theta) {
  static_assert(kRopeThreads == kSpliceThreads, "one workgroup size for both parts");
  extern __shared__ float2 cs[];
  __shared__ int bid_s[kKeyBlockRows / kPoolBlockRows];
  if ((int)blockIdx.x < n_splice) {
    splice_block(reinterpret_cast<u32x4 *>(k), reinterpret_cast<u32x4 *>(v), kf, vf, row_tok,
                 (int64_t)blockIdx.x * kSpliceBlockUnits, total, units_per_row);
    return;
  }
  const int4 kb = kblocks[blockIdx.x - n_splice];
  if (kb.x < 0) return;  // a block of fresh rows: copied by the splice workgroups
  pool_block<T, kHalf>(k, v, pool_k, pool_v, kb.x, kb.y, segs, chunk_block_ptr, block_ids,
                       req_tok_ptr, h_kv, head_dim, pool_blocks, theta, cs, bid_s);
}

template <typename T, bool kHalf>
int launch_pool_rope_splice(const PlanHeader &h, const int32_t *plan_dev, void *k, void *v,
                            const void *pool_k, const void *pool_v, int64_t pool_blocks,
                            const int32_t *cbp, const int32_t *bids, const void *k_fresh,
                            const void *v_fresh, int64_t total, int units_per_row, int head_dim,
                            const ThetaTable &theta, hipStream_t s) {
  const int64_t n_splice = (total + kSpliceBlockUnits - 1) / kSpliceBlockUnits;
  const int64_t n_kb = h[PIC_H_N_KBLOCKS];
  if (n_splice + n_kb > kMaxFusedBlocks) return PIC_EUNSUPPORTED;
  if (n_splice + n_kb == 0) return PIC_OK;
  const size_t lds = (size_t)(head_dim / 2) * sizeof(float2);
  hipLaunchKernelGGL((pool_rope_splice_kernel<T, kHalf>), dim3((unsigned)(n_splice + n_kb)),
                     dim3(kRopeThreads), lds, s, static_cast<T *>(k), static_cast<T *>(v),
                     static_cast<const T *>(pool_k), static_cast<const T *>(pool_v),
                     static_cast<const u32x4 *>(k_fresh), static_cast<const u32x4 *>(v_fresh),
                     plan_dev + h[PIC_H_O_ROW_TOK], total, units_per_row, (int)n_splice,
                     reinterpret_cast<const int4 *>(plan_dev + h[PIC_H_O_KBLOCKS]),
                     plan_dev + h[PIC_H_O_SEGS], cbp, bids, plan_dev + h[PIC_H_O_REQ_TOK_PTR],
                     h[PIC_H_H_KV], head_dim, pool_blocks, theta);
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}

template <typename T, bool kAbs>
int launch_rope_splice(const PlanHeader &h, const int32_t *plan_dev, void *k, void *v,
                       const void *k_fresh, const void *v_fresh, int64_t total,
                       int units_per_row, int head_dim, int layout, const ThetaTable &theta,
                       hipStream_t s) {
  const int n_tiles = h[PIC_H_N_ROPE_TILES];
  const int split = rope_split(n_tiles, h[PIC_H_H_KV], kAbs);
  const int64_t n_splice = (total + kSpliceBlockUnits - 1) / kSpliceBlockUnits;
  if (n_splice + (int64_t)n_tiles * split > kMaxFusedBlocks) {
    if (n_tiles > 0) {
      const int st = launch_rope<T, kAbs>(h, plan_dev, k, head_dim, layout, theta, s);
      if (st != PIC_OK) return st;
    }
    return total > 0 ? launch_splice(h, plan_dev, k, v, k_fresh, v_fresh, total, units_per_row, s)
                     : PIC_OK;
  }
  const RopeTile *tiles = reinterpret_cast<const RopeTile *>(plan_dev + h[PIC_H_O_ROPE_TILES]);
  const dim3 grid((unsigned)(n_splice + (int64_t)n_tiles * split));
  const size_t lds = (kAbs ? PIC_ROPE_TILE_ROWS : 1) * (size_t)(head_dim / 2) * sizeof(float2);
  const int32_t *row_tok = plan_dev + h[PIC_H_O_ROW_TOK];
  if (layout == PIC_ROPE_HALF)
    hipLaunchKernelGGL((rope_splice_kernel<T, true, kAbs>), grid, dim3(kRopeThreads), lds, s,
                       static_cast<T *>(k), static_cast<T *>(v),
                       static_cast<const u32x4 *>(k_fresh), static_cast<const u32x4 *>(v_fresh),
                       row_tok, total, units_per_row, (int)n_splice, tiles, h[PIC_H_H_KV],
                       head_dim, split, theta);
  else
    hipLaunchKernelGGL((rope_splice_kernel<T, false, kAbs>), grid, dim3(kRopeThreads), lds, s,
                       static_cast<T *>(k), static_cast<T *>(v),
                       static_cast<const u32x4 *>(k_fresh), static_cast<const u32x4 *>(v_fresh),
                       row_tok, total, units_per_row, (int)n_splice, tiles, h[PIC_H_H_KV],
                       head_dim, split, theta);
  PIC_LAUNCH_CHECK();
  return PIC_OK;
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
  int64_t total;
  int units_per_row;
  const int st = splice_check(h, plan_dev, k, v, k_fresh, v_fresh, dtype, head_dim, &total,
                              &units_per_row);
  if (st != PIC_OK || total == 0) return st;
  return launch_splice(h, plan_dev, k, v, k_fresh, v_fresh, total, units_per_row,
                       static_cast<hipStream_t>(stream));
}

extern "C" int pic_rope_splice(const int32_t *plan_host, const int32_t *plan_dev, void *k,
                               void *v, const void *k_fresh, const void *v_fresh, int32_t dtype,
                               int32_t head_dim, int32_t rope_layout, double rope_base,
                               int32_t rope_mode, void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (rope_mode != PIC_ROPE_BY_DELTA && rope_mode != PIC_ROPE_AT_POSITION) return PIC_EINVAL;
  const bool abs = rope_mode == PIC_ROPE_AT_POSITION;
  int st = abs ? rope_check<true>(h, plan_dev, k, dtype, head_dim, rope_layout, rope_base)
               : rope_check<false>(h, plan_dev, k, dtype, head_dim, rope_layout, rope_base);
  if (st != PIC_OK) return st;
  int64_t total;
  int units_per_row = 0;
  st = splice_check(h, plan_dev, k, v, k_fresh, v_fresh, dtype, head_dim, &total,
                    &units_per_row);
  if (st != PIC_OK) return st;
  if (total == 0 && h[PIC_H_N_ROPE_TILES] == 0) return PIC_OK;
  const ThetaTable theta = make_theta(head_dim, rope_base);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PIC_BF16)
    return abs ? launch_rope_splice<__bf16, true>(h, plan_dev, k, v, k_fresh, v_fresh, total,
                                                  units_per_row, head_dim, rope_layout, theta, s)
               : launch_rope_splice<__bf16, false>(h, plan_dev, k, v, k_fresh, v_fresh, total,
                                                   units_per_row, head_dim, rope_layout, theta,
                                                   s);
  return abs ? launch_rope_splice<float, true>(h, plan_dev, k, v, k_fresh, v_fresh, total,
                                               units_per_row, head_dim, rope_layout, theta, s)
             : launch_rope_splice<float, false>(h, plan_dev, k, v, k_fresh, v_fresh, total,
                                                units_per_row, head_dim, rope_layout, theta, s);
}

extern "C" int pic_rope_splice_pool(const int32_t *plan_host, const int32_t *plan_dev,
                                    const void *pool_k, const void *pool_v, int64_t pool_blocks,
                                    int32_t block_size, const int32_t *chunk_block_ptr,
                                    int32_t n_pool_chunks, const int32_t *block_ids, void *k,
                                    void *v, const void *k_fresh, const void *v_fresh,
                                    int32_t dtype, int32_t head_dim, int32_t rope_layout,
                                    double rope_base, void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || !h[PIC_H_PAGED]) return PIC_EINVAL;
  if (dtype != PIC_BF16 && dtype != PIC_F32) return PIC_EINVAL;
  if (rope_layout != PIC_ROPE_ADJACENT && rope_layout != PIC_ROPE_HALF) return PIC_EINVAL;
  if (head_dim <= 0 || head_dim % 2 != 0 || !(rope_base > 0.0) || !std::isfinite(rope_base) ||
      pool_blocks < 0)
    return PIC_EINVAL;
  const int unit = rope_layout == PIC_ROPE_HALF ? 16 : 8;
  if (block_size != kPoolBlockRows || head_dim % unit != 0 || head_dim > 2 * kMaxPairs)
    return PIC_EUNSUPPORTED;
  const int32_t *segs_h = plan_host + h[PIC_H_O_SEGS];
  for (int32_t c = 0; c < h[PIC_H_N_CHUNKS]; ++c)
    if (segs_h[8 * c + 3] >= n_pool_chunks) return PIC_EINVAL;
  if (h[PIC_H_N_TOKENS] == 0) return PIC_OK;
  if (!plan_dev || !k || !v) return PIC_EINVAL;
  if (h[PIC_H_N_CHUNKS] > 0 && (!pool_k || !pool_v || !chunk_block_ptr || !block_ids))
    return PIC_EINVAL;
  if (h[PIC_H_N_ROWS] > 0 && (!k_fresh || !v_fresh)) return PIC_EINVAL;
  const int64_t row_bytes = (int64_t)h[PIC_H_H_KV] * head_dim * (int64_t)dtype_size(dtype);
  const int units_per_row = (int)(row_bytes / 16);
  const int64_t total = (int64_t)h[PIC_H_N_ROWS] * units_per_row;
  const ThetaTable theta = make_theta(head_dim, rope_base);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool half = rope_layout == PIC_ROPE_HALF;
#define PIC_POOL(T_, H_)                                                                   \
  return launch_pool_rope_splice<T_, H_>(h, plan_dev, k, v, pool_k, pool_v, pool_blocks,   \
                                         chunk_block_ptr, block_ids, k_fresh, v_fresh, total, \
                                         units_per_row, head_dim, theta, s)
  if (dtype == PIC_BF16) {
    if (half) PIC_POOL(__bf16, true);
    PIC_POOL(__bf16, false);
  }
  if (half) PIC_POOL(float, true);
  PIC_POOL(float, false);
#undef PIC_POOL
}
