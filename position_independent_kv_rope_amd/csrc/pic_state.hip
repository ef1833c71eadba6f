// Linear-layer state composition over the chunks of a request (pic_state_compose).
//
// HYPIC, section 2.1: a linear-attention head keeps one state matrix S [d_k, d_v]; a
// segment C is cached as its cumulative transition T_C (the product of its tokens'
// transitions) and its state from a zero start S(C|0), and after any prefix the state
// is S(prefix . C) = T_C S(prefix) + S(C|0).  For every request of a paged plan (the
// request's chunks name pool chunks) and every head this walks the chunks in prompt
// order: S_j = T_j S_{j-1} + S_j(0), writing the state after each chunk and the final
// state.
//
// One workgroup per (request, head), 8 waves.  S_{j-1} lives in LDS (it is the B
// operand every wave reads), the chunk's T [128 x 128] is staged to LDS through
// registers, and each wave computes a 32 x 64 block of S_j with v_mfma_f32_16x16x4_f32
// (fp32 operands and accumulation: the scan compounds rounding, so no bf16 here).  T rows
// have a stride of 132 floats, so the A reads (16 rows x 4 k) are conflict-free.  S is
// kept with its four 16-column blocks of each 64-column half interleaved, so a lane's B
// operands for the four column tiles of one k are one 16-byte read, and its four
// accumulator values of one row one 16-byte write (16 lanes cover 256 contiguous
// bytes).  While a chunk is multiplied, the next chunk's T and S(C|0) are already being
// loaded into registers.
#include <algorithm>

#include "pic_device.h"
#include "pic_internal.h"

namespace pic {
namespace {

constexpr int kSD = 128;                  // d_k = d_v
constexpr int kSThreads = 512;            // 8 waves: 4 row blocks x 2 column blocks
constexpr int kTStride = kSD + 4;         // floats per T row in LDS
constexpr int kTFloats = kSD * kSD / kSThreads;  // floats of T (and of S(C|0)) per thread

// S element (r, c) in LDS: column c = 64 h + 16 j + i (half h, block j, column i) sits at
// r * 128 + 4 (16 h + i) + j, so the four blocks' column i are adjacent.
__device__ __forceinline__ int sidx(int r, int c) {
  return r * kSD + 4 * (16 * (c >> 6) + (c & 15)) + ((c >> 4) & 3);
}

__global__ __launch_bounds__(kSThreads, 1) void state_compose_kernel(
    const int32_t *__restrict__ segs, const int32_t *__restrict__ req_chunk_ptr, int n_heads,
    const float *__restrict__ t_pool, const float *__restrict__ s_pool,
    const float *__restrict__ s_init, float *__restrict__ prefix_out,
    float *__restrict__ final_out) {
  __shared__ __attribute__((aligned(16))) float t_lds[kSD * kTStride];
  __shared__ __attribute__((aligned(16))) float s_lds[kSD * kSD];
  const int b = blockIdx.x / n_heads, h = blockIdx.x - b * n_heads;
  const int c0 = req_chunk_ptr[b], c1 = req_chunk_ptr[b + 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave & 3, wc = wave >> 2;  // rows 32 wr .., columns 64 wc ..
  const int col = lane & 15, quad = lane >> 4;
  const int64_t mat = (int64_t)kSD * kSD;

  // Matrix loads go through buffer resources: one per-lane offset and the element's
  // distance from it in the scalar offset, so the many loads in flight cost no address
  // registers.  (Every offset lies inside the 64 KiB matrix.)
  auto rsrc = [](const float *m) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)m, 0, kSD * kSD * 4, 0x00020000);
  };
  // this thread's share of a matrix load: kTFloats / 4 float4, rows tid / 32 + 16 r
  const int lrow = threadIdx.x >> 5, lcol = 4 * (threadIdx.x & 31);
  auto load_mat = [&](const float *m, f32x4 (&reg)[kTFloats / 4]) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(m);
    const int vo = (lrow * kSD + lcol) * 4;
#pragma unroll
    for (int r = 0; r < kTFloats / 4; ++r) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 16 * r * kSD * 4, 0);
      reg[r] = f32x4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                     __uint_as_float(v[3])};
    }
  };
  auto store_t = [&](const f32x4 (&reg)[kTFloats / 4]) {
#pragma unroll
    for (int r = 0; r < kTFloats / 4; ++r)
      *reinterpret_cast<f32x4 *>(t_lds + (lrow + 16 * r) * kTStride + lcol) = reg[r];
  };
  auto store_s = [&](const f32x4 (&reg)[kTFloats / 4]) {  // once per request
#pragma unroll
    for (int r = 0; r < kTFloats / 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) s_lds[sidx(lrow + 16 * r, lcol + j)] = reg[r][j];
  };
  // S(C|0) straight into the accumulator layout: tile (i, jt) of this wave covers rows
  // 32 wr + 16 i + 4 quad + e, column 64 wc + 16 jt + col
  auto load_acc = [&](const float *m, f32x4 (&a)[2][4]) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(m);
    const int vo = ((32 * wr + 4 * quad) * kSD + 64 * wc + col) * 4;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a[i][jt][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rs, vo, ((16 * i + e) * kSD + 16 * jt) * 4, 0));
  };
  auto store_acc = [&](float *m, const f32x4 (&a)[2][4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          m[(32 * wr + 16 * i + 4 * quad + e) * kSD + 64 * wc + 16 * jt + col] = a[i][jt][e];
  };
  auto chunk_mat = [&](const float *pool, int c) {
    return pool + ((int64_t)segs[8 * c + 3] * n_heads + h) * mat;
  };

  // S_{-1}: the initial state (zero when none is given)
  {
    f32x4 reg[kTFloats / 4];
    if (s_init) {
      load_mat(s_init + ((int64_t)b * n_heads + h) * mat, reg);
    } else {
#pragma unroll
      for (int r = 0; r < kTFloats / 4; ++r) reg[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    store_s(reg);
  }
  f32x4 acc[2][4];
  if (c0 == c1) {  // no chunks: the state stays the initial one
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[i][jt][e] = s_lds[sidx(32 * wr + 16 * i + 4 * quad + e, 64 * wc + 16 * jt + col)];
    store_acc(final_out + ((int64_t)b * n_heads + h) * mat, acc);
    return;
  }
  f32x4 treg[kTFloats / 4];
  f32x4 snext[2][4];
  load_mat(chunk_mat(t_pool, c0), treg);
  load_acc(chunk_mat(s_pool, c0), snext);
  store_t(treg);
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) acc[i][jt] = snext[i][jt];
    if (c + 1 < c1) {  // next chunk's operands, in flight during the products
      load_mat(chunk_mat(t_pool, c + 1), treg);
      load_acc(chunk_mat(s_pool, c + 1), snext);
    }
    // acc += T[32 wr .. +31][:] S[:][64 wc .. +63], 4 k per MFMA; one 16-byte read
    // gives row k + quad, column col of the four column tiles
    const float *ta = t_lds + (32 * wr + col) * kTStride + quad;
    const float *sb = s_lds + quad * kSD + 4 * (16 * wc + col);
    for (int k0 = 0; k0 < kSD; k0 += 16) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k = k0 + 4 * kk;
        const float a0 = ta[k], a1 = ta[16 * kTStride + k];
        const f32x4 bq = *reinterpret_cast<const f32x4 *>(sb + k * kSD);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          acc[0][jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, bq[jt], acc[0][jt], 0, 0, 0);
          acc[1][jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bq[jt], acc[1][jt], 0, 0, 0);
        }
      }
    }
    // every wave is done reading T_c and S_{c-1} (LDS only: the loads and stores in
    // flight keep going)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<f32x4 *>(s_lds + sidx(32 * wr + 16 * i + 4 * quad + e, 64 * wc + col)) =
            f32x4{acc[i][0][e], acc[i][1][e], acc[i][2][e], acc[i][3][e]};
    if (prefix_out) store_acc(prefix_out + ((int64_t)c * n_heads + h) * mat, acc);
    if (c + 1 < c1) store_t(treg);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // S_c and T_{c+1} in LDS
  }
  store_acc(final_out + ((int64_t)b * n_heads + h) * mat, acc);
}

}  // namespace
}  // namespace pic

extern "C" int pic_state_compose(const int32_t *plan_host, const int32_t *plan_dev,
                                 int32_t n_heads, int32_t d_k, int32_t d_v, const void *t_pool,
                                 const void *s_pool, int32_t n_pool_chunks, const void *s_init,
                                 void *prefix_out, void *final_out, int32_t dtype,
                                 void *stream) {
  using namespace pic;
  const PlanHeader h{plan_host};
  if (!h.valid() || !h[PIC_H_PAGED]) return PIC_EINVAL;
  if (n_heads <= 0 || d_k <= 0 || d_v <= 0 || n_pool_chunks < 0) return PIC_EINVAL;
  if (dtype != PIC_BF16 && dtype != PIC_F32) return PIC_EINVAL;
  if (dtype != PIC_F32 || d_k != kSD || d_v != kSD) return PIC_EUNSUPPORTED;
  if ((int64_t)h[PIC_H_N_REQ] * n_heads > 0x7fffffffLL) return PIC_EUNSUPPORTED;
  const int32_t *segs_h = plan_host + h[PIC_H_O_SEGS];
  for (int32_t c = 0; c < h[PIC_H_N_CHUNKS]; ++c)
    if (segs_h[8 * c + 3] >= n_pool_chunks) return PIC_EINVAL;
  if (h[PIC_H_N_REQ] == 0) return PIC_OK;
  if (!plan_dev || !final_out) return PIC_EINVAL;
  if (h[PIC_H_N_CHUNKS] > 0 && (!t_pool || !s_pool)) return PIC_EINVAL;
  hipLaunchKernelGGL(state_compose_kernel, dim3(h[PIC_H_N_REQ] * n_heads), dim3(kSThreads), 0,
                     static_cast<hipStream_t>(stream), plan_dev + h[PIC_H_O_SEGS],
                     plan_dev + h[PIC_H_O_REQ_CHUNK_PTR], n_heads,
                     static_cast<const float *>(t_pool), static_cast<const float *>(s_pool),
                     static_cast<const float *>(s_init), static_cast<float *>(prefix_out),
                     static_cast<float *>(final_out));
  PIC_LAUNCH_CHECK();
  return PIC_OK;
}
