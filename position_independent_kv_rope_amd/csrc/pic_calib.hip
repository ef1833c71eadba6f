// Calibration kernels for the measured peaks that bench.py reports beside the
// specification peaks: what a plain HBM stream and a plain MFMA loop reach on the GPU
// at hand.  They carry none of the splicing method and are built into their own
// library (libpic_calib.so); the C entry points are declared in include/pic_calib.h.
//
// - read: every 16-byte chunk of a buffer is loaded once (eight loads in flight per
//   thread) and folded into a per-wave XOR, so no load can be dropped;
// - copy: the same stream, each chunk stored to a second buffer;
// - update: each chunk written back complemented to where it was read (in place);
// - mfma: each wave runs four independent v_mfma_f32_32x32x16_bf16 chains on operands
//   read once from a buffer of random bf16 values (the operands differ from one MFMA to
//   the next, as real data does; constant operands let the chip clock higher than any
//   real workload), two waves per SIMD.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int kUnroll = 8;                    // 16-byte chunks in flight per thread
constexpr int64_t kMaxGrid = 256 * 16;        // stream workgroups (grid-stride beyond)
constexpr int kMfmaChains = 4;                // independent accumulators per wave

__global__ __launch_bounds__(kThreads) void calib_read_kernel(const u32x4 *__restrict__ p,
                                                              int64_t n16,
                                                              uint32_t *__restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      const int64_t i = base + (int64_t)q * kThreads;
      v[q] = i < n16 ? p[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) acc ^= v[q];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = x;
}

__global__ __launch_bounds__(kThreads) void calib_copy_kernel(const u32x4 *__restrict__ src,
                                                              u32x4 *__restrict__ dst,
                                                              int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      const int64_t i = base + (int64_t)q * kThreads;
      if (i < n16) v[q] = src[i];
    }
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      const int64_t i = base + (int64_t)q * kThreads;
      if (i < n16) dst[i] = v[q];
    }
  }
}

// In place: every chunk read and written back complemented, the access pattern of an
// in-place row rotation (reads and writes each byte once, at the same address).
__global__ __launch_bounds__(kThreads) void calib_update_kernel(u32x4 *__restrict__ p,
                                                                int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      const int64_t i = base + (int64_t)q * kThreads;
      if (i < n16) v[q] = p[i];
    }
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      const int64_t i = base + (int64_t)q * kThreads;
      if (i < n16) p[i] = ~v[q];
    }
  }
}

// operands: 2 * kMfmaChains * 64 bf16x8 values (A fragments, then B fragments); every
// wave reads the same ones.  sink: one float per thread of the grid.
__global__ __launch_bounds__(kThreads, 2) void calib_mfma_kernel(const bf16x8 *__restrict__ ops,
                                                                 float *__restrict__ sink,
                                                                 int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[kMfmaChains], b[kMfmaChains];
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) {
    a[c] = ops[c * 64 + lane];
    b[c] = ops[(kMfmaChains + c) * 64 + lane];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  }
  // rounds of kMfmaChains iterations, so every operand index is a constant
  for (int it = 0; it < iters; it += kMfmaChains) {
#pragma unroll
    for (int r = 0; r < kMfmaChains; ++r)
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[(c + r) % kMfmaChains],
                                                         acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

unsigned stream_grid(int64_t n16) {
  const int64_t per = (int64_t)kThreads * kUnroll;
  int64_t g = (n16 + per - 1) / per;
  if (g > kMaxGrid) g = kMaxGrid;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

extern "C" int64_t pic_calib_read_sink_words(int64_t bytes) {
  return bytes < 16 ? 0 : (int64_t)stream_grid(bytes / 16) * (kThreads / 64);
}

extern "C" int pic_calib_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0) return -1;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(calib_read_kernel, dim3(stream_grid(n16)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf), n16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int pic_calib_copy(const void *src, void *dst, int64_t bytes, void *stream) {
  if (!src || !dst || bytes < 16 || bytes % 16 != 0) return -1;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(calib_copy_kernel, dim3(stream_grid(n16)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src),
                     static_cast<u32x4 *>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int pic_calib_update(void *buf, int64_t bytes, void *stream) {
  if (!buf || bytes < 16 || bytes % 16 != 0) return -1;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(calib_update_kernel, dim3(stream_grid(n16)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4 *>(buf), n16);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int64_t pic_calib_mfma_flops(int32_t n_workgroups, int32_t iters) {
  return (int64_t)n_workgroups * (kThreads / 64) * iters * kMfmaChains * (2LL * 32 * 32 * 16);
}

extern "C" int pic_calib_mfma(const void *operands, float *sink, int32_t n_workgroups,
                              int32_t iters, void *stream) {
  if (!operands || !sink || n_workgroups <= 0 || iters <= 0 || iters % kMfmaChains != 0)
    return -1;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)n_workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const bf16x8 *>(operands),
                     sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
