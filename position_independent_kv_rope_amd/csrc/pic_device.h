// Device-side helpers shared by the kernels of libpic.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pic {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Launch checks: every entry point maps a failed launch to PIC_EDEVICE.
#define PIC_LAUNCH_CHECK()                                  \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return PIC_EDEVICE; \
  } while (0)

__device__ __forceinline__ float bf16_to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }  // RNE

// cos and sin of delta * theta for an integer delta (|delta| <= 2^24) and theta given as
// an fp32 hi/lo split of its fp64 value.  The angle is carried as a double-float: the
// product delta * theta_hi is made exact with an FMA (its rounding error recovered as a
// second term), and the reduction modulo 2*pi uses a three-part Cody-Waite constant
// whose first product is exact, so the reduced angle is accurate to a few 1e-7 rad even
// at delta ~ 1e5 (a plain fp32 product would be off by ~2e-3 rad there).
constexpr float kTwoPi1 = 6.2831854820251465f;  // 2*pi = kTwoPi1 + kTwoPi2 + kTwoPi3
constexpr float kTwoPi2 = -1.7484555314695172e-07f;
constexpr float kTwoPi3 = -6.8604980400235275e-15f;
constexpr float kInvTwoPi = 0.15915493667125702f;

__device__ __forceinline__ float2 delta_cos_sin(int delta, float th_hi, float th_lo) {
  const float d = (float)delta;
  const float p = d * th_hi;
  const float e = fmaf(d, th_hi, -p);    // exact rounding error of d * th_hi
  const float tail = fmaf(d, th_lo, e);  // small remainder of the angle
  const float n = rintf(p * kInvTwoPi);
  float r = fmaf(-n, kTwoPi1, p);        // exact
  r = fmaf(-n, kTwoPi2, r);
  r = r + fmaf(-n, kTwoPi3, tail);
  float s, c;
  sincosf(r, &s, &c);
  return make_float2(c, s);
}

constexpr int kMaxPairs = 128;  // head_dim <= 256

// theta_i = base^(-2i/D) as fp32 hi/lo pairs (filled on the host in fp64), passed by value.
struct ThetaTable {
  float hi[kMaxPairs];
  float lo[kMaxPairs];
};

// Host: theta_i = base^(-2i/D) in fp64, split into fp32 hi/lo pairs.
inline ThetaTable make_theta(int head_dim, double base) {
  ThetaTable t{};
  for (int i = 0; i < head_dim / 2 && i < kMaxPairs; ++i) {
    const double th = __builtin_pow(base, -2.0 * i / (double)head_dim);
    t.hi[i] = (float)th;
    t.lo[i] = (float)(th - (double)t.hi[i]);
  }
  return t;
}

}  // namespace pic
