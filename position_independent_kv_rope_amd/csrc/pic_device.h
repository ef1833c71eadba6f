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

}  // namespace pic
