/* Calibration kernels (libpic_calib.so): what a plain HBM stream and a plain MFMA loop
 * reach on the GPU at hand, so measured rates can be set beside the specification
 * peaks.  They are measurement infrastructure, not part of the splicing path in pic.h.
 *
 * All pointers are device pointers; every launch is asynchronous on `stream` (a
 * hipStream_t, NULL for the default stream).  Return 0 on success, -1 for an invalid
 * argument (nothing launched), -4 when the launch failed.  The caller owns every buffer.
 */
#ifndef PIC_CALIB_H
#define PIC_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of uint32 words pic_calib_read writes to `sink` for a buffer of `bytes`. */
int64_t pic_calib_read_sink_words(int64_t bytes);

/* Read every byte of buf[0, bytes) once (bytes a positive multiple of 16, buf 16-byte
 * aligned); one XOR of the data per wave goes to sink[0, pic_calib_read_sink_words). */
int pic_calib_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/* dst[0, bytes) = src[0, bytes) (bytes a positive multiple of 16, both 16-byte aligned,
 * not overlapping). */
int pic_calib_copy(const void *src, void *dst, int64_t bytes, void *stream);

/* buf[0, bytes) = ~buf[0, bytes) in place, bitwise (bytes a positive multiple of 16,
 * buf 16-byte aligned): each byte read once and written once at the same address. */
int pic_calib_update(void *buf, int64_t bytes, void *stream);

/* Floating-point operations of one pic_calib_mfma launch. */
int64_t pic_calib_mfma_flops(int32_t n_workgroups, int32_t iters);

/* n_workgroups x 4 waves, each running `iters` (a positive multiple of 4) rounds of
 * four independent v_mfma_f32_32x32x16_bf16 (fp32 accumulate) on operands read once
 * from `operands` (512 bf16x8 values = 8 KiB of bf16, A fragments then B fragments,
 * 16-byte aligned; random values make the run representative); one float per thread
 * goes to sink[0, n_workgroups * 256). */
int pic_calib_mfma(const void *operands, float *sink, int32_t n_workgroups, int32_t iters,
                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PIC_CALIB_H */
