/*
 * gdn_calib.h -- two measurement kernels that give the attainable peaks of the GPU a
 * benchmark compares against, in the same run: a streaming device copy (HBM) and a loop of
 * independent fp16 matrix-core products.  They are not part of the GDN computation and live in
 * their own library (libgdn_calib.so).
 *
 * Both enqueue on `stream` (a hipStream_t, or NULL for the default stream), allocate nothing,
 * keep no state and return 0 on success, 1 for invalid arguments (nothing launched), 3 for a
 * launch error.
 */
#ifndef GDN_CALIB_H
#define GDN_CALIB_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copies `bytes` bytes of device memory from src to dst with 16-byte loads and stores over a
 * grid of `blocks` workgroups of 256 threads (grid-stride).  variant 0: four loads in flight
 * per thread; 1: eight; 2: eight, with non-temporal stores; 3: eight, in place (src == dst:
 * every line is read and written back, the access pattern of an in-place state update);
 * 4: each workgroup copies one contiguous slice of bytes / blocks, eight loads in flight.
 * src and dst: device pointers, 16-byte aligned; not overlapping, except src == dst for
 * variant 3; bytes a multiple of 32768 (of 32768 * blocks for variant 4).
 */
int gdn_calib_copy(const void *src, void *dst, size_t bytes, int blocks, int variant,
                   void *stream);

/*
 * Runs `iters` rounds of 8 independent v_mfma_f32_16x16x32_f16 products per wavefront on
 * `blocks` workgroups of 4 wavefronts; each thread writes one float (a sum of its accumulators)
 * to out[blocks * 256].  Matrix-core flops performed: blocks * 4 * iters * 8 * 16384.
 * out: device pointer to blocks * 256 floats.  1 <= iters <= 1 << 20.
 */
int gdn_calib_mfma(float *out, int blocks, int iters, void *stream);

/*
 * The same loop with a clock record: form 0 runs 8 independent v_mfma_f32_16x16x32_f16 chains
 * per wavefront (flops as above), form 1 four independent v_mfma_f32_32x32x16_f16 chains
 * (blocks * 4 * iters * 4 * 32768 flops).  Wavefront 0 of workgroup b writes
 * clk[2b] = shader-clock cycles and clk[2b + 1] = constant-rate wall-clock ticks spent in its
 * loop; cycles / ticks * gdn_calib_wall_clock_khz() is the engine clock (kHz) during the loop.
 * out: device pointer to blocks * 256 floats; clk: device pointer to 2 * blocks unsigned
 * 64-bit integers.  1 <= iters <= 1 << 20, form 0 or 1.
 */
int gdn_calib_mfma_clock(float *out, unsigned long long *clk, int blocks, int iters, int form,
                         void *stream);

/* The rate of the constant wall clock of the current device in kHz, or -1 on error. */
int gdn_calib_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CALIB_H */
