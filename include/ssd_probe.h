/* ssd_probe.h -- measurements of the machine the SSD kernels run on (libssd_probe.so).
 *
 * Not part of the SSD computation: these calls measure the constants its roofline is
 * priced against -- the dense bf16 matrix-core rate that the chip actually reaches and
 * the shader clock it runs at, alone or beside other work -- so that a benchmark can
 * report against measured peaks as well as the published ones (256 CUs, 2.4 GHz,
 * 2.5 PFLOP/s dense bf16).
 *
 * Conventions as in ssd.h: device pointers are the caller's, every launch goes on the
 * caller's stream (a hipStream_t passed as void*, NULL for the default stream), nothing
 * is allocated and nothing synchronizes.  Return 0 on success, SSD_ERR_INVALID_ARG (-1)
 * for bad arguments (nothing enqueued), SSD_ERR_HIP (-4) when a launch fails.
 *
 * Clock stamps: each workgroup b writes four unsigned 64-bit values to stamps[4 b ..]:
 * the shader-clock counter (s_memtime) and the 100 MHz real-time counter (s_memrealtime)
 * when its first wave starts, then the same two when it ends.  The shader clock over the
 * workgroup's life is (stamp[2] - stamp[0]) / (stamp[3] - stamp[1]) * 100 MHz.
 */
#ifndef SSD_PROBE_H
#define SSD_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 MFMA rate: `blocks` workgroups of 256 threads (one wave per SIMD; use two
 * per CU to give each SIMD two waves), each wave issuing 4 * iters independent
 * v_mfma_f32_32x32x16_bf16 on register operands (32768 flops each).  Total flops =
 * blocks * 4 waves * 4 * iters * 32768.  stamps: [blocks][4] uint64 (device).
 * iters in [1, 2^30], blocks in [1, 65536]. */
int ssd_probe_mfma_bf16(int64_t iters, int blocks, uint64_t* stamps, void* stream);

/* Clock sampler: `blocks` workgroups of one wave, each sleeping `spins` times 64 clocks
 * (s_sleep 1) between its two stamps; launched on a second stream beside a kernel that
 * leaves compute units free, its stamps give the clock while that kernel runs.
 * spins in [1, 2^24], blocks in [1, 65536]; stamps: [blocks][4] uint64 (device). */
int ssd_probe_clock(int64_t spins, int blocks, uint64_t* stamps, void* stream);

/* Device 0's compute-unit count and peak shader clock in kHz (host pointers).  Returns
 * SSD_ERR_HIP when the device cannot be queried. */
int ssd_probe_device(int* compute_units, int* max_clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* SSD_PROBE_H */
