/*
 * ssd_peak.h -- libssd_peak.so, a measurement-only library beside libssd.so: register-resident
 * MFMA loops that give the attainable matrix-core rate of the two MFMA shapes the SSD kernels
 * issue, so that measured peaks can be set beside the published ones the rooflines quote.
 * Nothing in libssd.so depends on it.
 */
#ifndef SSD_PEAK_H_
#define SSD_PEAK_H_

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one launch on `stream`: `blocks` workgroups of 256 threads, every wavefront running
 * `iters` rounds of four independent MFMA chains with operands held in registers.
 * kind 0: v_mfma_f32_16x16x4_f32 (2048 flops each); kind 1: v_mfma_f32_16x16x32_bf16 (16384).
 * `out`: caller-owned device buffer of blocks * 256 floats, receives a checksum (keeps the
 * loop live).  Returns 0; 1 for an unknown kind, blocks or iters <= 0 or a null `out` (nothing
 * launched); otherwise the HIP error code of the launch.  Time it with events on `stream`. */
int ssd_peak_mfma_launch(int kind, int blocks, int iters, float* out, hipStream_t stream);

/* Floating-point operations of one such launch. */
double ssd_peak_mfma_flops(int kind, int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* SSD_PEAK_H_ */
