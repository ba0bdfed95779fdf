/*
 * ssd_tuning.h -- measurement entry points of libssd.so: launch-shape options passed per
 * call, and per-kernel timing events.
 *
 * The plain entry points of ssd.h take the built-in launch choice, which is a pure function of
 * their arguments.  The *_ex variants below take the same arguments plus an optional
 * ssd_launch_opts_t (NULL or all-zero = the built-in choice, i.e. exactly the plain entry
 * point) and optional timing events.  Nothing is kept between calls: the options of one call
 * never affect another, and concurrent calls with different options do not interfere.
 * Results never depend on the options except where a field says so (to rounding).
 */
#ifndef SSD_TUNING_H_
#define SSD_TUNING_H_

#include "ssd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launch-shape options.  Every field 0 = the built-in choice; values that do not apply to the
 * call's sizes (no such instantiation) fall back to the built-in choice. */
typedef struct {
  int32_t scan_variant;     /* chunk_scan decomposition: 1 = one workgroup per 64-row block of a
                             * chunk, 2 = one workgroup per whole chunk, 3 = one workgroup per chunk,
                             * group and slice of the group's heads, C B^T formed once per slice
                             * (SSD_BF16, chunk 256, headdim 64, dstate 128) */
  int32_t heads_per_block;  /* chunk_scan heads per workgroup sharing one C B^T evaluation: 1 or 2
                             * for decompositions 1 and 2, any divisor of nheads / ngroups for 3
                             * (ignored unless it divides nheads / ngroups) */
  int32_t min_blocks;       /* whole-chunk decomposition: minimum workgroup count the head-block
                             * choice aims for (built-in 512) */
  int32_t rows_group;       /* row blocks: units (b, c, head) per dispatch group on one XCD
                             * (built-in 16) */
  int32_t state_path;       /* chunk states: 1 = chunk_state then state_passing, 2 = one pass over
                             * the chunks per (b, h, headdim slice), 3 = segments of consecutive
                             * chunks per (b, group, slice of heads), each from a zero state, joined
                             * by state_passing over the segments (SSD_BF16, chunk 256, headdim 64,
                             * dstate 128, with chunk_scan decomposition 3); the paths sum the states
                             * in different orders, so results agree to rounding */
  int32_t state_slice;      /* one-pass chunk states: headdim rows per workgroup (0 = all) */
  int32_t conv_tokens;      /* ssd_conv1d_silu tokens per thread (rounded up to a multiple of 4) */
  int32_t state_heads;      /* segmented chunk states: heads per workgroup (1, 2, 4 or 5) */
  int32_t state_chunks;     /* segmented chunk states: chunks per segment (at least 2) */
  int32_t bwd_heads;        /* ssd_bwd: heads per bwd_dxdb and bwd_dc workgroup, whose dB and dC
                             * contributions are summed in registers before they leave the chip: 1,
                             * or 4 for SSD_BF16 when it divides nheads / ngroups (else 1); the
                             * summation order changes, results agree to rounding */
} ssd_launch_opts_t;

/* ssd_fwd with options and per-kernel timing.  `opts` may be NULL.  `stage_events` is NULL or
 * an array of 6 caller-created events (hipEventCreate): [2k] and [2k + 1] are the start and
 * stop of kernel k (0 chunk_state, 1 state_passing, 2 chunk_scan), recorded by the kernel's own
 * dispatch (hipExtLaunchKernelGGL), so hipEventElapsedTime of a pair is that kernel's execution
 * time alone, as in a profiler's kernel trace.  On the one-pass path kernel 0 is
 * chunk_state_seq and the state_passing pair is recorded back to back around no kernel.  Event
 * records cannot be captured into a graph: with non-NULL stage_events on a stream under capture
 * the call returns SSD_ERR_UNSUPPORTED and launches nothing. */
ssd_status_t ssd_fwd_ex(const ssd_dims_t* dims,
                        const void* x, const void* dt, const float* dt_bias, const float* A,
                        const void* B, const void* C, const float* D, const void* z, int chunk_size,
                        const float* initial_state, void* y, float* final_state,
                        void* workspace, size_t workspace_bytes, hipStream_t stream,
                        const ssd_launch_opts_t* opts, hipEvent_t* stage_events);

/* ssd_bwd with options and per-stage timing: `stage_events` NULL or 20 caller-created events,
 * [2k] and [2k + 1] the start and stop of stage k, recorded by the dispatches themselves:
 * 0 chunk_state, 1 state_passing (forward recompute), 2 chunk_scan of the pre-gate output and
 * 3 the gate's backward (both recorded back to back, i.e. empty, without a gate), 4 chunk_state
 * of the output gradients, 5 reverse state_passing, 6 the anti-causal kernel, 7 the causal
 * kernel, 8 finalize, 9 the two reduction kernels.  Refuses a stream under graph capture when
 * stage_events is given (SSD_ERR_UNSUPPORTED, nothing launched). */
ssd_status_t ssd_bwd_ex(const ssd_dims_t* dims,
                        const void* x, const void* dt, const float* dt_bias, const float* A,
                        const void* B, const void* C, const float* D, const void* z, int chunk_size,
                        const float* initial_state, const void* dout, const float* dfinal_state,
                        void* dx, void* ddt, float* ddt_bias, float* dA, void* dB, void* dC, float* dD,
                        void* dz, float* dinitial_state,
                        void* workspace, size_t workspace_bytes, hipStream_t stream,
                        const ssd_launch_opts_t* opts, hipEvent_t* stage_events);

/* ssd_step with timing: `events` NULL or 2 caller-created events, the start and stop of the
 * step's kernel recorded by its own dispatch.  Refuses a stream under graph capture when events
 * are given (SSD_ERR_UNSUPPORTED, nothing launched). */
ssd_status_t ssd_step_ex(const ssd_dims_t* dims, float* state,
                         const void* x, const void* dt, const float* dt_bias, const float* A,
                         const void* B, const void* C, const float* D, const void* z,
                         void* y, hipStream_t stream, hipEvent_t* events);

/* ssd_gated_rmsnorm with timing: `events` NULL or 2 caller-created events, the start and stop
 * of the kernel recorded by its own dispatch.  Refuses a stream under graph capture when events
 * are given (SSD_ERR_UNSUPPORTED, nothing launched). */
ssd_status_t ssd_gated_rmsnorm_ex(const ssd_dims_t* dims, const void* y, const void* z, const float* weight,
                                  float eps, int norm_heads, void* out, hipStream_t stream, hipEvent_t* events);

/* ssd_conv1d_silu with options (field conv_tokens). */
ssd_status_t ssd_conv1d_silu_ex(const ssd_dims_t* dims, int conv_width, const void* xbc,
                                const float* weight, const float* bias, const void* conv_state_in,
                                void* conv_state_out, void* x, void* B, void* C, hipStream_t stream,
                                const ssd_launch_opts_t* opts);

/* Which chunk-state path ssd_fwd_ex takes for these sizes and options (NULL = the built-in
 * choice of ssd_fwd): 1 = chunk_state then state_passing (three forward kernels), 2 = one pass
 * over the chunks (two forward kernels: no state_passing launch; the state_passing events of
 * ssd_fwd_ex then bracket no kernel), 3 = segmented chunk states (chunk_state_seg in place of
 * chunk_state, state_passing over the segments), 0 = invalid or empty arguments.  Pure host
 * logic. */
int ssd_fwd_state_path(const ssd_dims_t* dims, int chunk_size, const ssd_launch_opts_t* opts);

/* Chunks per segment on the segmented path (3) for these sizes and options, 0 on the other paths
 * or for invalid or empty arguments.  Pure host logic. */
int ssd_fwd_state_segment_chunks(const ssd_dims_t* dims, int chunk_size, const ssd_launch_opts_t* opts);

/* Heads per bwd_dxdb and bwd_dc workgroup that ssd_bwd_ex takes for these sizes and options
 * (NULL = the built-in choice of ssd_bwd): 1, or 4 when dB and dC are summed over slices of four
 * heads on chip; 0 for invalid arguments.  Pure host logic. */
int ssd_bwd_heads(const ssd_dims_t* dims, int chunk_size, const ssd_launch_opts_t* opts);

#ifdef __cplusplus
}
#endif

#endif /* SSD_TUNING_H_ */
