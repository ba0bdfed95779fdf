/*
 * ssd_tuning.h -- process-wide launch-shape knobs of libssd.so, for measurement tools.
 *
 * Results never depend on keys 0-4 and 6 (only the grouping of work into workgroups does); key 5
 * changes the order in which the chunk states are summed, so results agree to rounding.
 * The setting is global to the process and not synchronised: set it before issuing work,
 * never while another thread calls into the library.
 */
#ifndef SSD_TUNING_H_
#define SSD_TUNING_H_

#include "ssd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* key 0: heads per chunk_scan workgroup (heads of one group sharing one C B^T evaluation):
 *        1 or 2; 0 restores the built-in choice; ignored unless it divides nheads / ngroups.
 * key 1: minimum chunk_scan workgroup count the built-in choice aims for (default 512).
 * key 2: chunk_scan decomposition: 1 = one workgroup per 64-row block of a chunk,
 *        2 = one workgroup per whole chunk, 0 = built-in choice (1).
 * key 3: tokens per thread of ssd_conv1d_silu (rounded up to a multiple of 4); 0 restores
 *        the built-in choice (64, fewer on small inputs).
 * key 4: chunk_scan row blocks: units (b, c, head) per dispatch group on one XCD, whose row
 *        blocks run together (heaviest first within the group); 0 restores the built-in 16.
 * key 5: chunk states: 1 = chunk_state then state_passing, 2 = one pass over the chunks per
 *        (b, h, headdim slice) where an instantiation exists, 0 = built-in choice.
 * key 6: one-pass chunk states: headdim rows per workgroup (0 = all of them).
 * Unknown keys are ignored. */
void ssd_tune_set(int key, int value);

/* Which chunk-state path ssd_fwd takes for these sizes under the current settings:
 * 1 = chunk_state then state_passing (three forward kernels), 2 = one pass over the chunks
 * (two forward kernels: no state_passing launch; the stage events of ssd_fwd_timed for
 * state_passing then bracket no kernel), 0 = invalid or empty arguments.  Pure host logic. */
int ssd_fwd_state_path(const ssd_dims_t* dims, int chunk_size);

#ifdef __cplusplus
}
#endif

#endif /* SSD_TUNING_H_ */
