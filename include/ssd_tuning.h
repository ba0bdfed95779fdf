/*
 * ssd_tuning.h -- process-wide launch-shape knobs of libssd.so, for measurement tools.
 *
 * Results never depend on these settings (only the grouping of work into workgroups does).
 * The setting is global to the process and not synchronised: set it before issuing work,
 * never while another thread calls into the library.
 */
#ifndef SSD_TUNING_H_
#define SSD_TUNING_H_

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
 * Unknown keys are ignored. */
void ssd_tune_set(int key, int value);

#ifdef __cplusplus
}
#endif

#endif /* SSD_TUNING_H_ */
