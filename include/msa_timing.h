/*
 * msa_timing.h — kernel timing for measurement tools (the measurement build only).
 *
 * These two calls are exported by libmsa_timed.so, a build of the same kernel
 * and API objects as libmsa.so plus this timing hook. The product library
 * libmsa.so does not export them and holds no mutable state: its calls are
 * re-entrant.
 *
 * msa_prof_begin(kernel, n): from now on, the library records a HIP event pair
 * on the launch stream around each of the next n launches of kernel `kernel`
 * (one of MSA_K_*), or of any kernel with MSA_K_ALL. Calling it again discards
 * the previous recording.
 * msa_prof_end(ms, launches): waits for the recorded events and writes, for
 * each kernel id x, the summed duration in milliseconds (ms[x]) and the number
 * of launches timed (launches[x]); both arrays hold MSA_K_COUNT entries and
 * either may be NULL. Recording then stops.
 *
 * The recording is process-wide state guarded by a mutex: one measuring caller
 * at a time. Errors: MSA_ERR_SHAPE for an unknown kernel or n outside
 * [1, 100000]; MSA_ERR_DEVICE when an event cannot be created or read.
 */
#ifndef MSA_TIMING_H
#define MSA_TIMING_H

#include "msa.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MSA_K_INDEX_BLOCKMAX = 0, MSA_K_TOPK = 1, MSA_K_BUCKET_HIST = 2, MSA_K_BUCKET_SCAN = 3,
  MSA_K_BUCKET_SCATTER = 4, MSA_K_WORK_ITEMS = 5, MSA_K_SPARSE_ATTN = 6, MSA_K_COMBINE = 7,
  MSA_K_KL_IDX_STATS = 8, MSA_K_KL_IDX_LSE = 9, MSA_K_KL_MAIN = 10, MSA_K_KL_REDUCE = 11,
  MSA_K_ATTN_BWD = 12, MSA_K_IDX_BWD = 13, MSA_K_DENSE_LSE = 14, MSA_K_KL_DENSE = 15,
  MSA_K_RECALL = 16, MSA_K_DENSE_LSE_IDX = 17, MSA_K_INDEX_FP8 = 18, MSA_K_QUANTIZE_FP8 = 19,
  MSA_K_KL_DENSE_CHAIN = 20, MSA_K_BUCKET_SORT = 21, MSA_K_BWD_FINALIZE = 22,
  MSA_K_COUNT = 23, MSA_K_ALL = -1
};
msa_status msa_prof_begin(int kernel, int max_launches);
msa_status msa_prof_end(float* ms, int* launches);

#ifdef __cplusplus
}
#endif

#endif /* MSA_TIMING_H */
