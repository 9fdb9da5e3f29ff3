/*
 * arrms_tuning.h -- tuning and verification hooks of libarrms.so. Not part of
 * the stable interface of arrms.h: the launch-shape sweep of the benchmark and
 * the parity tests use them; an application has no need to.
 */
#ifndef ARRMS_TUNING_H
#define ARRMS_TUNING_H

#include "arrms.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Verification flag for arrms_fused and its variants: every element takes the
 * exact rounding branch (round-to-odd fp64 -> fp32, IEEE division and the
 * software E4M3 encoder) instead of the fast ones. The results are the same
 * bits; the tests use it to check the fast branches against the exact ones. */
#define ARRMS_EXACT_ONLY 64

/*
 * arrms_fused_config -- arrms_fused with an explicit launch shape for the row
 * kernel (the automatic choice is the shape arrms_fused takes). ppt: 16-byte
 * packs per thread and row (1 to 4); tpr: threads per row (a multiple of 64,
 * tpr * ppt covering the row); rows_per_block: rows handled side by side by
 * one block (tpr * rows_per_block at most 1024 threads with ppt = 1 or fp32
 * data, else 512); blocks: the number of blocks launched -- with fewer blocks
 * than row groups each block takes every blocks-th group of rows in turn;
 * load_window: how many 16-byte loads a thread keeps in flight -- 1 a narrow
 * window (for large launches whose rows are all resident at once), 2 a wide
 * one (the whole row, up to a cap: small launches, and large ones that run in
 * several rounds of blocks), 3 a medium one (8 loads). 0 in any of them keeps
 * the automatic value; a negative value (or a load_window above 3) gives
 * ARRMS_ERR_INVALID and a shape that cannot cover a row
 * ARRMS_ERR_UNSUPPORTED. All other arguments, the results and the error
 * behaviour are arrms_fused's.
 */
ARRMS_API int arrms_fused_config(const void *const *rank_in, int R, const void *residual,
                                 const void *weight, void *out, void *residual_out, void *fp8_out,
                                 float *fp8_scale, int M, int H, float eps, int flags, int ppt,
                                 int tpr, int rows_per_block, int blocks, int load_window,
                                 hipStream_t stream);

/*
 * The row-kernel launch arrms_fused (arrms_fused_quant for quant != 0) makes
 * for these sizes: the one-stage launch, or the two-stage path's row pass over
 * its first chunk (with the default staging size). Written to info[0 ..
 * ARRMS_LAUNCH_INFO - 1]:
 *   [0] path (ARRMS_PATH_*)     [1] packs per thread   [2] threads per row
 *   [3] rows per block          [4] load window (1 narrow, 2 wide, 3 medium)
 *   [5] occupancy cap (1: at most 16 waves per compute unit)
 *   [6] blocks of this shape (narrow-window kernel) one compute unit holds
 *   [7] compute units
 * flags: ARRMS_DTYPE_* | ARRMS_GEMMA | ARRMS_FORCE_* (ARRMS_FP8 means quant =
 * ARRMS_QUANT_FP8_TOKEN); quant: 0 (T output) or ARRMS_QUANT_*; mirror: the T
 * mirror of a quantised output is written. Returns ARRMS_OK or the status
 * arrms_query_path (or arrms_fused_quant's group checks) would give.
 *
 * arrms_query_launch asks the current device for [6] and [7] (its occupancy
 * for each kernel and its compute units). arrms_plan_launch takes them as
 * arguments and touches no device: pure host code, the same rules, for
 * checking them against recorded measurements.
 */
#define ARRMS_LAUNCH_INFO 8
ARRMS_API int arrms_query_launch(int M, int H, int R, int flags, int quant, int mirror, int *info);
ARRMS_API int arrms_plan_launch(int M, int H, int R, int flags, int quant, int mirror, int blocks_per_cu,
                                int cus, int *info);

#ifdef __cplusplus
}
#endif

#endif /* ARRMS_TUNING_H */
