/*
 * arrms.h -- fused rank-sum + residual-add + RMSNorm (+ per-token FP8 E4M3)
 * epilogue for MI355X (gfx950), C ABI of libarrms.so.
 *
 * The operation is the epilogue of a tensor-parallel all-reduce, taken as the
 * share of work one GPU can show: R rank-input buffers, all resident in this
 * GPU's HBM, stand in for the peer-visible registered buffers of the
 * collective. Sources: ROCm/aiter PR #6699 "gfx1250 fused all-reduce +
 * RMSNorm" (sections Changes and Test results, and the commit notes), PR
 * #3462 "optimize fused AllReduce + RMSNorm" (section Technical Details), PR
 * #5807 "Specialize partial tiles in two-stage custom all-reduce" (section
 * Proposed modifications).
 *
 * Every entry point is a plain C function; buffers are raw pointers, sizes
 * are ints, the stream is a HIP stream handle. Nothing here prints, throws or
 * aborts: failures come back as a negative status (see ARRMS_ERR_*), and on
 * any failure nothing has been launched and no output has been written.
 */
#ifndef ARRMS_H
#define ARRMS_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef ARRMS_API
#define ARRMS_API __attribute__((visibility("default")))
#endif

/* ---- status codes ---------------------------------------------------- */
#define ARRMS_OK 0
#define ARRMS_ERR_INVALID (-1)     /* NULL required pointer, R/M/H out of range, bad flags, overlap */
#define ARRMS_ERR_UNSUPPORTED (-2) /* misaligned pointer, H*sizeof(T) not a multiple of 16 bytes,
                                      FP8 with fp32 data: the caller takes its unfused path,
                                      as the communicator on the pages does for padded rows */
#define ARRMS_ERR_NO_STAGING (-3)  /* two-stage path needed inside stream capture, no staging reserved */
#define ARRMS_ERR_HIP (-4)         /* a HIP runtime call or kernel launch failed */

/* ---- flags (bit field) ------------------------------------------------ */
#define ARRMS_DTYPE_BF16 0         /* bits 0-1: element type T of inputs, residual, weight, outputs */
#define ARRMS_DTYPE_FP16 1
#define ARRMS_DTYPE_FP32 2
#define ARRMS_DTYPE_MASK 3
#define ARRMS_GEMMA 4              /* scale by (1 + w) instead of w (gemma_norm, PR #6699 Changes) */
#define ARRMS_FP8 8                /* per-token FP8 E4M3 output + fp32 per-row scales (PR #6699 Changes) */
#define ARRMS_FORCE_ONE_STAGE 16   /* force the one-stage direct-read path */
#define ARRMS_FORCE_TWO_STAGE 32   /* force the two-stage path (flat rank reduce into staging, then row pass) */

/* ---- quantised outputs of arrms_fused_quant ------------------------------- */
#define ARRMS_QUANT_FP8_TOKEN 1    /* per-token FP8: as arrms_fused with ARRMS_FP8 */
#define ARRMS_QUANT_FP8_GROUP 2    /* per-group FP8: E4M3 codes [M][H], fp32 scales [M][H/128] */
#define ARRMS_QUANT_MXFP4 3        /* MXFP4: packed E2M1 codes [M][H/2], E8M0 scales [M][H/32] */
#define ARRMS_FP8_GROUP_SIZE 128   /* columns per per-group FP8 scale (no page fixes it; see arrms_fused_quant) */
#define ARRMS_MX_BLOCK 32          /* columns per MXFP4 scale (OCP MX block size) */

/* ---- limits -------------------------------------------------------------- */
#define ARRMS_MAX_RANKS 8          /* the pages go up to TP8 (PR #3462 Test Results) */
#define ARRMS_MAX_HIDDEN 16384
#define ARRMS_MAX_ROW_BYTES 65536 /* H * sizeof(T): bf16/fp16 rows up to 32 KiB, fp32 up to 64 KiB */
#define ARRMS_DEFAULT_STAGING_BYTES (16u << 20) /* 16 MiB staging region (PR #6699 Changes) */
#define ARRMS_NOALLOC_SCRATCH_BYTES (16u << 20) /* fixed staging of arrms_fused_noalloc, per GPU */

/* ---- paths returned by arrms_query_path ---------------------------------- */
#define ARRMS_PATH_NONE 0          /* M == 0: nothing to launch */
#define ARRMS_PATH_ONE_STAGE 1
#define ARRMS_PATH_TWO_STAGE 2

/*
 * arrms_fused -- the fused epilogue (PR #6699 Changes: direct-read one-stage
 * and exact two-stage fused kernels; PR #3462 Technical Details: rank-ordered
 * fp32 reduce).
 *
 * For every row m < M and column j < H, with T the type named by flags:
 *   a      = RNE_T( x_0 + x_1 + ... + x_{R-1} )      fp32 adds in rank order 0..R-1,
 *                                                    accumulator starting at x_0
 *   h      = RNE_T( fl32(a + residual) )             -> residual_out[m][j]
 *   rstd   = 1 / sqrt( sum_j h^2 / H + eps )         statistics in fp64
 *   y      = RNE_T( (h * w_eff) * rstd )             w_eff = w, or 1 + w with ARRMS_GEMMA;
 *                                                    one rounding from fp64 -> out[m][j]
 *   FP8:   amax = max_j |y| ; scale = fl32(amax / 448) -> fp8_scale[m]
 *          q = E4M3_RNE_saturating( fl32(y / scale) ) -> fp8_out[m][j]
 *          (amax == 0 gives scale 0 and q = +-0 with the sign of y; a NaN y
 *          makes amax and the scale NaN, and every NaN quotient codes as
 *          0x7F, without sign)
 * For T = fp32 the two RNE_T steps before the norm are the fp32 operations.
 *
 * rank_in      host array of R device pointers, each to [M][H] T (row-major,
 *              contiguous). The array is read during the call and its values
 *              are baked into the launch (and into a captured graph); the
 *              caller may reuse it after return. Rank pointers may repeat.
 * R            1 .. ARRMS_MAX_RANKS.
 * residual     device [M][H] T.
 * weight       device [H] T.
 * out          device [M][H] T. Required without ARRMS_FP8; with ARRMS_FP8 it is
 *              the optional T mirror of the quantised output (NULL: not written).
 * residual_out device [M][H] T; may equal residual exactly (in place).
 * fp8_out      device [M][H] bytes (E4M3 codes), required with ARRMS_FP8, else ignored.
 * fp8_scale    device [M] float, required with ARRMS_FP8, else ignored.
 * M            rows, >= 0 (0: returns ARRMS_OK, launches nothing).
 * H            hidden size, 1 .. ARRMS_MAX_HIDDEN, with H * sizeof(T) % 16 == 0 and
 *              H * sizeof(T) <= ARRMS_MAX_ROW_BYTES.
 * eps          finite, >= 0.
 * flags        ARRMS_DTYPE_* | ARRMS_GEMMA | ARRMS_FP8 | at most one ARRMS_FORCE_*
 *              (and the verification bit of arrms_tuning.h). ARRMS_FP8 requires
 *              bf16 or fp16.
 * stream       HIP stream; all work is enqueued on it, asynchronously.
 *
 * Every device pointer must be 16-byte aligned (fp8_scale: 4-byte aligned).
 * No output may overlap an input or another output, except residual_out ==
 * residual. The buffers are caller-owned; the library keeps no reference.
 * No host synchronisation and no allocation happen on the one-stage path.
 * The two-stage path uses the library's staging buffer on the current device
 * (arrms_reserve_staging); outside stream capture it is reserved on first use,
 * inside capture an unreserved buffer yields ARRMS_ERR_NO_STAGING. Two-stage
 * calls on one device share that buffer: issue them on one stream, or order
 * them. The same inputs give the same bits on every call and on both paths.
 */
ARRMS_API int arrms_fused(const void *const *rank_in, int R, const void *residual, const void *weight,
                void *out, void *residual_out, void *fp8_out, float *fp8_scale, int M, int H,
                float eps, int flags, hipStream_t stream);

/*
 * arrms_fused_noalloc -- arrms_fused for callers that cannot allocate device
 * memory: code under HIP graph capture with no staging reserved beforehand,
 * tight serving loops, harnesses that forbid hipMalloc. Arguments, results,
 * paths and errors are arrms_fused's; no call allocates or frees anything.
 *
 * The two-stage path stages its rows in a fixed region of
 * ARRMS_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on every GPU it
 * runs on until the process ends (rows go through it in chunks that fit; a row
 * wider than the region would be ARRMS_ERR_UNSUPPORTED, which no H up to
 * ARRMS_MAX_HIDDEN reaches). The region's address is looked up once per device,
 * on the first call there with valid arguments and M > 0 (ARRMS_ERR_HIP if
 * that fails): make that first call outside graph capture. Every call on one GPU
 * shares the region, and its contents are whatever the last call left (every
 * byte a call reads there it has written first): two-stage calls that overlap
 * in time on one GPU -- on different streams, or from different threads --
 * race on it and must be ordered by the caller. The one-stage path uses no
 * scratch at all.
 */
ARRMS_API int arrms_fused_noalloc(const void *const *rank_in, int R, const void *residual,
                                  const void *weight, void *out, void *residual_out, void *fp8_out,
                                  float *fp8_scale, int M, int H, float eps, int flags,
                                  hipStream_t stream);

/*
 * arrms_fused_strided -- arrms_fused over row-strided (padded) matrices. The
 * pages' communicator declines padded or strided rows and falls back to its
 * unfused path (PR #6699 Changes); this entry point takes them fused.
 *
 * Row m of rank input r starts at element m * ld_in of rank_in[r]; likewise
 * ld_residual, ld_out and ld_residual_out for residual, out and residual_out,
 * all counted in elements of T, and ld_fp8 for fp8_out, counted in bytes
 * (ignored without ARRMS_FP8). Only the first H elements of each row are read
 * or written: the padding between rows is never touched. Every stride is at
 * least H and no matrix spans more than 2^48 bytes (else ARRMS_ERR_INVALID);
 * every stride spans a multiple of 16 bytes, ld_fp8 a multiple of 8 bytes
 * (else ARRMS_ERR_UNSUPPORTED). In place (residual_out == residual) requires
 * ld_residual_out == ld_residual. Overlap is judged on each matrix's whole
 * byte range, first element to last, padding included. Everything else --
 * arguments, results, paths, staging and error behaviour -- is arrms_fused's;
 * with every stride equal to H the call is arrms_fused.
 */
ARRMS_API int arrms_fused_strided(const void *const *rank_in, int R, const void *residual,
                                  const void *weight, void *out, void *residual_out, void *fp8_out,
                                  float *fp8_scale, int M, int H, long long ld_in,
                                  long long ld_residual, long long ld_out, long long ld_residual_out,
                                  long long ld_fp8, float eps, int flags, hipStream_t stream);

/*
 * arrms_fused_quant -- arrms_fused with one of the quantised outputs the pages
 * name for the fused op (PR #6699 Motivation and Changes: the per-token, the
 * per-group and the MXFP4 quant forms). The pages do not define the last two;
 * this library reads them as:
 *   ARRMS_QUANT_FP8_GROUP  the per-token FP8 steps on each group of
 *       ARRMS_FP8_GROUP_SIZE (128) consecutive columns -- no page gives a
 *       group size: 128 is this library's choice (the usual 1 x 128
 *       activation grouping), not a reading of the pages: scale = fl32(gmax /
 *       448) over the T-rounded y of the group, q = E4M3_RNE_sat(fl32(y /
 *       scale)), an all-zero group gives scale 0 and signed zeros, a NaN
 *       in the group a NaN scale and codes 0x7F.
 *       q_out: [M][H] E4M3 codes; q_scale: [M][H/128] fp32 (4-byte aligned).
 *   ARRMS_QUANT_MXFP4  OCP Microscaling Formats v1.0 MXFP4 over blocks of
 *       ARRMS_MX_BLOCK (32) columns: X = 2^(floor(log2 bmax) - 2) with the
 *       exponent clamped to [-127, 127], stored as its E8M0 code (an all-zero
 *       block gives code 0; a NaN or an infinity in the block gives 0xFF and
 *       +-6's element code with y's sign, 0x7 for a NaN element); elements
 *       E2M1_RNE_sat(y / X) (y / X is exact).
 *       q_out: [M][H/2] bytes, two codes per byte, the even column in the
 *       low nibble (sign in bit 3 of each nibble); q_scale: [M][H/32] bytes.
 *   ARRMS_QUANT_FP8_TOKEN  exactly arrms_fused with ARRMS_FP8 (q_scale [M] fp32).
 * out is the optional T mirror (NULL: not written). H must be a multiple of
 * the group (else ARRMS_ERR_UNSUPPORTED), T bf16 or fp16; flags as for
 * arrms_fused but without ARRMS_FP8 (ARRMS_ERR_INVALID), quant outside 1..3
 * is ARRMS_ERR_INVALID. Rows are contiguous. Both paths, the results'
 * determinism and every other rule are arrms_fused's.
 */
ARRMS_API int arrms_fused_quant(const void *const *rank_in, int R, const void *residual,
                                const void *weight, void *out, void *residual_out, void *q_out,
                                void *q_scale, int M, int H, float eps, int flags, int quant,
                                hipStream_t stream);

/*
 * arrms_allreduce_sum -- the plain rank all-reduce without the norm epilogue
 * (the flattened message sweep of PR #5807 Proposed modifications, and the
 * rank-ordered reduce of PR #3462 Technical Details): for every element
 * i < n, out[i] = RNE_T(x_0[i] + x_1[i] + ... + x_{R-1}[i]) with fp32 adds in
 * rank order 0..R-1 and the accumulator starting at x_0 (for T = fp32 the
 * fp32 sum itself).
 *
 * rank_in  host array of R device pointers, each to n elements of T (read
 *          during the call, as in arrms_fused). Rank pointers may repeat.
 * R        1 .. ARRMS_MAX_RANKS.
 * out      device n elements of T; may equal one of the rank pointers
 *          exactly (in place), must not overlap any of them otherwise.
 * n        elements, >= 0 (0: returns ARRMS_OK, launches nothing), at most
 *          2^48 bytes (else ARRMS_ERR_INVALID), with n * sizeof(T) % 16 == 0
 *          (else ARRMS_ERR_UNSUPPORTED).
 * flags    ARRMS_DTYPE_* only; any other bit gives ARRMS_ERR_INVALID.
 * stream   HIP stream; one kernel launch, asynchronous, no allocation, no
 *          shared state (safe in graph capture and on concurrent streams).
 *
 * Every device pointer must be 16-byte aligned (else ARRMS_ERR_UNSUPPORTED).
 * Complete 512-pack tiles run without bounds checks; only the last tile of a
 * ragged message checks them (PR #5807 Proposed modifications, has_tail).
 */
ARRMS_API int arrms_allreduce_sum(const void *const *rank_in, int R, void *out, long long n, int flags,
                                  hipStream_t stream);

/*
 * arrms_reserve_staging -- make the staging buffer of the two-stage path on
 * the current device at least `bytes` (0: ARRMS_DEFAULT_STAGING_BYTES), the
 * per-rank staging region of PR #6699 Changes. A larger existing buffer is
 * kept. A smaller one is replaced by a new allocation and retired, not freed:
 * two-stage work still in flight, and HIP graphs captured earlier (whose
 * launches hold the old address), keep valid memory until
 * arrms_release_staging. Call it before capturing a graph that may take the
 * two-stage path. Returns ARRMS_OK or ARRMS_ERR_HIP (allocation failed;
 * nothing changed).
 */
ARRMS_API int arrms_reserve_staging(size_t bytes);

/* arrms_release_staging -- free the current device's staging buffer and every
 * buffer retired by an earlier growth, after synchronising the device. Any HIP
 * graph captured with a two-stage call on this device holds those addresses:
 * destroy such graphs before calling it (a replay afterwards would touch freed
 * memory). A later two-stage call reserves a new buffer. Returns ARRMS_OK or
 * ARRMS_ERR_HIP. */
ARRMS_API int arrms_release_staging(void);

/* arrms_staging_bytes -- size of the current device's staging buffer (0 if none). */
ARRMS_API size_t arrms_staging_bytes(void);

/*
 * arrms_query_path -- which path arrms_fused takes for these sizes and flags
 * (ARRMS_PATH_*), or a negative status if the arguments are invalid. Pure host
 * code; touches no device. The choice follows PR #6699 Changes (wide rows
 * above a size threshold go two-stage, the rest one-stage) with thresholds
 * measured on MI355X rather than the pages' multi-GPU ones.
 */
ARRMS_API int arrms_query_path(int M, int H, int R, int flags);

/* arrms_status_string -- static description of a status code. */
ARRMS_API const char *arrms_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ARRMS_H */
