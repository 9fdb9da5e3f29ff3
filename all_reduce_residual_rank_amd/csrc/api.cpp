// api.cpp -- the C ABI of libarrms.so (include/arrms.h): argument checks,
// path and launch-shape choice, the staging buffer, and the launches.
//
// Path choice follows ROCm/aiter PR #6699 "gfx1250 fused all-reduce +
// RMSNorm" (section Changes): a direct-read one-stage kernel, and an exact
// two-stage path (reduce into a staging region, then a row pass applying the
// residual and the norm) that the collective prefers for wide rows. On one
// GPU both read the same R inputs; the thresholds here come from measurement
// on MI355X, not from the pages' multi-GPU numbers.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "arrms.h"
#include "arrms_tuning.h"
#include "launch.hpp"
#include "staging.hpp"

namespace {

using arrms::DT_BF16;
using arrms::DT_FP16;
using arrms::DT_FP32;

constexpr int kKnownFlags = ARRMS_DTYPE_MASK | ARRMS_GEMMA | ARRMS_FP8 | ARRMS_FORCE_ONE_STAGE |
                            ARRMS_FORCE_TWO_STAGE | ARRMS_EXACT_ONLY;
using arrms::kMaxDevices;

int esize(int dt) { return dt == DT_FP32 ? 4 : 2; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const Span &a, const Span &b) { return a.lo < b.hi && b.lo < a.hi; }

// Row strides of the fused call, in elements of each tensor (fp8: bytes).
struct Strides {
    long long in, res, out, rout, q;
};

// Bytes spanned by a strided [M][H] matrix: (M - 1) rows of ld plus one row.
uintptr_t span_bytes(int M, int H, long long ld, int e)
{
    return (uintptr_t)(M - 1) * (uintptr_t)ld * (uintptr_t)e + (uintptr_t)H * (uintptr_t)e;
}

// No operand may span more than 2^48 bytes (far beyond any device memory):
// with that bound every byte offset the kernels form fits in 64 bits.
constexpr long long kMaxSpanBytes = 1ll << 48;

// Whether M rows of H elements (e bytes each) at row stride ld (>= H >= 1)
// span at most kMaxSpanBytes, computed without overflow.
bool span_fits(long long M, long long H, long long ld, int e)
{
    if (ld > kMaxSpanBytes / e || H > ld)
        return false;
    return M <= 1 || (M - 1) <= (kMaxSpanBytes - H * e) / (ld * e);
}

// Quantised outputs: none, per-token FP8 (ARRMS_FP8), per-group FP8, MXFP4.
enum Quant { Q_NONE = 0, Q_TOKEN = 1, Q_GROUP = 2, Q_MX = 3 };

// Checks that need no device: sizes, flags, pointers, alignment, overlap.
int validate(const void *const *rank_in, int R, const void *residual, const void *weight,
             const void *out, const void *residual_out, const void *fp8_out,
             const void *fp8_scale, int M, int H, float eps, int flags, const Strides &ld, int quant)
{
    if (flags & ~kKnownFlags)
        return ARRMS_ERR_INVALID;
    const int dt = flags & ARRMS_DTYPE_MASK;
    if (dt > DT_FP32)
        return ARRMS_ERR_INVALID;
    if ((flags & ARRMS_FORCE_ONE_STAGE) && (flags & ARRMS_FORCE_TWO_STAGE))
        return ARRMS_ERR_INVALID;
    if (R < 1 || R > ARRMS_MAX_RANKS || M < 0 || H < 1)
        return ARRMS_ERR_INVALID;
    if (!(eps >= 0.0f) || eps > 3.4028234e38f)  // rejects NaN, negative, +inf
        return ARRMS_ERR_INVALID;
    const bool fp8 = quant != Q_NONE;
    if ((flags & ARRMS_FP8) && quant != Q_TOKEN)
        return ARRMS_ERR_INVALID;
    if (!rank_in || !residual || !weight || !residual_out)
        return ARRMS_ERR_INVALID;
    for (int r = 0; r < R; ++r)
        if (!rank_in[r])
            return ARRMS_ERR_INVALID;
    if (!fp8 && !out)
        return ARRMS_ERR_INVALID;
    if (fp8 && (!fp8_out || !fp8_scale))
        return ARRMS_ERR_INVALID;
    if (H > ARRMS_MAX_HIDDEN)
        return ARRMS_ERR_UNSUPPORTED;
    if (fp8 && dt == DT_FP32)
        return ARRMS_ERR_UNSUPPORTED;
    if ((quant == Q_GROUP && H % ARRMS_FP8_GROUP_SIZE) || (quant == Q_MX && H % ARRMS_MX_BLOCK))
        return ARRMS_ERR_UNSUPPORTED;
    if (((long long)H * esize(dt)) % 16 != 0 || (long long)H * esize(dt) > ARRMS_MAX_ROW_BYTES)
        return ARRMS_ERR_UNSUPPORTED;
    for (int r = 0; r < R; ++r)
        if (!aligned16(rank_in[r]))
            return ARRMS_ERR_UNSUPPORTED;
    if (!aligned16(residual) || !aligned16(weight) || !aligned16(residual_out) ||
        (out && !aligned16(out)))
        return ARRMS_ERR_UNSUPPORTED;
    if (fp8 && (!aligned16(fp8_out) || (quant != Q_MX && ((uintptr_t)fp8_scale & 3u))))
        return ARRMS_ERR_UNSUPPORTED;
    // strides: at least a row, rows 16-byte aligned
    const int e = esize(dt);
    const long long lds[4] = {ld.in, ld.res, ld.out, ld.rout};
    for (int i = 0; i < 4; ++i) {
        if (lds[i] < H || !span_fits(M, H, lds[i], e))
            return ARRMS_ERR_INVALID;
        if ((lds[i] * e) % 16 != 0)
            return ARRMS_ERR_UNSUPPORTED;
    }
    if (fp8) {
        // codes go out 8 bytes per pack (E4M3) or 4 (packed E2M1): rows must
        // start aligned to that
        const long long qrow = quant == Q_MX ? H / 2 : H;
        if (ld.q < qrow || !span_fits(M, qrow, ld.q, 1))
            return ARRMS_ERR_INVALID;
        if (ld.q % (quant == Q_MX ? 4 : 8) != 0)
            return ARRMS_ERR_UNSUPPORTED;
    }
    const bool inplace = residual_out == residual;
    if (inplace && ld.rout != ld.res)
        return ARRMS_ERR_INVALID;

    // overlap: outputs against inputs and against each other (a strided matrix
    // counts as the whole byte range from its first to its last element)
    if (M == 0)
        return ARRMS_OK;
    Span ins[ARRMS_MAX_RANKS + 2];
    int nin = 0;
    for (int r = 0; r < R; ++r)
        ins[nin++] = {(uintptr_t)rank_in[r], (uintptr_t)rank_in[r] + span_bytes(M, H, ld.in, e)};
    const Span res_span = {(uintptr_t)residual, (uintptr_t)residual + span_bytes(M, H, ld.res, e)};
    ins[nin++] = {(uintptr_t)weight, (uintptr_t)weight + (uintptr_t)H * e};
    Span outs[4];
    int nout = 0;
    outs[nout++] = {(uintptr_t)residual_out, (uintptr_t)residual_out + span_bytes(M, H, ld.rout, e)};
    if (out)
        outs[nout++] = {(uintptr_t)out, (uintptr_t)out + span_bytes(M, H, ld.out, e)};
    if (fp8) {
        const int qrow = quant == Q_MX ? H / 2 : H;
        uintptr_t sbytes = (uintptr_t)M * 4u;
        if (quant == Q_GROUP)
            sbytes = (uintptr_t)M * (uintptr_t)(H / ARRMS_FP8_GROUP_SIZE) * 4u;
        else if (quant == Q_MX)
            sbytes = (uintptr_t)M * (uintptr_t)(H / ARRMS_MX_BLOCK);
        outs[nout++] = {(uintptr_t)fp8_out, (uintptr_t)fp8_out + span_bytes(M, qrow, ld.q, 1)};
        outs[nout++] = {(uintptr_t)fp8_scale, (uintptr_t)fp8_scale + sbytes};
    }
    for (int o = 0; o < nout; ++o) {
        for (int i = 0; i < nin; ++i)
            if (overlaps(outs[o], ins[i]))
                return ARRMS_ERR_INVALID;
        const bool is_res_out = o == 0;
        if (!(is_res_out && inplace) && overlaps(outs[o], res_span))
            return ARRMS_ERR_INVALID;
        for (int p = o + 1; p < nout; ++p)
            if (overlaps(outs[o], outs[p]))
                return ARRMS_ERR_INVALID;
    }
    return ARRMS_OK;
}

int validate_sizes(int M, int H, int R, int flags)
{
    if (flags & ~kKnownFlags)
        return ARRMS_ERR_INVALID;
    const int dt = flags & ARRMS_DTYPE_MASK;
    if (dt > DT_FP32)
        return ARRMS_ERR_INVALID;
    if ((flags & ARRMS_FORCE_ONE_STAGE) && (flags & ARRMS_FORCE_TWO_STAGE))
        return ARRMS_ERR_INVALID;
    if (R < 1 || R > ARRMS_MAX_RANKS || M < 0 || H < 1)
        return ARRMS_ERR_INVALID;
    if (H > ARRMS_MAX_HIDDEN)
        return ARRMS_ERR_UNSUPPORTED;
    if ((flags & ARRMS_FP8) && dt == DT_FP32)
        return ARRMS_ERR_UNSUPPORTED;
    if (((long long)H * esize(dt)) % 16 != 0 || (long long)H * esize(dt) > ARRMS_MAX_ROW_BYTES)
        return ARRMS_ERR_UNSUPPORTED;
    return ARRMS_OK;
}

int choose_path(int M, int H, int R, int flags)
{
    (void)H;
    (void)R;
    if (M == 0)
        return ARRMS_PATH_NONE;
    if (flags & ARRMS_FORCE_TWO_STAGE)
        return ARRMS_PATH_TWO_STAGE;
    if (flags & ARRMS_FORCE_ONE_STAGE)
        return ARRMS_PATH_ONE_STAGE;
    // One GPU: the one-stage kernel moves the fewest bytes (R inputs + residual
    // in, two outputs); two-stage adds a staging write and read. Measured: at
    // none of the 324 points of the launch-shape sweep (rows 1-4096, hidden
    // 512-8192, 2/4/8 ranks, bf16 T output and fp16 per-token FP8) is it the
    // fastest; it takes 1.18 to 2.6 times the best one-stage launch.
    return ARRMS_PATH_ONE_STAGE;
}

// Row kernel launch shape by rule (the fallback of choose_shape below, and the
// shape of launches the measured table does not cover): packs per thread
// (PPT) in 1..4, threads per row tpr = the PPT-covering multiple of 64, at most 512. Exact cover first, then
// least padding, then more packs per thread (fewer, busier threads: measured
// faster on MI355X for large launches) as long as a thread's R+1 input packs
// stay within 20 (80 registers). Launches of fewer than 512 rows cap PPT at 2
// (more threads per row make up for the few rows), launches of fewer than 64
// rows of 513 to 1024 packs take one pack per thread (blocks of up to 1024
// threads), and the FP8 epilogue, with more per-element work after the row
// reduction, caps PPT at 3.
arrms::RowShape rule_shape(int P, int R, long long M, bool fp8, bool fp32)
{
    // fp32 kernels take blocks of up to 1024 threads at any PPT (rows of up to
    // 4096 packs); the others at one pack per thread only
    const int wide_block = fp32 ? 1024 : 512;
    arrms::RowShape best = {0, 0, 0, false, 0, 0, false};
    long long best_key = -1;
    int cap = fp8 ? 3 : 4;
    if (M < 512 && cap > 2)
        cap = 2;
    // a handful of wide rows (each on its own compute unit, latency-bound): one
    // pack per thread, the most waves per row (16 x 6144 bf16: 4.32 us against
    // 4.45-4.47 with two packs per thread; rows of at most 512 packs gain
    // nothing: 1 x 2880 and 64 x 2880 equal either way)
    if (M < 64 && P > 512 && P <= 1024)
        cap = 1;
    const int ppts[4] = {1, 2, 3, 4};
    for (int c = 0; c < 4; ++c) {
        const int ppt = ppts[c];
        if (ppt > cap)
            continue;
        if (ppt > 1 && ppt * (R + 1) > 20)
            continue;
        int tpr = (P + ppt - 1) / ppt;
        tpr = (tpr + 63) / 64 * 64;
        if (tpr > (cap == 1 ? 1024 : wide_block))  // one pack per thread: blocks of up to 1024
            continue;
        const int waste = tpr * ppt - P;
        const long long key = (long long)waste * 16 + (4 - ppt);
        if (best_key < 0 || key < best_key) {
            best_key = key;
            best = {ppt, tpr, 1, waste != 0, 0, 0, false};
        }
    }
    if (best.ppt == 0) {
        // wide rows with many ranks: the register budget gives way to coverage
        for (int c = 0; c < 4 && best.ppt == 0; ++c) {
            int tpr = (P + ppts[c] - 1) / ppts[c];
            tpr = (tpr + 63) / 64 * 64;
            if (tpr <= wide_block)
                best = {ppts[c], tpr, 1, tpr * ppts[c] != P, 0, 0, false};
        }
    }
    if (best.ppt == 0)
        return best;
    best.rpb = best.tpr >= 256 ? 1 : 256 / best.tpr;
    return best;
}

#include "dispatch_table.inc"

// Index of the grid value nearest to v on a log scale.
template <int N> int nearest_log(const int (&grid)[N], double v)
{
    const double lv = std::log2(v);
    int best = 0;
    double bd = 1e300;
    for (int i = 0; i < N; ++i) {
        const double d = std::fabs(std::log2((double)grid[i]) - lv);
        if (d < bd) {
            bd = d;
            best = i;
        }
    }
    return best;
}

// The measured launch shape: the dispatch table's entry (dispatch_table.inc,
// written by gen_dispatch_table.py from the launch-shape sweep that bench.py
// --sweep records on MI355X, profiles/dispatch_sweep_train.csv) at the grid
// point nearest to this launch -- kind of call (T output or a quantised
// output), ranks, packs per row and rows, each on a log scale. ppt == 0 when
// the entry's packs per thread cannot cover this row in one block.
arrms::RowShape measured_shape(int P, int R, long long M, bool quant, bool fp32)
{
    arrms::RowShape s = {0, 0, 0, false, 0, 0, false};
    const int v = kTab[quant ? 1 : 0][nearest_log(kTabR, R)][nearest_log(kTabP, P)][nearest_log(kTabM, (double)M)];
    const int ppt = v & 15, win = v >> 4;
    const int tpr = ((P + ppt - 1) / ppt + 63) / 64 * 64;
    if (ppt < 1 || ppt > 4 || win < 1 || win > 3 || tpr > ((ppt == 1 || fp32) ? 1024 : 512))
        return s;
    s = {ppt, tpr, tpr >= 256 ? 1 : 256 / tpr, tpr * ppt != P, 0, win, false};
    return s;
}

// Launch shape of a row-kernel launch (one-stage, and the two-stage row pass,
// which takes the one-stage shape of the whole launch so that both paths sum
// each row's squares in the same order): the measured shape, with its load
// window -- unless no table entry applies, or the row width is not one of the
// swept ones and the measured packs per thread would pad this row by more than
// a sixteenth beyond what the rule shape pads.
arrms::RowShape choose_shape(int P, int R, long long M, bool quant, bool fp32)
{
    const arrms::RowShape r = rule_shape(P, R, M, quant, fp32);
    const arrms::RowShape m = measured_shape(P, R, M, quant, fp32);
    if (m.ppt == 0)
        return r;
    const bool swept = kTabP[nearest_log(kTabP, P)] == P;
    if (!swept && r.ppt != 0 && (m.tpr * m.ppt - P) > (r.tpr * r.ppt - P) + P / 16)
        return r;
    return m;
}

hipError_t launch_row(int dt, int quant, bool mirror, const arrms::RowArgs &a, int R,
                      const arrms::RowShape &s, hipStream_t st)
{
    switch (dt) {
    case DT_BF16:
        switch (quant) {
        case Q_NONE: return arrms::launch_row_bf16_t(a, R, s, st);
        case Q_TOKEN:
            return mirror ? arrms::launch_row_bf16_fp8t(a, R, s, st) : arrms::launch_row_bf16_fp8(a, R, s, st);
        case Q_GROUP: return arrms::launch_row_bf16_fp8g(a, R, s, st);
        default: return arrms::launch_row_bf16_mx4(a, R, s, st);
        }
    case DT_FP16:
        switch (quant) {
        case Q_NONE: return arrms::launch_row_fp16_t(a, R, s, st);
        case Q_TOKEN:
            return mirror ? arrms::launch_row_fp16_fp8t(a, R, s, st) : arrms::launch_row_fp16_fp8(a, R, s, st);
        case Q_GROUP: return arrms::launch_row_fp16_fp8g(a, R, s, st);
        default: return arrms::launch_row_fp16_mx4(a, R, s, st);
        }
    default:
        return arrms::launch_row_fp32_t(a, R, s, st);
    }
}

int row_occupancy(int dt, int quant, bool mirror, int R, const arrms::RowShape &s)
{
    switch (dt) {
    case DT_BF16:
        switch (quant) {
        case Q_NONE: return arrms::occupancy_row_bf16_t(R, s);
        case Q_TOKEN: return mirror ? arrms::occupancy_row_bf16_fp8t(R, s) : arrms::occupancy_row_bf16_fp8(R, s);
        case Q_GROUP: return arrms::occupancy_row_bf16_fp8g(R, s);
        default: return arrms::occupancy_row_bf16_mx4(R, s);
        }
    case DT_FP16:
        switch (quant) {
        case Q_NONE: return arrms::occupancy_row_fp16_t(R, s);
        case Q_TOKEN: return mirror ? arrms::occupancy_row_fp16_fp8t(R, s) : arrms::occupancy_row_fp16_fp8(R, s);
        case Q_GROUP: return arrms::occupancy_row_fp16_fp8g(R, s);
        default: return arrms::occupancy_row_fp16_mx4(R, s);
        }
    default:
        return arrms::occupancy_row_fp32_t(R, s);
    }
}

// Compute units of the current device (cached per device; 0 if the runtime
// cannot tell).
int device_cus()
{
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 0;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// A launch is "large" when its input streams exceed 16 MiB: then the load
// window, not the size of the launch, sets how many bytes are in flight.
bool large_launch(int R, long long rows, int P) { return (long long)(R + 1) * rows * P * 16 > (16ll << 20); }

// Load window and occupancy cap of a row-kernel launch over `rows` rows of P
// packs with R input ranks, shape s; resident = blocks of this shape (narrow
// window) the device holds at once. An explicit window (s.window != 0) is kept.
//  * The narrow window when the whole launch is resident at once, it is large
//    and a row has at most 6 input streams; the wide window otherwise
//    (resident 1024 x 6144 bf16 rows: R = 5 17.8 us narrow, 19.0 wide; R = 6
//    21.4 narrow, 21.0 wide; R = 8 25.1 narrow, 24.7 wide).
//  * The occupancy cap (at most 16 waves per compute unit) for large
//    wide-window launches of 6 or more input streams per row that run in
//    several rounds of blocks: R = 5, 6, 7, 8 at 2048 x 7168 bf16 41.1 -> 39.6,
//    46.1 -> 44.3, 50.8 -> 48.9, 55.9 -> 54.3 us; R = 8 at 2048 x 6144 47.6 ->
//    46.6; R = 8 at 4096 x 4096 equal. With 5 streams it measured mixed (2800 x
//    6144 fp16 rows -0.1 us, 2048 x 7168 bf16 +0.25 us, the FP8 epilogue +0.2
//    us), so R <= 4 keeps the full occupancy.
void plan_window(arrms::RowShape &s, int R, long long rows, int P, long long resident)
{
    const long long groups = (rows + s.rpb - 1) / s.rpb;
    const long long grid = (s.grid > 0 && s.grid < groups) ? s.grid : groups;
    const bool large = large_launch(R, rows, P);
    if (s.window == 0)
        s.window = large && grid <= resident && R <= 5 ? 1 : 2;
    s.cap16 = s.window == 2 && large && grid > resident && R >= 5;
}

// Resident blocks of shape s on the current device (narrow-window kernel), or
// 0 when the launch is not large (the rules then do not need it).
long long resident_blocks(int dt, int quant, bool mirror, int R, long long rows, int P, const arrms::RowShape &s)
{
    if (!large_launch(R, rows, P))
        return 0;
    arrms::RowShape q = s;
    q.window = 1;
    return (long long)row_occupancy(dt, quant, mirror, R, q) * device_cus();
}

hipError_t launch_flat(int dt, const arrms::FlatArgs &a, int R, hipStream_t st)
{
    switch (dt) {
    case DT_BF16: return arrms::launch_flat_bf16(a, R, st);
    case DT_FP16: return arrms::launch_flat_fp16(a, R, st);
    default: return arrms::launch_flat_fp32(a, R, st);
    }
}

// ---- staging buffers: one per device, owned by the library (staging.hpp) ----
int staging_alloc(void **p, size_t bytes)
{
    if (hipMalloc(p, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return 0;
}

int staging_wait(void)
{
    if (hipDeviceSynchronize() != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return 0;
}

int staging_free(void *p)
{
    if (hipFree(p) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    return 0;
}

std::mutex g_staging_mu;
arrms::StagingPool<kMaxDevices> g_staging({staging_alloc, staging_wait, staging_free});

int reserve_locked(int dev, size_t bytes)
{
    return g_staging.reserve(dev, bytes) == 0 ? ARRMS_OK : ARRMS_ERR_HIP;
}

int current_device(int *dev)
{
    if (hipGetDevice(dev) != hipSuccess) {
        (void)hipGetLastError();
        return ARRMS_ERR_HIP;
    }
    if (*dev < 0 || *dev >= kMaxDevices)
        return ARRMS_ERR_HIP;
    return ARRMS_OK;
}

}  // namespace

extern "C" {

const char *arrms_status_string(int status)
{
    switch (status) {
    case ARRMS_OK: return "ok";
    case ARRMS_ERR_INVALID: return "invalid argument (pointer, size, flags or overlap)";
    case ARRMS_ERR_UNSUPPORTED:
        return "unsupported layout (alignment, H*sizeof(T) % 16, FP8 with fp32, row too wide)";
    case ARRMS_ERR_NO_STAGING: return "two-stage path inside stream capture without reserved staging";
    case ARRMS_ERR_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
    }
}

int arrms_query_path(int M, int H, int R, int flags)
{
    const int v = validate_sizes(M, H, R, flags);
    if (v != ARRMS_OK)
        return v;
    return choose_path(M, H, R, flags);
}

int arrms_reserve_staging(size_t bytes)
{
    int dev;
    int rc = current_device(&dev);
    if (rc != ARRMS_OK)
        return rc;
    if (bytes == 0)
        bytes = ARRMS_DEFAULT_STAGING_BYTES;
    std::lock_guard<std::mutex> lk(g_staging_mu);
    return reserve_locked(dev, bytes);
}

int arrms_release_staging(void)
{
    int dev;
    int rc = current_device(&dev);
    if (rc != ARRMS_OK)
        return rc;
    std::lock_guard<std::mutex> lk(g_staging_mu);
    return g_staging.release(dev) == 0 ? ARRMS_OK : ARRMS_ERR_HIP;
}

size_t arrms_staging_bytes(void)
{
    int dev;
    if (current_device(&dev) != ARRMS_OK)
        return 0;
    std::lock_guard<std::mutex> lk(g_staging_mu);
    return g_staging.bytes(dev);
}

}  // extern "C"

namespace {

struct ShapeReq {
    int ppt, tpr, rpb, grid, window;  // 0 = automatic
};

// Apply an explicit shape request on top of the automatic choice; returns
// false when the request cannot cover a row of P packs.
bool apply_shape(const ShapeReq *req, int P, int R, long long M, bool fp32, arrms::RowShape &s)
{
    (void)R;
    (void)M;
    if (!req)
        return true;
    if (req->ppt || req->tpr)
        s.window = 0;  // a window measured for another shape does not carry over
    if (req->ppt) {
        if (req->ppt < 1 || req->ppt > 4)
            return false;
        s.ppt = req->ppt;
        int tpr = (P + s.ppt - 1) / s.ppt;
        s.tpr = (tpr + 63) / 64 * 64;
    }
    if (req->tpr) {
        if (req->tpr % 64)
            return false;
        s.tpr = req->tpr;
    }
    // blocks of one pack per thread or of fp32 rows may hold 1024 threads, others 512
    const int max_block = (s.ppt == 1 || fp32) ? 1024 : 512;
    if ((long long)s.tpr * s.ppt < P || s.tpr > max_block)
        return false;
    s.tail = s.tpr * s.ppt != P;
    s.rpb = req->rpb ? req->rpb : (s.tpr >= 256 ? 1 : 256 / s.tpr);
    if (s.rpb < 1 || s.tpr * s.rpb > max_block)
        return false;
    s.grid = req->grid;
    if (req->window < 0 || req->window > 3)
        return false;
    if (req->window)
        s.window = req->window;
    return true;
}

int fused_impl(const void *const *rank_in, int R, const void *residual, const void *weight,
               void *out, void *residual_out, void *fp8_out, void *fp8_scale, int M, int H,
               float eps, int flags, const Strides &ld, const ShapeReq *req, hipStream_t stream,
               int quant, void *fixed_staging = nullptr, size_t fixed_staging_bytes = 0)
{
    int rc = validate(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H,
                      eps, flags, ld, quant);
    if (rc != ARRMS_OK)
        return rc;
    const int path = choose_path(M, H, R, flags);
    if (path == ARRMS_PATH_NONE)
        return ARRMS_OK;

    const int dt = flags & ARRMS_DTYPE_MASK;
    const int e = esize(dt);
    const int P = H * e / 16;
    const bool fp8 = quant != Q_NONE;  // any quantised output
    const int qgroups = quant == Q_GROUP ? H / ARRMS_FP8_GROUP_SIZE : quant == Q_MX ? H / ARRMS_MX_BLOCK : 1;
    const size_t scale_row = quant == Q_GROUP ? (size_t)qgroups * 4u : quant == Q_MX ? (size_t)qgroups : 4u;

    arrms::RowArgs a;
    memset(&a, 0, sizeof(a));
    a.residual = residual;
    a.weight = weight;
    a.out = out;
    a.residual_out = residual_out;
    a.fp8_out = fp8 ? fp8_out : nullptr;
    a.fp8_scale = quant == Q_TOKEN ? (float *)fp8_scale : nullptr;
    a.q_scale = (quant == Q_GROUP || quant == Q_MX) ? fp8_scale : nullptr;
    a.qgroups = qgroups;
    a.P = P;
    a.H = H;
    a.ld_in = ld.in * e;
    a.ld_res = ld.res * e;
    a.ld_out = ld.out * e;
    a.ld_rout = ld.rout * e;
    a.ld_q = ld.q;
    a.eps = eps;
    a.gemma = (flags & ARRMS_GEMMA) != 0;
    a.exact_only = (flags & ARRMS_EXACT_ONLY) != 0;

    (void)hipGetLastError();  // launches below report their own errors
    if (path == ARRMS_PATH_ONE_STAGE) {
        for (int r = 0; r < R; ++r)
            a.in[r] = rank_in[r];
        a.M = M;
        arrms::RowShape s = choose_shape(P, R, M, fp8, dt == DT_FP32);
        if (s.ppt == 0 || !apply_shape(req, P, R, M, dt == DT_FP32, s))
            return ARRMS_ERR_UNSUPPORTED;
        plan_window(s, R, M, P, resident_blocks(dt, quant, out != nullptr, R, M, P, s));
        a.tpr = s.tpr;
        return launch_row(dt, quant, out != nullptr, a, R, s, stream) == hipSuccess ? ARRMS_OK : ARRMS_ERR_HIP;
    }

    // ---- two-stage: per row chunk, flat rank reduce into staging, then the
    // row pass with the staging rows as its single input. The staging is the
    // library's buffer of the current device, or the caller's fixed region
    // (which never allocates).
    void *staging = fixed_staging;
    size_t staging_bytes = fixed_staging_bytes;
    if (!fixed_staging) {
        int dev;
        rc = current_device(&dev);
        if (rc != ARRMS_OK)
            return rc;
        std::lock_guard<std::mutex> lk(g_staging_mu);
        if (!g_staging.ptr(dev)) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
                (void)hipGetLastError();
                return ARRMS_ERR_HIP;
            }
            if (cs != hipStreamCaptureStatusNone)
                return ARRMS_ERR_NO_STAGING;
            rc = reserve_locked(dev, ARRMS_DEFAULT_STAGING_BYTES);
            if (rc != ARRMS_OK)
                return rc;
        }
        staging = g_staging.ptr(dev);
        staging_bytes = g_staging.bytes(dev);
    }
    const size_t row_bytes = (size_t)H * (size_t)e;
    const long long cap = (long long)(staging_bytes / row_bytes);  // rows the staging holds
    if (cap < 1)
        return fixed_staging ? ARRMS_ERR_UNSUPPORTED : ARRMS_ERR_NO_STAGING;
    // chunks of equal size (at most cap rows each): no small last chunk, whose
    // two launches would run a short, latency-bound round of blocks
    const long long nchunks = (M + cap - 1) / cap;
    const long long chunk = (M + nchunks - 1) / nchunks;
    for (long long m0 = 0; m0 < M; m0 += chunk) {
        const long long n = (M - m0) < chunk ? (M - m0) : chunk;
        arrms::FlatArgs f;
        memset(&f, 0, sizeof(f));
        for (int r = 0; r < R; ++r)
            f.in[r] = (const char *)rank_in[r] + (size_t)m0 * (size_t)a.ld_in;
        f.dst = staging;
        // contiguous inputs reduce as one flat run of packs, strided ones row by row
        if (ld.in == H) {
            f.rows = 1;
            f.P = n * P;
        } else {
            f.rows = n;
            f.P = P;
        }
        f.ld_in = a.ld_in / 16;
        f.ld_out = P;
        f.tiles = (f.P + arrms::kFlatTile - 1) / arrms::kFlatTile;
        if (launch_flat(dt, f, R, stream) != hipSuccess)
            return ARRMS_ERR_HIP;
        arrms::RowArgs b = a;
        b.in[0] = staging;
        b.ld_in = (long long)row_bytes;
        b.residual = (const char *)residual + (size_t)m0 * (size_t)a.ld_res;
        b.residual_out = (char *)residual_out + (size_t)m0 * (size_t)a.ld_rout;
        b.out = out ? (char *)out + (size_t)m0 * (size_t)a.ld_out : nullptr;
        if (fp8) {
            b.fp8_out = (char *)fp8_out + (size_t)m0 * (size_t)a.ld_q;
            if (quant == Q_TOKEN)
                b.fp8_scale = (float *)fp8_scale + m0;
            else
                b.q_scale = (char *)fp8_scale + (size_t)m0 * scale_row;
        }
        b.M = n;
        // the row pass takes the one-stage shape of the whole launch, so both paths
        // reduce the row statistics in the same order and give the same bits
        arrms::RowShape s = choose_shape(P, R, M, fp8, dt == DT_FP32);
        s.window = 0;  // the measured window is the one-stage launch's; the row pass takes the rule's
        if (s.ppt == 0 || !apply_shape(req, P, R, n, dt == DT_FP32, s))
            return ARRMS_ERR_UNSUPPORTED;
        plan_window(s, 1, n, P, resident_blocks(dt, quant, out != nullptr, 1, n, P, s));
        b.tpr = s.tpr;
        if (launch_row(dt, quant, out != nullptr, b, 1, s, stream) != hipSuccess)
            return ARRMS_ERR_HIP;
    }
    return ARRMS_OK;
}

}  // namespace

namespace arrms {

int fused_validate(const void *const *rank_in, int R, const void *residual, const void *weight, const void *out,
                   const void *residual_out, const void *fp8_out, const float *fp8_scale, int M, int H, float eps,
                   int flags)
{
    const Strides ld = {H, H, H, H, H};
    return validate(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, eps, flags, ld,
                    (flags & ARRMS_FP8) ? Q_TOKEN : Q_NONE);
}

int fused_fixed_staging(const void *const *rank_in, int R, const void *residual, const void *weight, void *out,
                        void *residual_out, void *fp8_out, float *fp8_scale, int M, int H, float eps, int flags,
                        void *staging, size_t staging_bytes, hipStream_t stream)
{
    const Strides ld = {H, H, H, H, H};
    return fused_impl(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, eps, flags, ld,
                      nullptr, stream, (flags & ARRMS_FP8) ? Q_TOKEN : Q_NONE, staging, staging_bytes);
}

}  // namespace arrms

extern "C" {

int arrms_fused(const void *const *rank_in, int R, const void *residual, const void *weight,
                void *out, void *residual_out, void *fp8_out, float *fp8_scale, int M, int H,
                float eps, int flags, hipStream_t stream)
{
    const Strides ld = {H, H, H, H, H};
    return fused_impl(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, eps,
                      flags, ld, nullptr, stream, (flags & ARRMS_FP8) ? Q_TOKEN : Q_NONE);
}

int arrms_fused_strided(const void *const *rank_in, int R, const void *residual, const void *weight,
                        void *out, void *residual_out, void *fp8_out, float *fp8_scale, int M, int H,
                        long long ld_in, long long ld_residual, long long ld_out,
                        long long ld_residual_out, long long ld_fp8, float eps, int flags,
                        hipStream_t stream)
{
    const Strides ld = {ld_in, ld_residual, ld_out, ld_residual_out, (flags & ARRMS_FP8) ? ld_fp8 : H};
    return fused_impl(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, eps,
                      flags, ld, nullptr, stream, (flags & ARRMS_FP8) ? Q_TOKEN : Q_NONE);
}

int arrms_fused_config(const void *const *rank_in, int R, const void *residual, const void *weight,
                       void *out, void *residual_out, void *fp8_out, float *fp8_scale, int M, int H,
                       float eps, int flags, int ppt, int tpr, int rows_per_block, int blocks,
                       int load_window, hipStream_t stream)
{
    if (ppt < 0 || tpr < 0 || rows_per_block < 0 || blocks < 0 || load_window < 0 || load_window > 3)
        return ARRMS_ERR_INVALID;
    const ShapeReq req = {ppt, tpr, rows_per_block, blocks, load_window};
    const Strides ld = {H, H, H, H, H};
    return fused_impl(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, eps,
                      flags, ld, &req, stream, (flags & ARRMS_FP8) ? Q_TOKEN : Q_NONE);
}

}  // extern "C"

namespace {

// arrms_query_launch / arrms_plan_launch: bpc < 0 asks the current device.
int plan_launch(int M, int H, int R, int flags, int quant, int mirror, int bpc, int cus, int *info)
{
    if (!info)
        return ARRMS_ERR_INVALID;
    if (flags & ARRMS_FP8) {
        if (quant != 0 && quant != ARRMS_QUANT_FP8_TOKEN)
            return ARRMS_ERR_INVALID;
        quant = ARRMS_QUANT_FP8_TOKEN;
        flags &= ~ARRMS_FP8;
    }
    if (quant < 0 || quant > ARRMS_QUANT_MXFP4)
        return ARRMS_ERR_INVALID;
    const int q = quant == 0 ? Q_NONE : quant == ARRMS_QUANT_FP8_TOKEN ? Q_TOKEN : quant == ARRMS_QUANT_FP8_GROUP ? Q_GROUP : Q_MX;
    int rc = validate_sizes(M, H, R, flags | (q != Q_NONE ? ARRMS_FP8 : 0));
    if (rc != ARRMS_OK)
        return rc;
    if ((q == Q_GROUP && H % ARRMS_FP8_GROUP_SIZE) || (q == Q_MX && H % ARRMS_MX_BLOCK))
        return ARRMS_ERR_UNSUPPORTED;
    for (int i = 0; i < ARRMS_LAUNCH_INFO; ++i)
        info[i] = 0;
    const int path = choose_path(M, H, R, flags);
    info[0] = path;
    if (path == ARRMS_PATH_NONE)
        return ARRMS_OK;
    const int dt = flags & ARRMS_DTYPE_MASK;
    const int e = esize(dt);
    const int P = H * e / 16;
    long long rows = M;
    int Rr = R;
    if (path == ARRMS_PATH_TWO_STAGE) {
        const long long cap = (long long)(ARRMS_DEFAULT_STAGING_BYTES / ((size_t)H * (size_t)e));
        const long long nchunks = (M + cap - 1) / cap;
        rows = (M + nchunks - 1) / nchunks;
        Rr = 1;
    }
    arrms::RowShape s = choose_shape(P, R, M, q != Q_NONE, dt == DT_FP32);
    if (s.ppt == 0)
        return ARRMS_ERR_UNSUPPORTED;
    if (path == ARRMS_PATH_TWO_STAGE)
        s.window = 0;
    long long resident;
    if (bpc < 0) {
        arrms::RowShape n = s;
        n.window = 1;
        bpc = row_occupancy(dt, q, mirror != 0, Rr, n);
        cus = device_cus();
        resident = resident_blocks(dt, q, mirror != 0, Rr, rows, P, s);
    } else {
        resident = large_launch(Rr, rows, P) ? (long long)bpc * cus : 0;
    }
    plan_window(s, Rr, rows, P, resident);
    info[1] = s.ppt;
    info[2] = s.tpr;
    info[3] = s.rpb;
    info[4] = s.window;
    info[5] = s.cap16 ? 1 : 0;
    info[6] = bpc;
    info[7] = cus;
    return ARRMS_OK;
}

}  // namespace

extern "C" {

int arrms_query_launch(int M, int H, int R, int flags, int quant, int mirror, int *info)
{
    return plan_launch(M, H, R, flags, quant, mirror, -1, 0, info);
}

int arrms_plan_launch(int M, int H, int R, int flags, int quant, int mirror, int blocks_per_cu, int cus, int *info)
{
    if (blocks_per_cu < 0 || cus < 0)
        return ARRMS_ERR_INVALID;
    return plan_launch(M, H, R, flags, quant, mirror, blocks_per_cu, cus, info);
}

int arrms_fused_quant(const void *const *rank_in, int R, const void *residual, const void *weight,
                      void *out, void *residual_out, void *q_out, void *q_scale, int M, int H, float eps,
                      int flags, int quant, hipStream_t stream)
{
    if (quant < ARRMS_QUANT_FP8_TOKEN || quant > ARRMS_QUANT_MXFP4 || (flags & ARRMS_FP8))
        return ARRMS_ERR_INVALID;
    const int q = quant == ARRMS_QUANT_FP8_TOKEN ? Q_TOKEN : quant == ARRMS_QUANT_FP8_GROUP ? Q_GROUP : Q_MX;
    const Strides ld = {H, H, H, H, q == Q_MX ? H / 2 : H};
    return fused_impl(rank_in, R, residual, weight, out, residual_out, q_out, q_scale, M, H, eps,
                      q == Q_TOKEN ? (flags | ARRMS_FP8) : flags, ld, nullptr, stream, q);
}

int arrms_allreduce_sum(const void *const *rank_in, int R, void *out, long long n, int flags,
                        hipStream_t stream)
{
    if (flags & ~ARRMS_DTYPE_MASK)
        return ARRMS_ERR_INVALID;
    const int dt = flags & ARRMS_DTYPE_MASK;
    if (dt > DT_FP32 || R < 1 || R > ARRMS_MAX_RANKS || n < 0 || !rank_in || !out)
        return ARRMS_ERR_INVALID;
    if (n > kMaxSpanBytes / esize(dt))
        return ARRMS_ERR_INVALID;
    for (int r = 0; r < R; ++r)
        if (!rank_in[r])
            return ARRMS_ERR_INVALID;
    const int e = esize(dt);
    if ((n * e) % 16 != 0)
        return ARRMS_ERR_UNSUPPORTED;
    if (!aligned16(out))
        return ARRMS_ERR_UNSUPPORTED;
    for (int r = 0; r < R; ++r)
        if (!aligned16(rank_in[r]))
            return ARRMS_ERR_UNSUPPORTED;
    if (n == 0)
        return ARRMS_OK;
    // the output may be one of the inputs exactly (in place), nothing else
    const uintptr_t bytes = (uintptr_t)n * (uintptr_t)e;
    const Span o = {(uintptr_t)out, (uintptr_t)out + bytes};
    for (int r = 0; r < R; ++r) {
        const Span i = {(uintptr_t)rank_in[r], (uintptr_t)rank_in[r] + bytes};
        if (rank_in[r] != out && overlaps(o, i))
            return ARRMS_ERR_INVALID;
    }
    arrms::FlatArgs f;
    memset(&f, 0, sizeof(f));
    for (int r = 0; r < R; ++r)
        f.in[r] = rank_in[r];
    f.dst = out;
    f.rows = 1;
    f.P = n * e / 16;
    f.ld_in = f.P;
    f.ld_out = f.P;
    f.tiles = (f.P + arrms::kFlatTile - 1) / arrms::kFlatTile;
    (void)hipGetLastError();
    return launch_flat(dt, f, R, stream) == hipSuccess ? ARRMS_OK : ARRMS_ERR_HIP;
}

}  // extern "C"
