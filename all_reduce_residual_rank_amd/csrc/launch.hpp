// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernel
// translation units (kern_<dtype>_<epilogue>.hip, one per dtype and epilogue).
// Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arrms {

enum Dtype { DT_BF16 = 0, DT_FP16 = 1, DT_FP32 = 2 };

constexpr int kMaxRanks = 8;
constexpr int kMaxDevices = 64;
constexpr int kMaxWavesPerBlock = 16;  // row kernel blocks are at most 1024 threads

// Arguments of the row kernel (one-stage, and stage 2 of two-stage with R = 1
// and the staging buffer as its only input). Pointers are to 16-byte packs.
struct RowArgs {
    const void *in[kMaxRanks];
    const void *residual;
    const void *weight;
    void *out;            // may be null when fp8 is set (no T mirror)
    void *residual_out;
    void *fp8_out;        // bytes: E4M3 [M][H], or packed E2M1 [M][H/2]
    float *fp8_scale;     // per-token FP8: [M]
    void *q_scale;        // per-group FP8: fp32 [M][qgroups]; MXFP4: E8M0 bytes [M][qgroups]
    int qgroups;          // quant groups per row (H / 128 or H / 32)
    long long M;          // rows
    int P;                // 16-byte packs per row
    // row strides in bytes: rank inputs, residual, out, residual_out, fp8 codes
    long long ld_in, ld_res, ld_out, ld_rout, ld_q;
    int H;                // elements per row
    int tpr;              // threads per row group (multiple of 64)
    int rpb;              // row groups per block (set by the launcher)
    long long groups;     // row groups in all, ceil(M / rpb) (set by the launcher)
    float eps;
    int gemma;
    int exact_only;
};

// Arguments of the flat rank reduce (stage 1 of two-stage, and the plain rank
// all-reduce).
// The reduced region is rows x P packs: row m of rank r starts at pack
// m * ld_in of in[r] and lands at pack m * ld_out of dst. Contiguous data is
// one row of all its packs.
struct FlatArgs {
    const void *in[kMaxRanks];
    void *dst;
    long long rows;
    long long P;          // packs per row
    long long ld_in;      // row stride of the inputs, in packs
    long long ld_out;     // row stride of dst, in packs
    long long tiles;      // tiles per row (ceil(P / kFlatTile))
};

// Row kernel shape: PPT packs per thread per row, tpr threads per row,
// rpb rows side by side per block; tail = tpr * PPT > packs per row. grid is
// the number of blocks: 0 (or at least the number of row groups) gives one
// block per group of rpb rows; fewer blocks each take every grid-th group in
// turn. window: phase-1 load window, 1 narrow, 2 wide, 3 medium (0 while the
// plan is open: the launch needs one of 1..3). cap16: hold at most 16 waves
// per compute unit (an LDS reservation the kernel does not use).
struct RowShape {
    int ppt;
    int tpr;
    int rpb;
    bool tail;
    int grid;
    int window;
    bool cap16;
};

constexpr int kFlatThreads = 256;
constexpr int kFlatPacksPerThread = 2;
constexpr int kFlatWindow = 2;  // 16-byte loads in flight per thread
constexpr int kFlatTile = kFlatThreads * kFlatPacksPerThread;

// Row kernels, one entry per dtype and epilogue (kern_<dtype>_<epilogue>.hip):
// _t writes the T output, _fp8 the per-token FP8 output only, _fp8t per-token
// FP8 plus the T mirror, _fp8g per-group FP8 and _mx4 MXFP4 (each with the T
// mirror when out is set).
hipError_t launch_row_bf16_t(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_bf16_fp8(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_bf16_fp8t(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_fp16_t(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_fp16_fp8(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_fp16_fp8t(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_fp32_t(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_bf16_fp8g(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_bf16_mx4(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_fp16_fp8g(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
hipError_t launch_row_fp16_mx4(const RowArgs &a, int R, const RowShape &s, hipStream_t st);
// The argument checks of arrms_fused alone (api.cpp): ARRMS_OK or its error status.
int fused_validate(const void *const *rank_in, int R, const void *residual, const void *weight, const void *out,
                   const void *residual_out, const void *fp8_out, const float *fp8_scale, int M, int H, float eps,
                   int flags);

// arrms_fused with a caller-provided staging region for the two-stage path
// (api.cpp): nothing is allocated; rows are chunked to fit staging_bytes.
int fused_fixed_staging(const void *const *rank_in, int R, const void *residual, const void *weight, void *out,
                        void *residual_out, void *fp8_out, float *fp8_scale, int M, int H, float eps, int flags,
                        void *staging, size_t staging_bytes, hipStream_t stream);

// Blocks of the row kernel of that shape (its tpr * rpb threads and its load
// window) that one compute unit of the current device holds; 0 if the runtime
// cannot tell. Cached per device.
int occupancy_row_bf16_fp8(int R, const RowShape &s);
int occupancy_row_bf16_fp8g(int R, const RowShape &s);
int occupancy_row_bf16_fp8t(int R, const RowShape &s);
int occupancy_row_bf16_mx4(int R, const RowShape &s);
int occupancy_row_bf16_t(int R, const RowShape &s);
int occupancy_row_fp16_fp8(int R, const RowShape &s);
int occupancy_row_fp16_fp8g(int R, const RowShape &s);
int occupancy_row_fp16_fp8t(int R, const RowShape &s);
int occupancy_row_fp16_mx4(int R, const RowShape &s);
int occupancy_row_fp16_t(int R, const RowShape &s);
int occupancy_row_fp32_t(int R, const RowShape &s);
hipError_t launch_flat_bf16(const FlatArgs &a, int R, hipStream_t st);
hipError_t launch_flat_fp16(const FlatArgs &a, int R, hipStream_t st);
hipError_t launch_flat_fp32(const FlatArgs &a, int R, hipStream_t st);

}  // namespace arrms
