// Launch entry points of the kernel translation units, replaced by functions
// that launch nothing: the argument sweep exercises the C ABI's host code
// (checks, shape choice, chunking) under the sanitizers without a GPU.
#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace arrms {
// occupancy: a fixed 4 blocks per compute unit, so that the launch planner runs
#define ARRMS_STUB_ROW(name) \
    hipError_t launch_row_##name(const RowArgs &, int, const RowShape &s, hipStream_t) \
    { return s.window >= 1 && s.window <= 3 ? hipSuccess : hipErrorInvalidValue; } \
    int occupancy_row_##name(int, const RowShape &) { return 4; }
ARRMS_STUB_ROW(bf16_t)
ARRMS_STUB_ROW(bf16_fp8)
ARRMS_STUB_ROW(bf16_fp8t)
ARRMS_STUB_ROW(fp16_t)
ARRMS_STUB_ROW(fp16_fp8)
ARRMS_STUB_ROW(fp16_fp8t)
ARRMS_STUB_ROW(fp32_t)
ARRMS_STUB_ROW(bf16_fp8g)
ARRMS_STUB_ROW(bf16_mx4)
ARRMS_STUB_ROW(fp16_fp8g)
ARRMS_STUB_ROW(fp16_mx4)
hipError_t launch_flat_bf16(const FlatArgs &, int, hipStream_t) { return hipSuccess; }
hipError_t launch_flat_fp16(const FlatArgs &, int, hipStream_t) { return hipSuccess; }
hipError_t launch_flat_fp32(const FlatArgs &, int, hipStream_t) { return hipSuccess; }
}  // namespace arrms
