// Launch entry points of the kernel translation units, replaced by functions
// that launch nothing: the argument sweep exercises the C ABI's host code
// (checks, shape choice, chunking) under the sanitizers without a GPU.
#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace arrms {
#define ARRMS_STUB_ROW(name) \
    hipError_t name(const RowArgs &, int, const RowShape &, hipStream_t) { return hipSuccess; }
ARRMS_STUB_ROW(launch_row_bf16_t)
ARRMS_STUB_ROW(launch_row_bf16_fp8)
ARRMS_STUB_ROW(launch_row_bf16_fp8t)
ARRMS_STUB_ROW(launch_row_fp16_t)
ARRMS_STUB_ROW(launch_row_fp16_fp8)
ARRMS_STUB_ROW(launch_row_fp16_fp8t)
ARRMS_STUB_ROW(launch_row_fp32_t)
ARRMS_STUB_ROW(launch_row_bf16_fp8g)
ARRMS_STUB_ROW(launch_row_bf16_mx4)
ARRMS_STUB_ROW(launch_row_fp16_fp8g)
ARRMS_STUB_ROW(launch_row_fp16_mx4)
hipError_t launch_flat_bf16(const FlatArgs &, int, hipStream_t) { return hipSuccess; }
hipError_t launch_flat_fp16(const FlatArgs &, int, hipStream_t) { return hipSuccess; }
hipError_t launch_flat_fp32(const FlatArgs &, int, hipStream_t) { return hipSuccess; }
}  // namespace arrms
