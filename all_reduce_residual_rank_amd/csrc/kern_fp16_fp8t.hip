// kern_fp16_fp8t.hip -- row kernels for T = fp16 with the FP8 output with the T mirror.
#include "kernels.hpp"

namespace arrms {

hipError_t launch_row_fp16_fp8t(const RowArgs &a, int R, const RowShape &s, hipStream_t st)
{
    return row_launch_epi<DT_FP16, EPI_FP8_T>(a, R, s, st);
}

int occupancy_row_fp16_fp8t(int R, const RowShape &s)
{
    return row_occupancy_epi<DT_FP16, EPI_FP8_T>(R, s);
}

}  // namespace arrms
