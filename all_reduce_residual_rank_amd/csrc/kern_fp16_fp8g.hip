// kern_fp16_fp8g.hip -- row kernels for T = fp16 with the per-group FP8 output (scale per 128 columns).
#include "kernels.hpp"

namespace arrms {

hipError_t launch_row_fp16_fp8g(const RowArgs &a, int R, const RowShape &s, hipStream_t st)
{
    return row_launch_epi<DT_FP16, EPI_FP8G>(a, R, s, st);
}

int occupancy_row_fp16_fp8g(int R, const RowShape &s)
{
    return row_occupancy_epi<DT_FP16, EPI_FP8G>(R, s);
}

}  // namespace arrms
