// kern_fp32_t.hip -- row kernels for T = fp32 with the T output, and the flat rank reduce.
#include "kernels.hpp"

namespace arrms {

hipError_t launch_row_fp32_t(const RowArgs &a, int R, const RowShape &s, hipStream_t st)
{
    return row_launch_epi<DT_FP32, EPI_T>(a, R, s, st);
}

int occupancy_row_fp32_t(int R, const RowShape &s)
{
    return row_occupancy_epi<DT_FP32, EPI_T>(R, s);
}

hipError_t launch_flat_fp32(const FlatArgs &a, int R, hipStream_t st)
{
    return flat_launch<DT_FP32>(a, R, st);
}

}  // namespace arrms
