// kern_fp16_mx4.hip -- row kernels for T = fp16 with the MXFP4 output (E8M0 scale per 32 columns, E2M1 codes).
#include "kernels.hpp"

namespace arrms {

hipError_t launch_row_fp16_mx4(const RowArgs &a, int R, const RowShape &s, hipStream_t st)
{
    return row_launch_epi<DT_FP16, EPI_MX4>(a, R, s, st);
}

int occupancy_row_fp16_mx4(int R, const RowShape &s)
{
    return row_occupancy_epi<DT_FP16, EPI_MX4>(R, s);
}

}  // namespace arrms
