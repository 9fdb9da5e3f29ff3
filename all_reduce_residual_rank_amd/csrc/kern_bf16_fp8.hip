// kern_bf16_fp8.hip -- row kernels for T = bf16 with the FP8 output (no T mirror).
#include "kernels.hpp"

namespace arrms {

hipError_t launch_row_bf16_fp8(const RowArgs &a, int R, const RowShape &s, hipStream_t st)
{
    return row_launch_epi<DT_BF16, EPI_FP8>(a, R, s, st);
}

int occupancy_row_bf16_fp8(int R, const RowShape &s)
{
    return row_occupancy_epi<DT_BF16, EPI_FP8>(R, s);
}

}  // namespace arrms
