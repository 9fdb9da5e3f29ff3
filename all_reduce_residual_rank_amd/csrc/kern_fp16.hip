// kern_fp16.hip -- instantiates the row and flat kernels for T = fp16.
#include "kernels.hpp"

namespace arrms {

hipError_t launch_row_fp16(const RowArgs &a, int R, const RowShape &s, hipStream_t st)
{
    return row_launch<DT_FP16>(a, R, s, st);
}

hipError_t launch_flat_fp16(const FlatArgs &a, int R, hipStream_t st)
{
    return flat_launch<DT_FP16>(a, R, st);
}

}  // namespace arrms
