// lds1d_bf16.hip -- bfloat16 storage instantiations (bfloat16 or float32 spectrum).
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_SIZES(HY_LDS1D_INSTANTIATE, uint16_t, uint16_t)
HY_LDS1D_SIZES(HY_LDS1D_INSTANTIATE, uint16_t, float)
}  // namespace hy
