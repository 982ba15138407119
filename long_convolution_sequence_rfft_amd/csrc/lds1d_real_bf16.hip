// lds1d_real_bf16.hip -- bfloat16 storage instantiations of the single-channel
// kernels (bfloat16 or float32 spectrum).
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_INSTANTIATE, uint16_t, uint16_t)
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_INSTANTIATE, uint16_t, float)
}  // namespace hy
