// lds1d_real_f16.hip -- _Float16 storage instantiations of the single-channel
// kernels (float32 spectrum).
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_INSTANTIATE, _Float16, float)
}  // namespace hy
