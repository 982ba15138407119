// lds1d_f16.hip -- _Float16 storage instantiations of the channel-pair
// single-workgroup kernels (float32 spectrum).
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_SIZES(HY_LDS1D_INSTANTIATE, _Float16, float)
}  // namespace hy
