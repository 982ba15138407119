// lds1d_real_f32.hip -- float32 storage instantiations of the single-channel
// kernels of the single-workgroup path.
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_INSTANTIATE, float, float)
}  // namespace hy
