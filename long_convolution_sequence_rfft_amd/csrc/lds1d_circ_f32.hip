// lds1d_circ_f32.hip -- periodic-boundary single-channel kernels, f32 storage.
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_REAL_SIZES(HY_LDS1D_CIRC_INSTANTIATE, float, float)
}  // namespace hy
