// lds1d_circ_f16.hip -- periodic-boundary single-channel kernels, f16 storage.
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_REAL_SIZES(HY_LDS1D_CIRC_INSTANTIATE, _Float16, float)
}  // namespace hy
