// lds1d_circ_bf16.hip -- periodic-boundary single-channel kernels, bf16 storage.
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_REAL_SIZES(HY_LDS1D_CIRC_INSTANTIATE, uint16_t, uint16_t)
HY_LDS1D_REAL_SIZES(HY_LDS1D_CIRC_INSTANTIATE, uint16_t, float)
}  // namespace hy
