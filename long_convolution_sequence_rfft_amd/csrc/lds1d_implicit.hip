// lds1d_implicit.hip -- single-channel spectrum kernels that evaluate the
// implicit filter's taps on the fly (all storage types).
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_REAL_SIZES(HY_LDS1D_IMPLICIT_INSTANTIATE, float, float)
HY_LDS1D_REAL_SIZES(HY_LDS1D_IMPLICIT_INSTANTIATE, uint16_t, uint16_t)
HY_LDS1D_REAL_SIZES(HY_LDS1D_IMPLICIT_INSTANTIATE, uint16_t, float)
HY_LDS1D_REAL_SIZES(HY_LDS1D_IMPLICIT_INSTANTIATE, _Float16, float)
}  // namespace hy
