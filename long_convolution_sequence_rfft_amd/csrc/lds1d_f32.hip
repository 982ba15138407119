// lds1d_f32.hip -- float32 storage instantiations of the single-workgroup path.
#include "lds1d_kernels.h"

namespace hy {
HY_LDS1D_SIZES(HY_LDS1D_INSTANTIATE, float, float)
}  // namespace hy
