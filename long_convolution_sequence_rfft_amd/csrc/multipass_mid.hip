// multipass_mid.hip -- instantiations of the middle passes of 3D grids
// (transforms along y between the two intermediates).
#include "multipass_kernels.h"

namespace hy {
HY_MP_LENGTHS(HY_MP_MID_INST, 0, )
}  // namespace hy
