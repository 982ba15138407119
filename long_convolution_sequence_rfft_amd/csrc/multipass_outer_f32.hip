// multipass_outer_f32.hip -- float32-storage instantiations of the outer passes.
#include "multipass_kernels.h"

namespace hy {
HY_MP_LENGTHS(HY_MP_OUTER_INST, float, )
}  // namespace hy
