// multipass_outer_f32.hip -- float32-storage instantiations of the outer passes.
#include "multipass_kernels.h"

namespace hy {
HY_MP_OUTER_LENGTHS(HY_MP_OUTER_INST, float, )
HY_MP_OUTER_CIRC_LENGTHS(HY_MP_OUTER_CIRC_INST, float, )
HY_MP_OUTER_IMP_LENGTHS(HY_MP_OUTER_IMP_INST, 0, )
}  // namespace hy
