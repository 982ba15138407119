// multipass_outer_f16.hip -- _Float16-storage instantiations of the outer passes.
#include "multipass_kernels.h"

namespace hy {
HY_MP_LENGTHS(HY_MP_OUTER_INST, _Float16, )
}  // namespace hy
