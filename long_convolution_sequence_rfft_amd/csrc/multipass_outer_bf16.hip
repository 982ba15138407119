// multipass_outer_bf16.hip -- bfloat16-storage instantiations of the outer passes.
#include "multipass_kernels.h"

namespace hy {
HY_MP_LENGTHS(HY_MP_OUTER_INST, uint16_t, )
}  // namespace hy
