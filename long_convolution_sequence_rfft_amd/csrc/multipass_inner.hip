// multipass_inner.hip -- instantiations of the inner passes (float32 and
// bfloat16 spectra).
#include "multipass_kernels.h"

namespace hy {
HY_MP_INNER_LENGTHS(HY_MP_INNER_INST, float, )
HY_MP_INNER_LENGTHS(HY_MP_INNER_INST, uint16_t, )
}  // namespace hy
