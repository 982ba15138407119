// fourstep.hip -- placeholder until the four-step kernels land.
#include <hip/hip_runtime.h>
#include "plan.h"
namespace hy {
hyena_status launch_fourstep_spectrum(const Plan&, const void*, void*, void*, void*)
{ return fail(HYENA_ERR_UNSUPPORTED, "FOURSTEP1D not built"); }
hyena_status launch_fourstep_forward(const Plan&, const void*, const void* const*, const void*,
                                     const float*, void*, void*, void*)
{ return fail(HYENA_ERR_UNSUPPORTED, "FOURSTEP1D not built"); }
hyena_status launch_fourstep_export(const Plan&, const void*, void*, void*)
{ return fail(HYENA_ERR_UNSUPPORTED, "FOURSTEP1D not built"); }
}
