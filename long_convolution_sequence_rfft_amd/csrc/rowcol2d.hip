// rowcol2d.hip -- placeholder until the row-column kernels land.
#include <hip/hip_runtime.h>
#include "plan.h"
namespace hy {
hyena_status launch_rowcol2d_spectrum(const Plan&, const void*, void*, void*, void*)
{ return fail(HYENA_ERR_UNSUPPORTED, "ROWCOL2D not built"); }
hyena_status launch_rowcol2d_forward(const Plan&, const void*, const void* const*, const void*,
                                     const float*, void*, void*, void*)
{ return fail(HYENA_ERR_UNSUPPORTED, "ROWCOL2D not built"); }
hyena_status launch_rowcol2d_export(const Plan&, const void*, void*, void*)
{ return fail(HYENA_ERR_UNSUPPORTED, "ROWCOL2D not built"); }
}
