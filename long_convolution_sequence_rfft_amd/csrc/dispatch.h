// dispatch.h -- run a generic launcher for a plan's storage types.
#pragma once

#include "plan.h"

namespace hy {

template <typename T>
struct type_tag {
    using type = T;
};

// f(type_tag<IO>{}, type_tag<SP>{}) for the plan's io and spectrum storage:
// (float, float), (bfloat16 bits, bfloat16 bits), (bfloat16 bits, float) or
// (_Float16, float).
template <typename F>
hyena_status by_storage(const Plan& p, F&& f)
{
    if (p.io_dtype == HYENA_F32) return f(type_tag<float>{}, type_tag<float>{});
    if (p.io_dtype == HYENA_F16) return f(type_tag<_Float16>{}, type_tag<float>{});
    if (p.spec_dtype == HYENA_BF16) return f(type_tag<uint16_t>{}, type_tag<uint16_t>{});
    return f(type_tag<uint16_t>{}, type_tag<float>{});
}

}  // namespace hy
