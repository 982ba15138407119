// api.hip -- the extern "C" entry points declared in include/hyena.h.
// Validation happens here, before anything is enqueued; the launchers in
// lds1d.hip, multipass.hip and implicit.hip only enqueue kernels.
#include <hip/hip_runtime.h>

#include <new>

#include "plan.h"

namespace hy {
const char* last_error_text();
}

struct hyena_plan_s {
    hy::Plan p;
};

using hy::fail;

namespace {

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

size_t io_bytes(const hy::Plan& p)
{
    return (size_t)p.B * (size_t)p.N * (size_t)p.d * (p.io_dtype == HYENA_F32 ? 4u : 2u);
}

size_t filter_bytes(const hy::Plan& p)
{
    size_t taps = (size_t)p.N;
    if (p.ndims == 2) taps = (size_t)(2 * p.X - 1) * (size_t)(2 * p.Y - 1);
    if (p.ndims == 3) taps = (size_t)(2 * p.X - 1) * (size_t)(2 * p.Y - 1) * (size_t)(2 * p.Z - 1);
    return (size_t)p.order * (size_t)p.d * taps * (p.io_dtype == HYENA_F32 ? 4u : 2u);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Last check before a call enqueues work that uses the workspace: it must
// hold this plan's tables (recorded by hyena_workspace_init and not released,
// overwritten by another plan's initialisation, or overlapped by another
// plan's intermediates since).
hyena_status check_ws(const hy::Plan& p, const void* ws)
{
    if (ws == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (!aligned16(ws)) return fail(HYENA_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
    if (!hy::ws_record_use(ws, p.workspace_bytes, p.token))
        return fail(HYENA_ERR_WORKSPACE,
                    "workspace does not hold this plan's tables: call hyena_workspace_init "
                    "(it was never initialised for this plan, was released, or another plan "
                    "has initialised or used memory overlapping it since)");
    return HYENA_OK;
}

}  // namespace

extern "C" {

hyena_status hyena_plan_create_ex(hyena_plan_t* plan, int64_t B, int64_t N, int64_t d,
                                  int32_t order, const int64_t* dims, int32_t ndims,
                                  int32_t io_dtype, int32_t spectrum_dtype, int32_t path,
                                  int32_t flags)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan output pointer is NULL");
    hyena_plan_s* s = new (std::nothrow) hyena_plan_s;
    if (s == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "out of host memory");
    const hyena_status st =
        hy::plan_build(s->p, B, N, d, order, dims, ndims, io_dtype, spectrum_dtype, path, flags);
    if (st != HYENA_OK) {
        delete s;
        return st;
    }
    *plan = s;
    return HYENA_OK;
}

hyena_status hyena_plan_create(hyena_plan_t* plan, int64_t B, int64_t N, int64_t d,
                               int32_t order, const int64_t* dims, int32_t ndims,
                               int32_t io_dtype, int32_t spectrum_dtype)
{
    return hyena_plan_create_ex(plan, B, N, d, order, dims, ndims, io_dtype, spectrum_dtype,
                                HYENA_PATH_AUTO, 0);
}

hyena_status hyena_plan_query(hyena_plan_t plan, size_t* spectrum_bytes, size_t* workspace_bytes)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (spectrum_bytes) *spectrum_bytes = plan->p.spectrum_bytes;
    if (workspace_bytes) *workspace_bytes = plan->p.workspace_bytes;
    return HYENA_OK;
}

hyena_status hyena_plan_path(hyena_plan_t plan, int32_t* path)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (path == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "path is NULL");
    *path = plan->p.path;
    return HYENA_OK;
}

hyena_status hyena_workspace_init(hyena_plan_t plan, void* workspace, void* stream)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (workspace == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (!aligned16(workspace))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "workspace is not 16-byte aligned");
    const hyena_status st = hy::launch_tw_init(plan->p, workspace, stream);
    if (st != HYENA_OK) return st;
    hy::ws_record_init(workspace, plan->p.workspace_bytes, plan->p.token);
    return HYENA_OK;
}

hyena_status hyena_workspace_release(hyena_plan_t plan, void* workspace)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (workspace == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    hy::ws_record_release(workspace, plan->p.token);
    return HYENA_OK;
}

hyena_status hyena_filter_spectrum(hyena_plan_t plan, const void* h, void* H, void* workspace,
                                   void* stream)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    const hy::Plan& p = plan->p;
    if (h == nullptr || H == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "h or H is NULL");
    if (!aligned16(h) || !aligned16(H))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "h and H must be 16-byte aligned");
    if (overlaps(h, filter_bytes(p), H, p.spectrum_bytes))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "H overlaps h");
    if (overlaps(workspace, p.workspace_bytes, H, p.spectrum_bytes))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "H overlaps the workspace");
    const hyena_status st = check_ws(p, workspace);
    if (st != HYENA_OK) return st;
    switch (p.path) {
        case HYENA_PATH_LDS1D: return hy::launch_lds1d_spectrum(p, h, H, workspace, stream);
        case HYENA_PATH_FOURSTEP1D: return hy::launch_fourstep_spectrum(p, h, H, workspace, stream);
        case HYENA_PATH_ROWCOL2D: return hy::launch_rowcol2d_spectrum(p, h, H, workspace, stream);
        case HYENA_PATH_ROWCOL3D: return hy::launch_rowcol3d_spectrum(p, h, H, workspace, stream);
        default: return fail(HYENA_ERR_UNSUPPORTED, "unknown path");
    }
}

}  // extern "C"

namespace hy {

// Argument checks of hyena_forward other than the workspace record; `ws` is
// the workspace the call will use (its first workspace_bytes bytes).
hyena_status check_forward_args(const Plan& p, const void* u, const void* const* gates,
                                const void* H, const float* D, const void* y, const void* ws)
{
    if (u == nullptr || gates == nullptr || H == nullptr || D == nullptr || y == nullptr)
        return fail(HYENA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (!aligned16(u) || !aligned16(H) || !aligned16(D) || !aligned16(y))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "u, H, D and y must be 16-byte aligned");
    const size_t nio = io_bytes(p);
    const size_t nD = (size_t)p.order * (size_t)p.d * 4u;
    for (int n = 0; n < p.order; ++n) {
        if (gates[n] == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "a gate pointer is NULL");
        if (!aligned16(gates[n]))
            return fail(HYENA_ERR_INVALID_ARGUMENT, "gate pointers must be 16-byte aligned");
        if (overlaps(y, nio, gates[n], nio))
            return fail(HYENA_ERR_INVALID_ARGUMENT, "y overlaps a gate");
    }
    if (overlaps(y, nio, u, nio)) return fail(HYENA_ERR_INVALID_ARGUMENT, "y overlaps u");
    if (overlaps(y, nio, H, p.spectrum_bytes)) return fail(HYENA_ERR_INVALID_ARGUMENT, "y overlaps H");
    if (overlaps(y, nio, D, nD)) return fail(HYENA_ERR_INVALID_ARGUMENT, "y overlaps D");
    if (overlaps(y, nio, ws, p.workspace_bytes))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "y overlaps the workspace");
    return HYENA_OK;
}

// Enqueue the whole chain (arguments already checked).
hyena_status run_forward(const Plan& p, const void* u, const void* const* gates, const void* H,
                         const float* D, void* y, void* ws, void* stream)
{
    switch (p.path) {
        case HYENA_PATH_LDS1D: return launch_lds1d_forward(p, u, gates, H, D, y, ws, stream);
        case HYENA_PATH_FOURSTEP1D: return launch_fourstep_forward(p, u, gates, H, D, y, ws, stream);
        case HYENA_PATH_ROWCOL2D: return launch_rowcol2d_forward(p, u, gates, H, D, y, ws, stream);
        case HYENA_PATH_ROWCOL3D: return launch_rowcol3d_forward(p, u, gates, H, D, y, ws, stream);
        default: return fail(HYENA_ERR_UNSUPPORTED, "unknown path");
    }
}

const Plan* plan_of(hyena_plan_t plan) { return plan ? &plan->p : nullptr; }

}  // namespace hy

extern "C" {

hyena_status hyena_forward(hyena_plan_t plan, const void* u, const void* const* gates,
                           const void* H, const float* D, void* y, void* workspace, void* stream)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    const hy::Plan& p = plan->p;
    hyena_status st = hy::check_forward_args(p, u, gates, H, D, y, workspace);
    if (st != HYENA_OK) return st;
    st = check_ws(p, workspace);
    if (st != HYENA_OK) return st;
    return hy::run_forward(p, u, gates, H, D, y, workspace, stream);
}

hyena_status hyena_nd_mixer_forward(hyena_plan_t plan, const hyena_nd_mixer* m, const void* H,
                                    const float* D, void* y, void* workspace, void* stream)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    const hy::Plan& p = plan->p;
    if ((p.ndims != 2 && p.ndims != 3) || p.order != 1)
        return fail(HYENA_ERR_UNSUPPORTED, "the HyenaND mixer needs an ndims = 2 or 3, order 1 plan");
    if (m == nullptr || m->q == nullptr || m->k == nullptr || m->v == nullptr ||
        m->short_w == nullptr || H == nullptr || D == nullptr || y == nullptr)
        return fail(HYENA_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (!aligned16(m->q) || !aligned16(m->k) || !aligned16(m->v) || !aligned16(H) ||
        !aligned16(D) || !aligned16(y))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "q, k, v, H, D and y must be 16-byte aligned");
    const size_t nio = io_bytes(p);
    if (overlaps(y, nio, m->q, nio) || overlaps(y, nio, m->k, nio) || overlaps(y, nio, m->v, nio))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "y overlaps q, k or v");
    if (overlaps(y, nio, H, p.spectrum_bytes)) return fail(HYENA_ERR_INVALID_ARGUMENT, "y overlaps H");
    if (overlaps(y, nio, D, (size_t)p.d * 4u)) return fail(HYENA_ERR_INVALID_ARGUMENT, "y overlaps D");
    if (overlaps(y, nio, workspace, p.workspace_bytes))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "y overlaps the workspace");
    const hyena_status st = check_ws(p, workspace);
    if (st != HYENA_OK) return st;
    if (p.ndims == 3) return hy::launch_rowcol3d_block(p, *m, H, D, y, workspace, stream);
    return hy::launch_rowcol2d_block(p, *m, H, D, y, workspace, stream);
}

hyena_status hyena_implicit_scratch_bytes(hyena_plan_t plan, int32_t hidden, size_t* bytes)
{
    if (plan == nullptr || bytes == nullptr)
        return fail(HYENA_ERR_INVALID_ARGUMENT, "plan or output pointer is NULL");
    if (plan->p.ndims != 1) return fail(HYENA_ERR_UNSUPPORTED, "implicit filters need ndims = 1");
    if (hidden < 1 || hidden > 256)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: hidden must be in 1..256");
    *bytes = hy::implicit_scratch_bytes(plan->p, hidden);
    return HYENA_OK;
}

hyena_status hyena_filter_spectrum_implicit(hyena_plan_t plan, const hyena_implicit_filter* f,
                                            void* H, void* workspace, void* scratch, void* stream)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    const hy::Plan& p = plan->p;
    if (p.ndims != 1) return fail(HYENA_ERR_UNSUPPORTED, "implicit filters need ndims = 1");
    if (f == nullptr || H == nullptr || scratch == nullptr)
        return fail(HYENA_ERR_INVALID_ARGUMENT, "filter description, H or scratch is NULL");
    if (f->W1 == nullptr || f->b1 == nullptr || f->W2 == nullptr || f->b2 == nullptr ||
        f->W3 == nullptr || f->b3 == nullptr || f->alpha == nullptr)
        return fail(HYENA_ERR_INVALID_ARGUMENT, "an implicit-filter weight pointer is NULL");
    if (f->n_freqs < 0 || f->n_freqs > 64)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: n_freqs must be in 0..64");
    if (f->hidden < 1 || f->hidden > 256)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: hidden must be in 1..256");
    if (!aligned16(H) || !aligned16(scratch))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "H and scratch must be 16-byte aligned");
    const size_t nscratch = hy::implicit_scratch_bytes(p, f->hidden);
    if (overlaps(H, p.spectrum_bytes, scratch, nscratch))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "H overlaps the scratch");
    if (overlaps(workspace, p.workspace_bytes, H, p.spectrum_bytes))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "H overlaps the workspace");
    if (overlaps(workspace, p.workspace_bytes, scratch, nscratch))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "the scratch overlaps the workspace");
    const hyena_status st = check_ws(p, workspace);
    if (st != HYENA_OK) return st;
    return hy::launch_implicit_spectrum(p, *f, H, workspace, scratch, stream);
}

hyena_status hyena_spectrum_export(hyena_plan_t plan, const void* H, void* natural, void* stream)
{
    if (plan == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (H == nullptr || natural == nullptr)
        return fail(HYENA_ERR_INVALID_ARGUMENT, "H or output is NULL");
    if (!aligned16(H) || !aligned16(natural))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "H and output must be 16-byte aligned");
    const hy::Plan& p = plan->p;
    switch (p.path) {
        case HYENA_PATH_LDS1D: return hy::launch_lds1d_export(p, H, natural, stream);
        case HYENA_PATH_FOURSTEP1D: return hy::launch_fourstep_export(p, H, natural, stream);
        case HYENA_PATH_ROWCOL2D: return hy::launch_rowcol2d_export(p, H, natural, stream);
        case HYENA_PATH_ROWCOL3D: return hy::launch_rowcol3d_export(p, H, natural, stream);
        default: return fail(HYENA_ERR_UNSUPPORTED, "unknown path");
    }
}

hyena_status hyena_plan_destroy(hyena_plan_t plan)
{
    if (plan != nullptr) {
        hy::ws_record_drop(plan->p.token);
        hy::log_msg("plan %llu destroyed", (unsigned long long)plan->p.token);
    }
    delete plan;
    return HYENA_OK;
}

const char* hyena_status_string(hyena_status status)
{
    switch (status) {
        case HYENA_OK: return "HYENA_OK";
        case HYENA_ERR_INVALID_ARGUMENT: return "HYENA_ERR_INVALID_ARGUMENT";
        case HYENA_ERR_UNSUPPORTED: return "HYENA_ERR_UNSUPPORTED";
        case HYENA_ERR_WORKSPACE: return "HYENA_ERR_WORKSPACE";
        case HYENA_ERR_DEVICE: return "HYENA_ERR_DEVICE";
        default: return "HYENA_ERR_UNKNOWN";
    }
}

const char* hyena_last_error(void) { return hy::last_error_text(); }

}  // extern "C"
