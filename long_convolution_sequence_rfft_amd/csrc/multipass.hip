// multipass.hip -- launch side of the four-step (1D, transforms longer than
// 16384 points, or forced) and row-column (2D and 3D) paths: chunk loop over
// channel pairs, per-length dispatch, and the spectrum export.
#include "multipass_kernels.h"

namespace hy {

HY_MP_OUTER_LENGTHS(HY_MP_OUTER_INST, float, extern)
HY_MP_OUTER_LENGTHS(HY_MP_OUTER_INST, uint16_t, extern)
HY_MP_OUTER_LENGTHS(HY_MP_OUTER_INST, _Float16, extern)
HY_MP_OUTER_CIRC_LENGTHS(HY_MP_OUTER_CIRC_INST, float, extern)
HY_MP_OUTER_CIRC_LENGTHS(HY_MP_OUTER_CIRC_INST, uint16_t, extern)
HY_MP_OUTER_CIRC_LENGTHS(HY_MP_OUTER_CIRC_INST, _Float16, extern)
HY_MP_OUTER_IMP_LENGTHS(HY_MP_OUTER_IMP_INST, 0, extern)
HY_MP_INNER_LENGTHS(HY_MP_INNER_INST, float, extern)
HY_MP_INNER_LENGTHS(HY_MP_INNER_INST, uint16_t, extern)
HY_MP_LENGTHS(HY_MP_MID_INST, 0, extern)

namespace {

int threads_per_transform(int L) { return L / lds1d_pts(L); }

// ---------------------------------------------------------------------------
// Chunks on two streams.  A chain that walks two or more chunks of channel
// pairs runs the odd chunks on a second stream with their own copy of the
// intermediate buffer, so one chunk's passes overlap the other's (an inner
// pass beside an outer one, each pass's tail beside the next one's start).
// The second stream forks from the caller's stream with an event and joins
// it again with another, so the call stays ordered on the caller's stream
// and can be captured into a graph.  Measured: 64K tokens at width 768 (two
// chunks) 1345-1361 -> 1270-1278 us, the 64^3 grid at width 64 1138-1149 ->
// 1076-1094 us; holding the second chunk back by one pass, so that inner and
// outer passes pair up, was no faster.  Stream and events are created on first
// use, one set per host thread and device (a plan may serve several threads
// at once), at default priority, and kept until the process ends.  Under
// graph capture, where creating them is not allowed, a thread that has none
// yet runs its chunks on the caller's stream alone.
// ---------------------------------------------------------------------------
struct SideStream {
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};

struct Fork {
    hipStream_t caller = nullptr;
    SideStream* ss = nullptr;  // null: one stream
    hipStream_t stream_of(int64_t chunk) const { return ss && (chunk & 1) ? ss->side : caller; }
    int copy_of(int64_t chunk) const { return ss ? (int)(chunk & 1) : 0; }
};

constexpr int kMaxForkDevices = 64;
thread_local int t_single_stream = 0;  // SingleStreamScope depth

hyena_status fork_begin(const Plan& p, hipStream_t s, Fork& f)
{
    f.caller = s;
    f.ss = nullptr;
    if (p.inter_copies < 2 || t_single_stream > 0) return HYENA_OK;
    thread_local SideStream per_dev[kMaxForkDevices];
    int dev = 0;
    hipError_t e = s != nullptr ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxForkDevices) return HYENA_OK;
    SideStream& ss = per_dev[dev];
    if (ss.side == nullptr) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
            return HYENA_OK;
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
        SideStream n;
        e = hipStreamCreateWithFlags(&n.side, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess) return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
        ss = n;
        log_msg("second stream %p for device %d on this thread", (void*)ss.side, dev);
    }
    if ((e = hipEventRecord(ss.fork, s)) != hipSuccess ||
        (e = hipStreamWaitEvent(ss.side, ss.fork, 0)) != hipSuccess)
        return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
    f.ss = &ss;
    return HYENA_OK;
}

// Joins the second stream back into the caller's (also after a failed launch,
// so nothing the call enqueued is left unordered); returns st, or the join's
// own failure.
hyena_status fork_end(const Fork& f, hyena_status st)
{
    if (f.ss == nullptr) return st;
    hipError_t e = hipEventRecord(f.ss->join, f.ss->side);
    if (e == hipSuccess) e = hipStreamWaitEvent(f.caller, f.ss->join, 0);
    if (e != hipSuccess && st == HYENA_OK) return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
    return st;
}

TwOffsets offsets_at(const Plan& p, int first)
{
    TwOffsets o;
    o.f1 = (int32_t)p.seg[first + 0].off;
    o.fL = (int32_t)p.seg[first + 1].off;
    o.i1 = (int32_t)p.seg[first + 2].off;
    o.i0 = (int32_t)p.seg[first + 3].off;
    return o;
}

// Pairs per outer workgroup: up to 16 (a 128-byte row of float32 pairs), and
// no more than the workgroup's transforms of the outer length g.La.
void set_pair_groups(const Plan& p, MpGeom& g)
{
    const int nf = kMpThreads / threads_per_transform(g.La);
    const int kp_max = nf < 16 ? nf : 16;
    int kp = 1;
    while (kp < kp_max && kp < p.npairs) kp <<= 1;
    g.kp_log2 = 0;
    while ((1 << g.kp_log2) < kp) ++g.kp_log2;
    g.groups_per_b = (int32_t)((p.npairs + kp - 1) / kp);
}

// Geometry common to all passes of a plan (chunk fields filled per launch).
MpGeom base_geom(const Plan& p)
{
    MpGeom g{};
    g.N = p.N;
    g.d = p.d;
    g.npairs = p.npairs;
    g.B = p.B;
    g.four_step = p.path == HYENA_PATH_FOURSTEP1D;
    g.full = p.circular;
    if (g.four_step) {
        g.La = (int32_t)p.M1;
        g.Lb = (int32_t)p.M2;
        g.Lb_live = (int32_t)p.M2;
        g.sa = p.M2;  // t = M2 n1 + n2
        g.so = 1;
        g.tw_step = p.seg[8].off;
    } else {
        g.La = (int32_t)p.P2;
        g.Lb = (int32_t)p.P1;
        g.Lb_live = (int32_t)p.X;
        g.sa = 1;  // t = Y p + q
        g.so = p.Y;
        g.tw_step = 0;
    }
    set_pair_groups(p, g);
    g.tw_a = offsets_at(p, 0);
    g.tw_b = offsets_at(p, 4);
    return g;
}

template <typename IO>
hyena_status outer_go(int L, int mode, bool half_spec, const OuterArgs& a, int64_t nb, hipStream_t s)
{
    const bool paired = a.g.three_d == 0;
    switch (L) {
#define HY_CASE(LL, A_, B_)                                                                        \
    case LL:                                                                                       \
        if (mode == OUTER_SPEC_IMP) {                                                              \
            if constexpr (LL >= 32 && LL <= 1024)                                               \
                return mp_outer_launch<LL, float, OUTER_SPEC_IMP, true, true>(a, nb, s);          \
            return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: four-step columns below 32");    \
        }                                                                                          \
        if (mode == OUTER_IN3) return mp_outer_launch<LL, IO, OUTER_IN3, true, false>(a, nb, s);   \
        if (mode == OUTER_OUT3) return mp_outer_launch<LL, IO, OUTER_OUT3, true, false>(a, nb, s); \
        if (a.g.full && (mode == OUTER_IN || mode == OUTER_MID || mode == OUTER_OUT)) {           \
            if constexpr (LL == 512 || LL == 1024) {                                               \
                if (mode == OUTER_IN) return mp_outer_launch<LL, IO, OUTER_IN, false, true>(a, nb, s);   \
                if (mode == OUTER_MID) return mp_outer_launch<LL, IO, OUTER_MID, false, true>(a, nb, s); \
                return mp_outer_launch<LL, IO, OUTER_OUT, false, true>(a, nb, s);                  \
            }                                                                                      \
            return fail(HYENA_ERR_UNSUPPORTED, "multi-pass: no periodic columns of this length");  \
        }                                                                                          \
        if (paired) {                                                                              \
            if (mode == OUTER_IN) return mp_outer_launch<LL, IO, OUTER_IN, true, true>(a, nb, s);   \
            if (mode == OUTER_MID) return mp_outer_launch<LL, IO, OUTER_MID, true, true>(a, nb, s); \
            if (mode == OUTER_OUT) return mp_outer_launch<LL, IO, OUTER_OUT, true, true>(a, nb, s); \
            if (half_spec) return mp_outer_launch<LL, IO, OUTER_SPEC, true, true>(a, nb, s);        \
            return mp_outer_launch<LL, IO, OUTER_SPEC, false, true>(a, nb, s);                      \
        }                                                                                          \
        if (mode == OUTER_IN) return mp_outer_launch<LL, IO, OUTER_IN, true, false>(a, nb, s);     \
        if (mode == OUTER_MID) return mp_outer_launch<LL, IO, OUTER_MID, true, false>(a, nb, s);   \
        if (mode == OUTER_OUT) return mp_outer_launch<LL, IO, OUTER_OUT, true, false>(a, nb, s);   \
        if (!half_spec) return mp_outer_launch<LL, IO, OUTER_SPEC, false, false>(a, nb, s);        \
        return fail(HYENA_ERR_UNSUPPORTED, "multi-pass: no half-input spectrum pass on 3D grids");
        HY_MP_OUTER_LENGTHS(HY_CASE, 0, 0)
#undef HY_CASE
        default: return fail(HYENA_ERR_UNSUPPORTED, "multi-pass: unsupported outer length");
    }
}

template <typename SP>
hyena_status inner_go(int L, int mode, bool half_b, const InnerArgs& a, int64_t nb, hipStream_t s)
{
    switch (L) {
#define HY_CASE(LL, A_, B_)                                                                   \
    case LL:                                                                                  \
        if (mode == INNER_SPEC) return mp_inner_launch<LL, SP, INNER_SPEC, false>(a, nb, s);  \
        if (half_b) return mp_inner_launch<LL, SP, INNER_CHAIN, true>(a, nb, s);              \
        return mp_inner_launch<LL, SP, INNER_CHAIN, false>(a, nb, s);
        HY_MP_INNER_LENGTHS(HY_CASE, 0, 0)
#undef HY_CASE
        default: return fail(HYENA_ERR_UNSUPPORTED, "multi-pass: unsupported inner length");
    }
}

hyena_status outer(const Plan& p, int mode, bool half_spec, const OuterArgs& a, int64_t nb,
                   hipStream_t s)
{
    if (p.io_dtype == HYENA_F32) return outer_go<float>(a.g.La, mode, half_spec, a, nb, s);
    if (p.io_dtype == HYENA_F16) return outer_go<_Float16>(a.g.La, mode, half_spec, a, nb, s);
    return outer_go<uint16_t>(a.g.La, mode, half_spec, a, nb, s);
}

hyena_status inner(const Plan& p, int mode, const InnerArgs& a, int64_t nb, hipStream_t s)
{
    const bool half_b = !a.g.four_step;
    // the inner kernels size their tile loops from (LB, HALF_B)
    if (mode == INNER_CHAIN && a.g.Lb_live != (half_b ? a.g.Lb / 2 : a.g.Lb))
        return fail(HYENA_ERR_UNSUPPORTED, "multi-pass: live inner rows do not match the kernel");
    return p.spec_dtype == HYENA_F32 ? inner_go<float>(a.g.Lb, mode, half_b, a, nb, s)
                                     : inner_go<uint16_t>(a.g.Lb, mode, half_b, a, nb, s);
}

size_t io_size(const Plan& p) { return p.io_dtype == HYENA_F32 ? 4 : 2; }

// SP elements of one filter's spectrum
int64_t spec_elems_per_filter(const Plan& p)
{
    return p.npairs * p.spec_entries_per_pair * kEntryElems;
}

hyena_status mp_forward_chunks(const Plan& p, const void* u, const void* const* gates,
                               const void* H, const float* D, void* y, void* ws, const Fork& fk,
                               const BlockArgs* blk)
{
    MpGeom g = base_geom(p);
    const int KP = 1 << g.kp_log2;
    const int C = (kMpThreads / threads_per_transform(g.La)) / KP;
    const int U = (kMpThreads / threads_per_transform(g.Lb)) / 2;
    const int64_t col_blocks = (g.Lb_live + C - 1) / C;
    const int64_t unit_blocks = (g.La / 2 + U - 1) / U;
    const int64_t total_groups = (int64_t)p.B * g.groups_per_b;
    int64_t chunk_groups = p.chunk_pairs / KP;
    if (chunk_groups < 1) chunk_groups = 1;
    const float2* tw = static_cast<const float2*>(ws);
    const size_t esz = p.spec_dtype == HYENA_F32 ? 4 : 2;
    g.pair_bytes = p.fwd_pair_bytes;
    for (int64_t g0 = 0, ci = 0; g0 < total_groups; g0 += chunk_groups, ++ci) {
        const hipStream_t s = fk.stream_of(ci);
        float2* F = reinterpret_cast<float2*>(static_cast<char*>(ws) + p.fwd_offset[fk.copy_of(ci)]);
        g.group0 = g0;
        g.ngroups = total_groups - g0 < chunk_groups ? total_groups - g0 : chunk_groups;
        OuterArgs oa{};
        oa.g = g;
        oa.act = u;
        oa.F = F;
        oa.tw = tw;
        if (blk) oa.blk = *blk;
        hyena_status st = outer(p, OUTER_IN, true, oa, col_blocks * g.ngroups, s);
        if (st != HYENA_OK) return st;
        for (int n = 0; n < p.order; ++n) {
            InnerArgs ia{};
            ia.g = g;
            ia.F = F;
            ia.spec = static_cast<const char*>(H) + (size_t)n * spec_elems_per_filter(p) * esz;
            ia.D = D + (int64_t)n * p.d;
            ia.tw = tw;
            st = inner(p, INNER_CHAIN, ia, unit_blocks * g.ngroups * KP, s);
            if (st != HYENA_OK) return st;
            oa.act = blk ? nullptr : gates[n];
            oa.out = y;
            st = outer(p, n + 1 < p.order ? OUTER_MID : OUTER_OUT, true, oa, col_blocks * g.ngroups, s);
            if (st != HYENA_OK) return st;
        }
    }
    return HYENA_OK;
}

hyena_status mp_forward(const Plan& p, const void* u, const void* const* gates, const void* H,
                        const float* D, void* y, void* ws, void* stream,
                        const BlockArgs* blk = nullptr)
{
    Fork fk;
    const hyena_status st = fork_begin(p, (hipStream_t)stream, fk);
    if (st != HYENA_OK) return st;
    return fork_end(fk, mp_forward_chunks(p, u, gates, H, D, y, ws, fk, blk));
}

// imp != nullptr: the taps are evaluated from an implicit filter's hidden
// features (four-step path) instead of read from h.
// The filter spectrum walks the same chunks over the whole intermediate
// area of the workspace (every copy the forward chain uses).  With two
// copies it splits the area in two and alternates chunks between the two
// streams, as the chain does, when each half holds at least one group of
// the spectrum's (larger) rows.
hyena_status mp_spectrum_chunks(const Plan& p, const void* h, void* H, void* ws, const Fork& fk,
                                size_t region, const ImpOuter* imp)
{
    MpGeom g = base_geom(p);
    g.B = 1;  // filters have no batch axis
    const int KP = 1 << g.kp_log2;
    const int C = (kMpThreads / threads_per_transform(g.La)) / KP;
    const int U = (kMpThreads / threads_per_transform(g.Lb)) / 2;
    const int64_t col_blocks = (g.Lb + C - 1) / C;
    const int64_t unit_blocks = (g.La / 2 + U - 1) / U;
    const int64_t total_groups = g.groups_per_b;
    int64_t chunk_groups = (int64_t)(region / (size_t)(p.spec_pair_bytes * KP));
    if (chunk_groups < 1) chunk_groups = 1;  // the plan sizes copy 0 for one group at least
    const float2* tw = static_cast<const float2*>(ws);
    const size_t esz = p.spec_dtype == HYENA_F32 ? 4 : 2;
    const int64_t taps = p.ndims == 1 ? p.N : (2 * p.X - 1) * (2 * p.Y - 1);
    g.pair_bytes = p.spec_pair_bytes;
    int64_t ci = 0;
    for (int n = 0; n < p.order; ++n) {
        for (int64_t g0 = 0; g0 < total_groups; g0 += chunk_groups, ++ci) {
            const hipStream_t s = fk.stream_of(ci);
            float2* F = reinterpret_cast<float2*>(static_cast<char*>(ws) + p.inter_offset +
                                                  (size_t)fk.copy_of(ci) * region);
            g.group0 = g0;
            g.ngroups = total_groups - g0 < chunk_groups ? total_groups - g0 : chunk_groups;
            OuterArgs oa{};
            oa.g = g;
            if (imp) {
                oa.imp = *imp;
                oa.imp.n = n;
            } else {
                oa.filt = static_cast<const char*>(h) + (size_t)n * p.d * taps * io_size(p);
            }
            oa.F = F;
            oa.tw = tw;
            hyena_status st = outer(p, imp ? OUTER_SPEC_IMP : OUTER_SPEC,
                                    g.four_step != 0 && !g.full, oa, col_blocks * g.ngroups, s);
            if (st != HYENA_OK) return st;
            InnerArgs ia{};
            ia.g = g;
            ia.F = F;
            ia.spec_out = static_cast<char*>(H) + (size_t)n * spec_elems_per_filter(p) * esz;
            ia.tw = tw;
            st = inner(p, INNER_SPEC, ia, unit_blocks * g.ngroups * KP, s);
            if (st != HYENA_OK) return st;
        }
    }
    return HYENA_OK;
}

hyena_status mp_spectrum(const Plan& p, const void* h, void* H, void* ws, void* stream,
                         const ImpOuter* imp = nullptr)
{
    // the intermediate area: copy 0 and the chain's further copies after it
    const size_t area = p.workspace_bytes - p.stage_bytes - p.inter_offset;
    const int KP = 1 << base_geom(p).kp_log2;
    const size_t group = (size_t)p.spec_pair_bytes * (size_t)KP;
    Fork fk;
    if (p.inter_copies == 2 && area / 2 / 256 * 256 >= group) {
        const hyena_status st = fork_begin(p, (hipStream_t)stream, fk);
        if (st != HYENA_OK) return st;
    } else {
        fk.caller = (hipStream_t)stream;
    }
    const size_t region = fk.ss ? area / 2 / 256 * 256 : area;
    return fork_end(fk, mp_spectrum_chunks(p, h, H, ws, fk, region, imp));
}

// One thread per entry (n, pair, unit kk, e); writes natural-order unscaled
// transfer functions.  1D: [order][d][M/2 + 1]; 2D: [order][d][P1][P2/2 + 1].
template <typename SP>
__global__ void hyena_mp_export(const SP* spec, float2* out, int64_t npairs, int64_t d, int La,
                                int Lb, int four_step, int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t per_pair = (int64_t)(La / 2) * Lb;
    const int64_t np = i / per_pair;
    const int64_t rem = i - np * per_pair;
    const int kk = (int)(rem / Lb), e = (int)(rem % Lb);
    const int64_t n = np / npairs, p = np - n * npairs;
    const int64_t c0 = 2 * p;
    const bool has_b = c0 + 1 < d;
    float2 P, Q;
    load_entry(spec, i, P, Q);
    const float M = (float)La * (float)Lb;
    const float2 ha = make_float2((P.x + Q.x) * M, (P.y + Q.y) * M);
    const float2 hb = make_float2((P.x - Q.x) * M, (P.y - Q.y) * M);
    if (four_step) {
        const int64_t Mtot = (int64_t)La * Lb, half = Mtot / 2;
        float2* oa = out + (n * d + c0) * (half + 1);
        float2* ob = oa + (half + 1);
        auto put = [&](int64_t k, float2 va, float2 vb) {
            if (k > half) {
                k = Mtot - k;
                va.y = -va.y;
                vb.y = -vb.y;
            }
            oa[k] = va;
            if (has_b) ob[k] = vb;
        };
        if (kk > 0) {
            put(kk + (int64_t)La * e, ha, hb);
        } else if (e == 0) {
            put(0, make_float2(ha.x, 0.0f), make_float2(hb.x, 0.0f));
            put(half, make_float2(ha.y, 0.0f), make_float2(hb.y, 0.0f));
        } else if (e < Lb / 2) {
            put((int64_t)La * e, ha, hb);
        } else {
            put(La / 2 + (int64_t)La * (e - Lb / 2), ha, hb);
        }
    } else {
        const int W = La / 2 + 1;  // kq = 0 .. P2/2
        float2* oa = out + (n * d + c0) * (int64_t)Lb * W;
        float2* ob = oa + (int64_t)Lb * W;
        auto put = [&](int kp, int kq, float2 va, float2 vb) {
            oa[(int64_t)kp * W + kq] = va;
            if (has_b) ob[(int64_t)kp * W + kq] = vb;
        };
        auto conj2 = [](float2 v) { return make_float2(v.x, -v.y); };
        if (kk > 0) {
            put(e, kk, ha, hb);
        } else if (e == 0 || e == Lb / 2) {
            const int kq = e == 0 ? 0 : La / 2;
            put(0, kq, make_float2(ha.x, 0.0f), make_float2(hb.x, 0.0f));
            put(Lb / 2, kq, make_float2(ha.y, 0.0f), make_float2(hb.y, 0.0f));
        } else {
            const int kq = e < Lb / 2 ? 0 : La / 2;
            const int kp = e < Lb / 2 ? e : e - Lb / 2;
            put(kp, kq, ha, hb);
            put(Lb - kp, kq, conj2(ha), conj2(hb));
        }
    }
}

hyena_status mp_export(const Plan& p, const void* H, void* out, void* stream)
{
    const MpGeom g = base_geom(p);
    const int64_t total = (int64_t)p.order * p.npairs * p.spec_entries_per_pair;
    const int bs = 256;
    const int64_t nb = (total + bs - 1) / bs;
    if (p.spec_dtype == HYENA_F32)
        HY_LAUNCH(kernel_label("hyena_mp_export", "float"), hyena_mp_export<float>, dim3((unsigned)nb),
                  dim3(bs), 0, (hipStream_t)stream, (const float*)H, (float2*)out, p.npairs, p.d,
                           g.La, g.Lb, g.four_step, total);
    else
        HY_LAUNCH(kernel_label("hyena_mp_export", "unsigned short"), hyena_mp_export<uint16_t>,
                  dim3((unsigned)nb), dim3(bs), 0, (hipStream_t)stream, (const uint16_t*)H, (float2*)out, p.npairs, p.d,
                           g.La, g.Lb, g.four_step, total);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// 3D grids: outer pass along z (rows (x, y), intermediate F1), middle pass
// along y (F1 <-> F2), inner pass along x on F2 with the composite outer
// index (ky, kz).
// ---------------------------------------------------------------------------
MpGeom base_geom3(const Plan& p)
{
    MpGeom g{};
    g.N = p.N;
    g.d = p.d;
    g.npairs = p.npairs;
    g.B = p.B;
    g.four_step = 0;
    g.three_d = 1;
    g.La = (int32_t)p.P3;
    g.Lb = (int32_t)(p.P1 * p.P2);  // rows (x, y) of the filter spectrum
    g.Lb_live = (int32_t)(p.X * p.Y);  // rows (x, y) of the chain
    g.sa = 1;  // t = Z (x Y + y) + z
    g.so = p.Z;
    g.tw_step = 0;
    g.gx = (int32_t)p.X;
    g.gy = (int32_t)p.Y;
    g.gz = (int32_t)p.Z;
    set_pair_groups(p, g);
    g.tw_a = offsets_at(p, 0);
    g.tw_b = offsets_at(p, 4);
    return g;
}

MpGeom geom3_inner(const Plan& p, const MpGeom& go)
{
    MpGeom g = go;
    g.La = (int32_t)(p.P2 * p.P3);
    g.Lb = (int32_t)p.P1;
    g.Lb_live = (int32_t)p.X;
    g.Lc = (int32_t)p.P3;
    return g;
}

hyena_status mid(int LY, int mode, bool half, const MidArgs& a, int64_t nb, hipStream_t s)
{
    switch (LY) {
#define HY_CASE(LL, A_, B_)                                                          \
    case LL:                                                                         \
        if (mode == MID_INV) return mp_mid_launch<LL, MID_INV, true>(a, nb, s);      \
        if (half) return mp_mid_launch<LL, MID_FWD, true>(a, nb, s);                 \
        return mp_mid_launch<LL, MID_FWD, false>(a, nb, s);
        HY_MP_LENGTHS(HY_CASE, 0, 0)
#undef HY_CASE
        default: return fail(HYENA_ERR_UNSUPPORTED, "multi-pass: unsupported middle length");
    }
}

MidArgs mid_args(const Plan& p, const MpGeom& g, float2* F1, float2* F2, bool spec, int mode,
                 const float2* tw)
{
    MidArgs m{};
    m.src = mode == MID_FWD ? F1 : F2;
    m.dst = mode == MID_FWD ? F2 : F1;
    m.tw = tw;
    m.tw_y = offsets_at(p, 8);
    m.f1_pair = (spec ? p.spec_pair_bytes : p.fwd_pair_bytes) / 8;
    m.f2_pair = (spec ? p.spec_pair_bytes2 : p.fwd_pair_bytes2) / 8;
    m.ncols = (spec ? p.P1 : p.X) * p.P3;
    m.nslots = g.ngroups * ((int64_t)1 << g.kp_log2);
    m.P3 = (int32_t)p.P3;
    m.ylen1 = (int32_t)(spec ? p.P2 : p.Y);
    return m;
}

int64_t mid_blocks(const Plan& p, const MidArgs& m)
{
    const int64_t nf = kMpThreads / threads_per_transform((int)p.P2);
    return (m.ncols + nf - 1) / nf * m.nslots;
}

hyena_status mp3_forward_chunks(const Plan& p, const void* u, const void* const* gates,
                                const void* H, const float* D, void* y, void* ws, const Fork& fk,
                                const BlockArgs* blk)
{
    MpGeom go = base_geom3(p);
    const int KP = 1 << go.kp_log2;
    const int C = (kMpThreads / threads_per_transform(go.La)) / KP;
    const int64_t col_blocks = (go.Lb_live + C - 1) / C;
    MpGeom gi = geom3_inner(p, go);
    const int U = (kMpThreads / threads_per_transform(gi.Lb)) / 2;
    const int64_t unit_blocks = (gi.La / 2 + U - 1) / U;
    const int64_t total_groups = (int64_t)p.B * go.groups_per_b;
    int64_t chunk_groups = p.chunk_pairs / KP;
    if (chunk_groups < 1) chunk_groups = 1;
    const float2* tw = static_cast<const float2*>(ws);
    const size_t esz = p.spec_dtype == HYENA_F32 ? 4 : 2;
    go.pair_bytes = p.fwd_pair_bytes;
    gi.pair_bytes = p.fwd_pair_bytes2;
    for (int64_t g0 = 0, ci = 0; g0 < total_groups; g0 += chunk_groups, ++ci) {
        const hipStream_t s = fk.stream_of(ci);
        const int cp = fk.copy_of(ci);
        float2* F1 = reinterpret_cast<float2*>(static_cast<char*>(ws) + p.fwd_offset[cp]);
        float2* F2 = reinterpret_cast<float2*>(static_cast<char*>(ws) + p.fwd2_offset[cp]);
        go.group0 = gi.group0 = g0;
        go.ngroups = gi.ngroups = total_groups - g0 < chunk_groups ? total_groups - g0 : chunk_groups;
        OuterArgs oa{};
        oa.g = go;
        oa.act = u;
        oa.F = F1;
        oa.tw = tw;
        if (blk) oa.blk = *blk;
        hyena_status st = outer(p, blk ? OUTER_IN3 : OUTER_IN, true, oa, col_blocks * go.ngroups, s);
        if (st != HYENA_OK) return st;
        const MidArgs mf = mid_args(p, go, F1, F2, false, MID_FWD, tw);
        const MidArgs mi = mid_args(p, go, F1, F2, false, MID_INV, tw);
        for (int n = 0; n < p.order; ++n) {
            st = mid((int)p.P2, MID_FWD, true, mf, mid_blocks(p, mf), s);
            if (st != HYENA_OK) return st;
            InnerArgs ia{};
            ia.g = gi;
            ia.F = F2;
            ia.spec = static_cast<const char*>(H) + (size_t)n * spec_elems_per_filter(p) * esz;
            ia.D = D + (int64_t)n * p.d;
            ia.tw = tw;
            st = inner(p, INNER_CHAIN, ia, unit_blocks * gi.ngroups * KP, s);
            if (st != HYENA_OK) return st;
            st = mid((int)p.P2, MID_INV, true, mi, mid_blocks(p, mi), s);
            if (st != HYENA_OK) return st;
            oa.act = blk ? nullptr : gates[n];
            oa.out = y;
            const int last = blk ? OUTER_OUT3 : OUTER_OUT;
            st = outer(p, n + 1 < p.order ? OUTER_MID : last, true, oa, col_blocks * go.ngroups, s);
            if (st != HYENA_OK) return st;
        }
    }
    return HYENA_OK;
}

hyena_status mp3_forward(const Plan& p, const void* u, const void* const* gates, const void* H,
                         const float* D, void* y, void* ws, void* stream,
                         const BlockArgs* blk = nullptr)
{
    Fork fk;
    const hyena_status st = fork_begin(p, (hipStream_t)stream, fk);
    if (st != HYENA_OK) return st;
    return fork_end(fk, mp3_forward_chunks(p, u, gates, H, D, y, ws, fk, blk));
}

hyena_status mp3_spectrum(const Plan& p, const void* h, void* H, void* ws, void* stream)
{
    const hipStream_t s = (hipStream_t)stream;
    MpGeom go = base_geom3(p);
    go.B = 1;  // filters have no batch axis
    const int KP = 1 << go.kp_log2;
    const int C = (kMpThreads / threads_per_transform(go.La)) / KP;
    const int64_t col_blocks = (go.Lb + C - 1) / C;
    MpGeom gi = geom3_inner(p, go);
    const int U = (kMpThreads / threads_per_transform(gi.Lb)) / 2;
    const int64_t unit_blocks = (gi.La / 2 + U - 1) / U;
    const int64_t total_groups = go.groups_per_b;
    int64_t chunk_groups = p.chunk_pairs / KP;
    if (chunk_groups < 1) chunk_groups = 1;
    float2* F1 = reinterpret_cast<float2*>(static_cast<char*>(ws) + p.inter_offset);
    float2* F2 = reinterpret_cast<float2*>(static_cast<char*>(ws) + p.inter2_offset);
    const float2* tw = static_cast<const float2*>(ws);
    const size_t esz = p.spec_dtype == HYENA_F32 ? 4 : 2;
    const int64_t taps = (2 * p.X - 1) * (2 * p.Y - 1) * (2 * p.Z - 1);
    go.pair_bytes = p.spec_pair_bytes;
    gi.pair_bytes = p.spec_pair_bytes2;
    for (int n = 0; n < p.order; ++n) {
        for (int64_t g0 = 0; g0 < total_groups; g0 += chunk_groups) {
            go.group0 = gi.group0 = g0;
            go.ngroups = gi.ngroups =
                total_groups - g0 < chunk_groups ? total_groups - g0 : chunk_groups;
            OuterArgs oa{};
            oa.g = go;
            oa.filt = static_cast<const char*>(h) + (size_t)n * p.d * taps * io_size(p);
            oa.F = F1;
            oa.tw = tw;
            hyena_status st = outer(p, OUTER_SPEC, false, oa, col_blocks * go.ngroups, s);
            if (st != HYENA_OK) return st;
            const MidArgs mf = mid_args(p, go, F1, F2, true, MID_FWD, tw);
            st = mid((int)p.P2, MID_FWD, false, mf, mid_blocks(p, mf), s);
            if (st != HYENA_OK) return st;
            InnerArgs ia{};
            ia.g = gi;
            ia.F = F2;
            ia.spec_out = static_cast<char*>(H) + (size_t)n * spec_elems_per_filter(p) * esz;
            ia.tw = tw;
            st = inner(p, INNER_SPEC, ia, unit_blocks * gi.ngroups * KP, s);
            if (st != HYENA_OK) return st;
        }
    }
    return HYENA_OK;
}

// One thread per entry (n, pair, unit, e) of a 3D spectrum; writes natural-
// order unscaled transfer functions [order][d][P1][P2][P3/2 + 1].  A bin and
// its mirror (-k) carry conjugate values; each is written where it falls in
// the stored half (kz <= P3/2).
template <typename SP>
__global__ void hyena_mp3_export(const SP* spec, float2* out, int64_t npairs, int64_t d, MpGeom g,
                                 int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int La = g.La, Lb = g.Lb, P3 = g.Lc, P2 = La / P3, W = P3 / 2 + 1;
    const int64_t per_pair = (int64_t)(La / 2) * Lb;
    const int64_t np = i / per_pair;
    const int64_t rem = i - np * per_pair;
    const int kk = (int)(rem / Lb), e = (int)(rem % Lb);
    const int64_t n = np / npairs, p = np - n * npairs;
    const int64_t c0 = 2 * p;
    const bool has_b = c0 + 1 < d;
    float2 P, Q;
    load_entry(spec, i, P, Q);
    const float M = (float)La * (float)Lb;
    const float2 ha = make_float2((P.x + Q.x) * M, (P.y + Q.y) * M);
    const float2 hb = make_float2((P.x - Q.x) * M, (P.y - Q.y) * M);
    float2* oa = out + (n * d + c0) * (int64_t)Lb * P2 * W;
    float2* ob = oa + (int64_t)Lb * P2 * W;
    auto put = [&](int kx, int col, float2 va, float2 vb) {
        const int ky = col / P3, kz = col - ky * P3;
        if (kz > P3 / 2) return;
        const int64_t at = ((int64_t)kx * P2 + ky) * W + kz;
        oa[at] = va;
        if (has_b) ob[at] = vb;
    };
    auto conj2 = [](float2 v) { return make_float2(v.x, -v.y); };
    int col0, col1;
    bool self;
    unit_columns(g, kk, col0, col1, self);
    if (!self) {
        put(e, col0, ha, hb);
        put((Lb - e) & (Lb - 1), col1, conj2(ha), conj2(hb));
    } else if (e == 0 || e == Lb / 2) {
        const int col = e == 0 ? col0 : col1;
        put(0, col, make_float2(ha.x, 0.0f), make_float2(hb.x, 0.0f));
        put(Lb / 2, col, make_float2(ha.y, 0.0f), make_float2(hb.y, 0.0f));
    } else {
        const int col = e < Lb / 2 ? col0 : col1;
        const int kx = e < Lb / 2 ? e : e - Lb / 2;
        put(kx, col, ha, hb);
        put(Lb - kx, col, conj2(ha), conj2(hb));
    }
}

hyena_status mp3_export(const Plan& p, const void* H, void* out, void* stream)
{
    const MpGeom g = geom3_inner(p, base_geom3(p));
    const int64_t total = (int64_t)p.order * p.npairs * p.spec_entries_per_pair;
    const int bs = 256;
    const int64_t nb = (total + bs - 1) / bs;
    if (p.spec_dtype == HYENA_F32)
        HY_LAUNCH(kernel_label("hyena_mp3_export", "float"), hyena_mp3_export<float>,
                  dim3((unsigned)nb), dim3(bs), 0, (hipStream_t)stream, (const float*)H,
                  (float2*)out, p.npairs, p.d, g, total);
    else
        HY_LAUNCH(kernel_label("hyena_mp3_export", "unsigned short"), hyena_mp3_export<uint16_t>,
                  dim3((unsigned)nb), dim3(bs), 0, (hipStream_t)stream, (const uint16_t*)H,
                  (float2*)out, p.npairs, p.d, g, total);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

}  // namespace

SingleStreamScope::SingleStreamScope() { ++t_single_stream; }
SingleStreamScope::~SingleStreamScope() { --t_single_stream; }

hyena_status launch_fourstep_forward(const Plan& p, const void* u, const void* const* gates,
                                     const void* H, const float* D, void* y, void* ws,
                                     void* stream)
{
    return mp_forward(p, u, gates, H, D, y, ws, stream);
}
hyena_status launch_fourstep_spectrum(const Plan& p, const void* h, void* H, void* ws, void* stream)
{
    return mp_spectrum(p, h, H, ws, stream);
}
hyena_status launch_fourstep_spectrum_implicit(const Plan& p, const float* z2, const float* W3,
                                               const float* b3, const float* alpha, int32_t hp,
                                               int32_t hidden, void* H, void* ws, void* stream)
{
    if (hp > kImpHidden) return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: hidden too wide");
    ImpOuter im{};
    im.z2 = z2;
    im.W3 = W3;
    im.b3 = b3;
    im.alpha = alpha;
    im.H = hidden;
    im.hp = hp;
    return mp_spectrum(p, nullptr, H, ws, stream, &im);
}
hyena_status launch_fourstep_export(const Plan& p, const void* H, void* out, void* stream)
{
    return mp_export(p, H, out, stream);
}
hyena_status launch_rowcol2d_forward(const Plan& p, const void* u, const void* const* gates,
                                     const void* H, const float* D, void* y, void* ws,
                                     void* stream)
{
    return mp_forward(p, u, gates, H, D, y, ws, stream);
}
hyena_status launch_rowcol2d_block(const Plan& p, const hyena_nd_mixer& m, const void* H,
                                   const float* D, void* y, void* ws, void* stream)
{
    BlockArgs b{};
    b.q = m.q;
    b.k = m.k;
    b.v = m.v;
    b.sw = m.short_w;
    b.sb = m.short_b;
    b.on = 1;
    return mp_forward(p, nullptr, nullptr, H, D, y, ws, stream, &b);
}
hyena_status launch_rowcol2d_spectrum(const Plan& p, const void* h, void* H, void* ws, void* stream)
{
    return mp_spectrum(p, h, H, ws, stream);
}
hyena_status launch_rowcol2d_export(const Plan& p, const void* H, void* out, void* stream)
{
    return mp_export(p, H, out, stream);
}

}  // namespace hy

namespace hy {

hyena_status launch_rowcol3d_forward(const Plan& p, const void* u, const void* const* gates,
                                     const void* H, const float* D, void* y, void* ws,
                                     void* stream)
{
    return mp3_forward(p, u, gates, H, D, y, ws, stream);
}
hyena_status launch_rowcol3d_spectrum(const Plan& p, const void* h, void* H, void* ws, void* stream)
{
    return mp3_spectrum(p, h, H, ws, stream);
}
hyena_status launch_rowcol3d_export(const Plan& p, const void* H, void* out, void* stream)
{
    return mp3_export(p, H, out, stream);
}
hyena_status launch_rowcol3d_block(const Plan& p, const hyena_nd_mixer& m, const void* H,
                                   const float* D, void* y, void* ws, void* stream)
{
    BlockArgs b{};
    b.q = m.q;
    b.k = m.k;
    b.v = m.v;
    b.sw = m.short_w;
    b.sb = m.short_b;
    b.on = 1;
    return mp3_forward(p, nullptr, nullptr, H, D, y, ws, stream, &b);
}

}  // namespace hy
