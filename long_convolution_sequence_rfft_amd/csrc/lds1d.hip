// lds1d.hip -- launch side of the single-workgroup path (kernels in
// lds1d_kernels.h, instantiated per storage type in lds1d_f32.hip and
// lds1d_bf16.hip), the spectrum export and the twiddle-table writer.
#include "lds1d_kernels.h"

namespace hy {

// instantiated in lds1d_f32.hip / lds1d_bf16.hip
HY_LDS1D_SIZES(HY_LDS1D_EXTERN, float, float)
HY_LDS1D_SIZES(HY_LDS1D_EXTERN, uint16_t, uint16_t)
HY_LDS1D_SIZES(HY_LDS1D_EXTERN, uint16_t, float)

// ---------------------------------------------------------------------------
// Twiddle tables: double-precision roots of unity rounded once to float.
// ---------------------------------------------------------------------------
struct TwInitArgs {
    TwSegment seg[kMaxTwSegments];
    int32_t nseg;
    int64_t total;
};

__global__ void hyena_tw_init(float2* tw, TwInitArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.total) return;
    for (int s = 0; s < a.nseg; ++s) {
        const int64_t len = (int64_t)(a.seg[s].radix - 1) * a.seg[s].ns;
        if (i >= a.seg[s].off && i < a.seg[s].off + len) {
            const int64_t loc = i - a.seg[s].off;
            const int64_t r = loc / a.seg[s].ns + 1, k = loc % a.seg[s].ns;
            const int64_t L = (int64_t)a.seg[s].ns * a.seg[s].radix;
            const int64_t m = (r * k) % L;
            double sn, cs;
            sincospi(-2.0 * (double)m / (double)L, &sn, &cs);
            tw[i] = make_float2((float)cs, (float)sn);
            return;
        }
    }
    tw[i] = make_float2(0.0f, 0.0f);
}

hyena_status launch_tw_init(const Plan& p, void* ws, void* stream)
{
    if (p.tw_elems == 0) return HYENA_OK;
    TwInitArgs a{};
    for (int s = 0; s < p.nseg; ++s) a.seg[s] = p.seg[s];
    a.nseg = p.nseg;
    a.total = p.tw_elems;
    const int bs = 256;
    const int64_t nb = (p.tw_elems + bs - 1) / bs;
    hipLaunchKernelGGL(hyena_tw_init, dim3((unsigned)nb), dim3(bs), 0, (hipStream_t)stream,
                       (float2*)ws, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Spectrum export: natural-order unscaled transfer functions, complex64
// [order][d][M/2 + 1], one thread per entry.
// ---------------------------------------------------------------------------
template <typename SP>
__global__ void hyena_lds1d_export(const SP* spec, float2* out, int64_t npairs, int64_t d,
                                   int64_t M, int64_t T, int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t half = M / 2;
    const int64_t np = i / half;  // n * npairs + p
    const int64_t rem = i - np * half;
    const int64_t e = rem / T, tau = rem - e * T;
    const int64_t n = np / npairs, p = np - n * npairs;
    const int64_t c0 = 2 * p;
    float2 P, Q;
    load_entry(spec, i, P, Q);
    const float sc = (float)M;
    float2* oa = out + (n * d + c0) * (half + 1);
    float2* ob = oa + (half + 1);
    const bool has_b = c0 + 1 < d;
    if (tau == 0 && e == 0) {
        oa[0] = make_float2((P.x + Q.x) * sc, 0.0f);
        oa[half] = make_float2((P.y + Q.y) * sc, 0.0f);
        if (has_b) {
            ob[0] = make_float2((P.x - Q.x) * sc, 0.0f);
            ob[half] = make_float2((P.y - Q.y) * sc, 0.0f);
        }
        return;
    }
    const int64_t k = entry_bin(M, T, tau, e);
    oa[k] = make_float2((P.x + Q.x) * sc, (P.y + Q.y) * sc);
    if (has_b) ob[k] = make_float2((P.x - Q.x) * sc, (P.y - Q.y) * sc);
}

hyena_status launch_lds1d_export(const Plan& p, const void* H, void* out, void* stream)
{
    const int64_t total = (int64_t)p.order * p.npairs * (p.M / 2);
    const int bs = 256;
    const int64_t nb = (total + bs - 1) / bs;
    const int64_t T = p.M / lds1d_pts((int)p.M);
    if (p.spec_dtype == HYENA_F32)
        hipLaunchKernelGGL(hyena_lds1d_export<float>, dim3((unsigned)nb), dim3(bs), 0,
                           (hipStream_t)stream, (const float*)H, (float2*)out, p.npairs, p.d,
                           p.M, T, total);
    else
        hipLaunchKernelGGL(hyena_lds1d_export<uint16_t>, dim3((unsigned)nb), dim3(bs), 0,
                           (hipStream_t)stream, (const uint16_t*)H, (float2*)out, p.npairs,
                           p.d, p.M, T, total);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// dispatch on M and storage types
// ---------------------------------------------------------------------------
namespace {

template <typename IO, typename SP>
hyena_status fwd_by_m(int64_t M, const Lds1dFwdArgs& a, bool fast, hipStream_t s)
{
    switch (M) {
#define HY_CASE(MM, I, S_) \
    case MM: return lds1d_forward_launch<MM, IO, SP>(a, fast, s);
        HY_LDS1D_SIZES(HY_CASE, IO, SP)
#undef HY_CASE
        default: return fail(HYENA_ERR_UNSUPPORTED, "LDS1D: unsupported transform length");
    }
}

template <typename IO, typename SP>
hyena_status spec_by_m(int64_t M, const Lds1dSpecArgs& a, hipStream_t s)
{
    switch (M) {
#define HY_CASE(MM, I, S_) \
    case MM: return lds1d_spectrum_launch<MM, IO, SP>(a, s);
        HY_LDS1D_SIZES(HY_CASE, IO, SP)
#undef HY_CASE
        default: return fail(HYENA_ERR_UNSUPPORTED, "LDS1D: unsupported transform length");
    }
}

TwOffsets lds1d_offsets(const Plan& p)
{
    TwOffsets o;
    o.f1 = (int32_t)p.seg[0].off;
    o.fL = (int32_t)p.seg[1].off;
    o.i1 = (int32_t)p.seg[2].off;
    o.i0 = (int32_t)p.seg[3].off;
    return o;
}

}  // namespace

hyena_status launch_lds1d_forward(const Plan& p, const void* u, const void* const* gates,
                                  const void* H, const float* D, void* y, const void* ws,
                                  void* stream)
{
    Lds1dFwdArgs a{};
    a.u = u;
    for (int n = 0; n < p.order; ++n) a.gates[n] = gates[n];
    a.y = y;
    a.spec = H;
    a.D = D;
    a.tw = static_cast<const float2*>(ws);
    a.N = p.N;
    a.d = p.d;
    a.npairs = p.npairs;
    a.nblocks = p.B * p.npairs;
    a.order = p.order;
    a.tw_off = lds1d_offsets(p);
    const bool fast = (p.d % 2 == 0) && (p.N * 2 == p.M);
    const hipStream_t s = (hipStream_t)stream;
    if (p.io_dtype == HYENA_F32) return fwd_by_m<float, float>(p.M, a, fast, s);
    if (p.spec_dtype == HYENA_BF16) return fwd_by_m<uint16_t, uint16_t>(p.M, a, fast, s);
    return fwd_by_m<uint16_t, float>(p.M, a, fast, s);
}

hyena_status launch_lds1d_spectrum(const Plan& p, const void* h, void* H, const void* ws,
                                   void* stream)
{
    Lds1dSpecArgs a{};
    a.h = h;
    a.spec = H;
    a.tw = static_cast<const float2*>(ws);
    a.N = p.N;
    a.d = p.d;
    a.npairs = p.npairs;
    a.nblocks = (int64_t)p.order * p.npairs;
    a.tw_off = lds1d_offsets(p);
    const hipStream_t s = (hipStream_t)stream;
    if (p.io_dtype == HYENA_F32) return spec_by_m<float, float>(p.M, a, s);
    if (p.spec_dtype == HYENA_BF16) return spec_by_m<uint16_t, uint16_t>(p.M, a, s);
    return spec_by_m<uint16_t, float>(p.M, a, s);
}

}  // namespace hy
