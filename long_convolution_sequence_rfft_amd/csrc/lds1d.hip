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
    HY_LAUNCH(kernel_label("hyena_tw_init"), hyena_tw_init, dim3((unsigned)nb), dim3(bs), 0,
              (hipStream_t)stream, (float2*)ws, a);
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
        HY_LAUNCH(kernel_label("hyena_lds1d_export", "float"), hyena_lds1d_export<float>,
                  dim3((unsigned)nb), dim3(bs), 0, (hipStream_t)stream, (const float*)H, (float2*)out, p.npairs, p.d,
                           p.M, T, total);
    else
        HY_LAUNCH(kernel_label("hyena_lds1d_export", "unsigned short"), hyena_lds1d_export<uint16_t>,
                  dim3((unsigned)nb), dim3(bs), 0, (hipStream_t)stream, (const uint16_t*)H, (float2*)out, p.npairs,
                           p.d, p.M, T, total);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// dispatch on M and storage types
// ---------------------------------------------------------------------------
namespace {

template <typename IO, typename SP>
hyena_status fwd_by_m(int64_t M, const Lds1dFwdArgs& a, int mode, hipStream_t s)
{
    switch (M) {
#define HY_CASE(MM, I, S_) \
    case MM: return lds1d_forward_launch<MM, IO, SP>(a, mode, s);
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

// ---------------------------------------------------------------------------
// Pair-major staging: [B][N][d] channels last <-> [B][pairs][N] pair elements
// (d even).  64 samples x one cache line of pairs per tile; both the row reads
// and the run writes are contiguous.
// ---------------------------------------------------------------------------
struct StageArgs {
    const void* src[kMaxOrder + 1];
    void* dst[kMaxOrder + 1];
    int64_t B, N, d, npairs;
};

// Tile: kStageTT samples x one 128-byte line of pairs.  Each thread first
// issues all of its loads, then writes LDS; after the barrier it reads all of
// its LDS values, then stores, so the memory latencies of one thread overlap.
constexpr int kStageTT = 128;

template <typename IO, bool TO_PAIRMAJOR>
__global__ void __launch_bounds__(256) hyena_stage_pairs(StageArgs a)
{
    using Raw = typename PairRaw<IO>::type;
    constexpr int TP = 128 / (int)sizeof(Raw);  // pairs per 128-byte line
    constexpr int TT = kStageTT;                // samples per tile
    constexpr int PER = TT * TP / 256;          // elements per thread
    static_assert(TT * TP % 256 == 0, "stage tile split");
    // row stride TP + 1 elements: both the row-wise and the column-wise
    // passes over the tile hit distinct banks
    __shared__ Raw tile[TT][TP + 1];
    const int64_t p0 = (int64_t)blockIdx.x * TP;
    const int64_t t0 = (int64_t)blockIdx.y * TT;
    const int64_t b = blockIdx.z % a.B;
    const int s = blockIdx.z / a.B;
    const Raw* src = static_cast<const Raw*>(a.src[s]);
    Raw* dst = static_cast<Raw*>(a.dst[s]);
    const int64_t P = a.npairs;
    const int64_t rowpairs = a.d / 2;  // pair elements per channels-last row
    const bool full = t0 + TT <= a.N && p0 + TP <= P;
    // (tr, pc) of element k of this thread: row-wise (pairs fastest) for the
    // channels-last side, column-wise (samples fastest) for the pair-major side
    auto rowwise = [&](int k, int& tr, int& pc) {
        const int i = (int)threadIdx.x + k * 256;
        tr = i / TP;
        pc = i % TP;
    };
    auto colwise = [&](int k, int& tr, int& pc) {
        const int i = (int)threadIdx.x + k * 256;
        pc = i / TT;
        tr = i % TT;
    };
    auto src_index = [&](int tr, int pc) {
        return TO_PAIRMAJOR ? (b * a.N + t0 + tr) * rowpairs + p0 + pc
                            : (b * P + p0 + pc) * a.N + t0 + tr;
    };
    auto dst_index = [&](int tr, int pc) {
        return TO_PAIRMAJOR ? (b * P + p0 + pc) * a.N + t0 + tr
                            : (b * a.N + t0 + tr) * rowpairs + p0 + pc;
    };
    auto in_range = [&](int tr, int pc) { return full || (t0 + tr < a.N && p0 + pc < P); };

    Raw x[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        int tr, pc;
        if (TO_PAIRMAJOR) rowwise(k, tr, pc);
        else colwise(k, tr, pc);
        if (in_range(tr, pc)) x[k] = src[src_index(tr, pc)];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        int tr, pc;
        if (TO_PAIRMAJOR) rowwise(k, tr, pc);
        else colwise(k, tr, pc);
        tile[tr][pc] = x[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        int tr, pc;
        if (TO_PAIRMAJOR) colwise(k, tr, pc);
        else rowwise(k, tr, pc);
        x[k] = tile[tr][pc];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        int tr, pc;
        if (TO_PAIRMAJOR) colwise(k, tr, pc);
        else rowwise(k, tr, pc);
        if (in_range(tr, pc)) dst[dst_index(tr, pc)] = x[k];
    }
}

template <typename IO>
hyena_status stage_launch(const StageArgs& a, int ntensors, bool to_pm, hipStream_t s)
{
    constexpr int TP = 128 / (int)sizeof(typename PairRaw<IO>::type);
    const dim3 grid((unsigned)((a.npairs + TP - 1) / TP), (unsigned)((a.N + kStageTT - 1) / kStageTT),
                    (unsigned)(a.B * ntensors));
    if (to_pm)
        HY_LAUNCH(kernel_label("hyena_stage_pairs", type_label<IO>(), true),
                  (hyena_stage_pairs<IO, true>), grid, dim3(256), 0, s, a);
    else
        HY_LAUNCH(kernel_label("hyena_stage_pairs", type_label<IO>(), false),
                  (hyena_stage_pairs<IO, false>), grid, dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

hyena_status launch_lds1d_forward(const Plan& p, const void* u, const void* const* gates,
                                  const void* H, const float* D, void* y, const void* ws,
                                  void* stream)
{
    const hipStream_t s = (hipStream_t)stream;
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
    a.order = p.order;
    a.tw_off = lds1d_offsets(p);
    const int mode = p.lds_io;
    int64_t K = 1;
    if (mode == IO_TILED) {
        K = 16384 / p.M < 16 ? 16384 / p.M : 16;
    }
    a.nblocks = p.B * ((p.npairs + K - 1) / K);
    StageArgs st{};
    if (mode == IO_PAIRMAJOR) {
        const size_t esz = p.io_dtype == HYENA_F32 ? 4 : 2;
        const size_t tensor = (size_t)p.B * p.N * p.d * esz;
        char* base = const_cast<char*>(static_cast<const char*>(ws)) + p.stage_offset;
        st.B = p.B;
        st.N = p.N;
        st.d = p.d;
        st.npairs = p.npairs;
        st.src[0] = u;
        st.dst[0] = base;
        for (int n = 0; n < p.order; ++n) {
            st.src[1 + n] = gates[n];
            st.dst[1 + n] = base + (size_t)(1 + n) * tensor;
        }
        a.u = base;
        for (int n = 0; n < p.order; ++n) a.gates[n] = base + (size_t)(1 + n) * tensor;
        a.y = base + (size_t)(1 + p.order) * tensor;
        const hyena_status r = p.io_dtype == HYENA_F32 ? stage_launch<float>(st, 1 + p.order, true, s)
                                                       : stage_launch<uint16_t>(st, 1 + p.order, true, s);
        if (r != HYENA_OK) return r;
    }
    hyena_status r;
    if (p.io_dtype == HYENA_F32) r = fwd_by_m<float, float>(p.M, a, mode, s);
    else if (p.spec_dtype == HYENA_BF16) r = fwd_by_m<uint16_t, uint16_t>(p.M, a, mode, s);
    else r = fwd_by_m<uint16_t, float>(p.M, a, mode, s);
    if (r != HYENA_OK || mode != IO_PAIRMAJOR) return r;
    StageArgs out{};
    out.B = p.B;
    out.N = p.N;
    out.d = p.d;
    out.npairs = p.npairs;
    out.src[0] = a.y;
    out.dst[0] = y;
    return p.io_dtype == HYENA_F32 ? stage_launch<float>(out, 1, false, s)
                                   : stage_launch<uint16_t>(out, 1, false, s);
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
