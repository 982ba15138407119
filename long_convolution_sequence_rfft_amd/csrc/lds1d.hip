// lds1d.hip -- launch side of the single-workgroup path (kernels in
// lds1d_kernels.h, instantiated per storage type in lds1d_{f32,bf16,f16}.hip,
// lds1d_real_*.hip and lds1d_circ_*.hip): the staging transposes, the
// spectrum export and the twiddle-table writer.
#include "dispatch.h"
#include "lds1d_kernels.h"

namespace hy {

// instantiated in lds1d_f32.hip / lds1d_bf16.hip / lds1d_real_*.hip
HY_LDS1D_SIZES(HY_LDS1D_EXTERN, float, float)
HY_LDS1D_SIZES(HY_LDS1D_EXTERN, uint16_t, uint16_t)
HY_LDS1D_SIZES(HY_LDS1D_EXTERN, uint16_t, float)
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_EXTERN, float, float)
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_EXTERN, uint16_t, uint16_t)
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_EXTERN, uint16_t, float)
HY_LDS1D_SIZES(HY_LDS1D_EXTERN, _Float16, float)
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_EXTERN, _Float16, float)

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
    if (tau == 0 && e == M / (4 * T)) {
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

// Single-channel layout: entry (S, Dl) of bin k gives H[k] = L (S + Dl) and
// H[L-k] = L conj(S - Dl); entry (tau 0, slot RL/2) gives H[0], H[L] and
// H[L/2].
template <typename SP>
__global__ void hyena_lds1d_real_export(const SP* spec, float2* out, int64_t L, int64_t T,
                                        int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t half = L / 2;  // entries per channel
    const int64_t nc = i / half;  // n * d + c
    const int64_t rem = i - nc * half;
    const int64_t e = rem / T, tau = rem - e * T;
    float2 S, Dl;
    load_entry(spec, i, S, Dl);
    const float sc = (float)L;
    float2* o = out + nc * (L + 1);
    if (tau == 0 && e == L / (4 * T)) {
        o[0] = make_float2((S.x + Dl.x) * sc, 0.0f);
        o[L] = make_float2((S.x - Dl.x) * sc, 0.0f);
        o[L / 2] = make_float2(S.y * sc, Dl.y * sc);
        return;
    }
    const int64_t k = real_entry_bin(L, T, tau, e);
    o[k] = make_float2((S.x + Dl.x) * sc, (S.y + Dl.y) * sc);
    o[L - k] = make_float2((S.x - Dl.x) * sc, -(S.y - Dl.y) * sc);
}

hyena_status launch_lds1d_export(const Plan& p, const void* H, void* out, void* stream)
{
    if (p.lds_io == IO_REAL) {
        const int64_t L = p.M / 2;
        const int64_t total = (int64_t)p.order * p.d * (L / 2);
        const int bs = 256;
        const int64_t nb = (total + bs - 1) / bs;
        const int64_t T = L / lds1d_pts((int)L);
        if (p.spec_dtype == HYENA_F32)
            HY_LAUNCH(kernel_label("hyena_lds1d_real_export", "float"), hyena_lds1d_real_export<float>,
                      dim3((unsigned)nb), dim3(bs), 0, (hipStream_t)stream, (const float*)H,
                      (float2*)out, L, T, total);
        else
            HY_LAUNCH(kernel_label("hyena_lds1d_real_export", "unsigned short"),
                      hyena_lds1d_real_export<uint16_t>, dim3((unsigned)nb), dim3(bs), 0,
                      (hipStream_t)stream, (const uint16_t*)H, (float2*)out, L, T, total);
        const hipError_t e = hipGetLastError();
        return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
    }
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
hyena_status fwd_by_m(int64_t M, const Lds1dFwdArgs& a, hipStream_t s)
{
    switch (M) {
#define HY_CASE(MM, I, S_) \
    case MM: return lds1d_forward_launch<MM, IO, SP>(a, s);
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

template <typename IO, typename SP>
hyena_status real_fwd_by_l(int64_t L, bool circ, const Lds1dFwdArgs& a, hipStream_t s)
{
    switch (L) {
#define HY_CASE(LL, I, S_)                                                    \
    case LL:                                                                  \
        return circ ? lds1d_real_forward_launch<LL, IO, SP, true>(a, s)       \
                    : lds1d_real_forward_launch<LL, IO, SP, false>(a, s);
        HY_LDS1D_REAL_SIZES(HY_CASE, IO, SP)
#undef HY_CASE
        default: return fail(HYENA_ERR_UNSUPPORTED, "LDS1D: unsupported single-channel length");
    }
}

template <typename IO, typename SP>
hyena_status real_spec_by_l(int64_t L, bool circ, const Lds1dSpecArgs& a, hipStream_t s)
{
    switch (L) {
#define HY_CASE(LL, I, S_)                                                          \
    case LL:                                                                        \
        return circ ? lds1d_real_spectrum_launch<LL, IO, SP, true>(a, s)     \
                    : lds1d_real_spectrum_launch<LL, IO, SP, false>(a, s);
        HY_LDS1D_REAL_SIZES(HY_CASE, IO, SP)
#undef HY_CASE
        default: return fail(HYENA_ERR_UNSUPPORTED, "LDS1D: unsupported single-channel length");
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
// Staging transposes between channels-last [B][N][d] and channel-major
// [B][d][N] runs (cols = d), one element E per channel.  Tile: kStageTT
// samples x one 128-byte line of channels.
// Each thread first issues all of its loads, then writes LDS; after the
// barrier it reads all of its LDS values, then stores, so the memory
// latencies of one thread overlap.
// ---------------------------------------------------------------------------
struct StageArgs {
    const void* src[kMaxOrder + 1];
    void* dst[kMaxOrder + 1];
    const void* gate;  // GATED (back to channels-last): y = gate . staged value
    int64_t B, N, cols;
};

constexpr int kStageTT = 128;

// GATED (channel-major -> channels-last only): each output is multiplied by
// the gate at its own channels-last position, read with the same coalesced
// index as the store.  The chain's last gate is applied here for float32
// storage, so that gate is never staged.
template <typename E, bool TO_COLS, bool GATED = false>
__global__ void __launch_bounds__(256) hyena_stage(StageArgs a)
{
    static_assert(!GATED || (!TO_COLS && sizeof(E) == 4), "gate on the way out, float32");
    constexpr int TP = 128 / (int)sizeof(E);  // elements per 128-byte line
    constexpr int TT = kStageTT;              // samples per tile
    constexpr int PER = TT * TP / 256;        // elements per thread
    static_assert(TT * TP % 256 == 0, "stage tile split");
    // row stride TP + 1 elements: both the row-wise and the column-wise
    // passes over the tile spread over the banks
    __shared__ E tile[TT][TP + 1];
    const int64_t p0 = (int64_t)blockIdx.x * TP;
    const int64_t t0 = (int64_t)blockIdx.y * TT;
    const int64_t b = blockIdx.z % a.B;
    const int s = blockIdx.z / a.B;
    const E* src = static_cast<const E*>(a.src[s]);
    E* dst = static_cast<E*>(a.dst[s]);
    const int64_t P = a.cols;
    const bool full = t0 + TT <= a.N && p0 + TP <= P;
    // (tr, pc) of element k of this thread: row-wise (columns fastest) on the
    // channels-last side, column-wise (samples fastest) on the other
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
        return TO_COLS ? (b * a.N + t0 + tr) * P + p0 + pc : (b * P + p0 + pc) * a.N + t0 + tr;
    };
    auto dst_index = [&](int tr, int pc) {
        return TO_COLS ? (b * P + p0 + pc) * a.N + t0 + tr : (b * a.N + t0 + tr) * P + p0 + pc;
    };
    auto in_range = [&](int tr, int pc) { return full || (t0 + tr < a.N && p0 + pc < P); };

    E gv[GATED ? PER : 1];
    if constexpr (GATED) {
        const E* gate = static_cast<const E*>(a.gate);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int tr, pc;
            rowwise(k, tr, pc);
            if (in_range(tr, pc)) gv[k] = gate[dst_index(tr, pc)];
        }
    }
    E x[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        int tr, pc;
        if (TO_COLS) rowwise(k, tr, pc);
        else colwise(k, tr, pc);
        if (in_range(tr, pc)) x[k] = src[src_index(tr, pc)];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        int tr, pc;
        if (TO_COLS) rowwise(k, tr, pc);
        else colwise(k, tr, pc);
        tile[tr][pc] = x[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        int tr, pc;
        if (TO_COLS) colwise(k, tr, pc);
        else rowwise(k, tr, pc);
        x[k] = tile[tr][pc];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        int tr, pc;
        if (TO_COLS) colwise(k, tr, pc);
        else rowwise(k, tr, pc);
        if constexpr (GATED) {
            if (in_range(tr, pc)) dst[dst_index(tr, pc)] = x[k] * gv[k];
        } else {
            if (in_range(tr, pc)) dst[dst_index(tr, pc)] = x[k];
        }
    }
}

// bfloat16 channel-major staging for even d, moving 4 bytes per access on
// both sides: two neighbouring channels of a channels-last row, or two
// neighbouring samples of a channel-major run.  Tile: kStageTT samples x 64
// channels; word (t, w) of the tile holds channels 2w, 2w+1 of sample t.
template <bool TO_COLS>
__global__ void __launch_bounds__(256) hyena_stage_bf16(StageArgs a)
{
    constexpr int TT = kStageTT, TC = 64, TW = TC / 2;
    constexpr int RS = TW + 1;  // words per tile row (odd: spreads the banks)
    constexpr int PER = TT * TW / 256;
    __shared__ uint32_t tile[TT * RS];
    uint16_t* tile16 = reinterpret_cast<uint16_t*>(tile);
    const int64_t c0 = (int64_t)blockIdx.x * TC;
    const int64_t t0 = (int64_t)blockIdx.y * TT;
    const int64_t b = blockIdx.z % a.B;
    const int s = blockIdx.z / a.B;
    const uint32_t* src = static_cast<const uint32_t*>(a.src[s]);
    uint32_t* dst = static_cast<uint32_t*>(a.dst[s]);
    const int64_t d = a.cols;
    const bool full = t0 + TT <= a.N && c0 + TC <= d;
    // channels-last side: word (tr, wc) = channels c0 + 2wc, +1 of sample t0 + tr
    auto row_word = [&](int k, int& tr, int& wc) {
        const int i = (int)threadIdx.x + k * 256;
        tr = i / TW;
        wc = i % TW;
    };
    // channel-major side: word (c, j) = samples t0 + 2j, +1 of channel c0 + c
    auto run_word = [&](int k, int& c, int& j) {
        const int i = (int)threadIdx.x + k * 256;
        c = i / (TT / 2);
        j = i % (TT / 2);
    };
    auto row_ok = [&](int tr, int wc) { return full || (t0 + tr < a.N && c0 + 2 * wc < d); };
    auto run_ok = [&](int c, int j) { return full || (c0 + c < d && t0 + 2 * j < a.N); };
    auto row_index = [&](int tr, int wc) { return ((b * a.N + t0 + tr) * d + c0) / 2 + wc; };
    auto run_index = [&](int c, int j) { return ((b * d + c0 + c) * a.N + t0) / 2 + j; };

    uint32_t x[PER];
    if (TO_COLS) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int tr, wc;
            row_word(k, tr, wc);
            x[k] = row_ok(tr, wc) ? src[row_index(tr, wc)] : 0u;
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int tr, wc;
            row_word(k, tr, wc);
            tile[tr * RS + wc] = x[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int c, j;
            run_word(k, c, j);
            const uint32_t lo = tile16[(2 * j) * 2 * RS + c];
            const uint32_t hi = tile16[(2 * j + 1) * 2 * RS + c];
            x[k] = lo | (hi << 16);
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int c, j;
            run_word(k, c, j);
            if (run_ok(c, j)) dst[run_index(c, j)] = x[k];
        }
    } else {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int c, j;
            run_word(k, c, j);
            x[k] = run_ok(c, j) ? src[run_index(c, j)] : 0u;
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int c, j;
            run_word(k, c, j);
            tile16[(2 * j) * 2 * RS + c] = (uint16_t)(x[k] & 0xffffu);
            tile16[(2 * j + 1) * 2 * RS + c] = (uint16_t)(x[k] >> 16);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int tr, wc;
            row_word(k, tr, wc);
            x[k] = tile[tr * RS + wc];
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            int tr, wc;
            row_word(k, tr, wc);
            if (row_ok(tr, wc)) dst[row_index(tr, wc)] = x[k];
        }
    }
}

// ---------------------------------------------------------------------------
// 16-bit staging in full tiles (N a multiple of 64, d of 64), the form used
// whenever the shape allows: one tile of 64 samples x 64 channels per
// workgroup.  Words move whole on both sides (two channels of one sample on
// the row side, two samples of one channel on the run side); each is split
// into its halves on the way into LDS and read back whole.  Global accesses
// are raw buffer accesses from the tile's base (scalar descriptor), a scalar
// offset per word and one lane offset, so a tile's addressing is a handful
// of scalar instructions: 27 VALU instructions per wave against 568 for the
// word-transposing form above (the LDS conflict rate is the same 40%).
// Every offset stays below 2^31 for d below 2^22 (N <= 16384 on this path).
// Measured at 8K tokens, bf16: stage-in 32.0 -> 29.3 us, stage-out 12.6 ->
// 11.3 us; tiles of 128 samples were 0.5 us slower each way, and two or four
// of them per workgroup (more in flight, fewer workgroups per CU) no faster.
// ---------------------------------------------------------------------------
constexpr int kS16TT = 64, kS16TC = 64;

__device__ __forceinline__ const char* uniform_ptr(const void* p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const char* p)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, 0x7fffffff, 0x00020000);
}

template <bool TO_COLS>
__global__ void __launch_bounds__(256) hyena_stage16_full(StageArgs a)
{
    constexpr int NT = 256, TT = kS16TT, TC = kS16TC, TW = TC / 2;
    constexpr int PER = TT * TW / NT;   // 8 words per thread
    constexpr int RROWS = NT / TW;      // 8 row-side samples per pass
    constexpr int RCH = NT / (TT / 2);  // 8 run-side channels per pass
    // TO_COLS: channel-major tile, channel c's samples at c * RSC (16-bit units);
    // back: sample-major tile, sample t's channels at t * RST
    constexpr int RSC = TT + 2, RST = TC + 2;
    __shared__ uint32_t tile[(TO_COLS ? TC * RSC : TT * RST) / 2];
    uint16_t* tile16 = reinterpret_cast<uint16_t*>(tile);
    const int tid = (int)threadIdx.x;
    const int rtr = tid / TW, rwc = tid % TW;
    const int uc = tid / (TT / 2), uj = tid % (TT / 2);
    const int64_t d = a.cols, N = a.N;
    const uint32_t row_lane = (uint32_t)(rtr * d * 2 + rwc * 4);  // bytes
    const uint32_t run_lane = (uint32_t)(uc * N * 2 + uj * 4);
    const int64_t row_k = RROWS * d * 2, run_k = RCH * N * 2;     // bytes per word step
    const int64_t ncx = d / TC, nty = N / TT;
    const int64_t u = blockIdx.x;  // tile: channel block fastest, then samples, batch row, tensor
    const int64_t cx = u % ncx;
    const int64_t r1 = u / ncx;
    const int64_t ty = r1 % nty;
    const int64_t z = r1 / nty;
    const int64_t b = z % a.B;
    const int s = (int)(z / a.B);
    const char* src = uniform_ptr(a.src[s]);
    const char* dst = uniform_ptr(a.dst[s]);
    const int64_t c0 = cx * TC, t0 = ty * TT;
    const int64_t row_base = ((b * N + t0) * d + c0) * 2;
    const int64_t run_base = ((b * d + c0) * N + t0) * 2;
    const __amdgpu_buffer_rsrc_t rrow = rsrc_of((TO_COLS ? src : dst) + row_base);
    const __amdgpu_buffer_rsrc_t rrun = rsrc_of((TO_COLS ? dst : src) + run_base);
    uint32_t x[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k)
        x[k] = TO_COLS ? __builtin_amdgcn_raw_buffer_load_b32(rrow, row_lane, (int)(k * row_k), 0)
                       : __builtin_amdgcn_raw_buffer_load_b32(rrun, run_lane, (int)(k * run_k), 0);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if constexpr (TO_COLS) {
            const int t = rtr + RROWS * k;
            tile16[(2 * rwc) * RSC + t] = (uint16_t)(x[k] & 0xffffu);
            tile16[(2 * rwc + 1) * RSC + t] = (uint16_t)(x[k] >> 16);
        } else {
            const int c = uc + RCH * k;
            tile16[(2 * uj) * RST + c] = (uint16_t)(x[k] & 0xffffu);
            tile16[(2 * uj + 1) * RST + c] = (uint16_t)(x[k] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k)
        x[k] = TO_COLS ? tile[((uc + RCH * k) * RSC) / 2 + uj] : tile[((rtr + RROWS * k) * RST) / 2 + rwc];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if constexpr (TO_COLS)
            __builtin_amdgcn_raw_buffer_store_b32(x[k], rrun, run_lane, (int)(k * run_k), 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(x[k], rrow, row_lane, (int)(k * row_k), 0);
    }
}

hyena_status stage16_full_launch(const StageArgs& a, int ntensors, bool to_cols, hipStream_t s)
{
    const unsigned grid = (unsigned)(a.cols / kS16TC * (a.N / kS16TT) * a.B * (int64_t)ntensors);
    if (to_cols)
        HY_LAUNCH(kernel_label("hyena_stage16_full", true), (hyena_stage16_full<true>), dim3(grid),
                  dim3(256), 0, s, a);
    else
        HY_LAUNCH(kernel_label("hyena_stage16_full", false), (hyena_stage16_full<false>), dim3(grid),
                  dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

// The float32 counterpart (d a multiple of 32): one tile of 128 samples x
// 32 channels (one 128-byte line) per workgroup, raw buffer accesses as
// above.  GATED (back to channels-last only): each output is multiplied by
// the gate read at its own channels-last position with the store's offsets.
// Measured at 2K tokens: stage-in 23.4-23.8 -> 21.6-21.9 us, gated
// stage-out 18.0 -> 17.1 us (the general gated form holds 166 VGPRs, three
// waves per SIMD; this one 37, eight).
template <bool TO_COLS, bool GATED>
__global__ void __launch_bounds__(256) hyena_stage32_full(StageArgs a)
{
    static_assert(!GATED || !TO_COLS, "gate on the way out");
    constexpr int NT = 256, TT = kStageTT, TC = 32;
    constexpr int PER = TT * TC / NT;   // 16 values per thread
    constexpr int RROWS = NT / TC;      // 8 row-side samples per pass
    constexpr int RCH = NT / TT;        // 2 run-side channels per pass
    // TO_COLS: channel-major tile (channel c's samples at c * (TT + 1));
    // back: sample-major tile (sample t's channels at t * (TC + 1))
    constexpr int RSC = TT + 1, RST = TC + 1;
    __shared__ float tile[TO_COLS ? TC * RSC : TT * RST];
    const int tid = (int)threadIdx.x;
    const int rtr = tid / TC, rwc = tid % TC;
    const int uc = tid / TT, uj = tid % TT;
    const int64_t d = a.cols, N = a.N;
    const uint32_t row_lane = (uint32_t)(rtr * d * 4 + rwc * 4);  // bytes
    const uint32_t run_lane = (uint32_t)(uc * N * 4 + uj * 4);
    const int64_t row_k = RROWS * d * 4, run_k = RCH * N * 4;     // bytes per step
    const int64_t ncx = d / TC, nty = N / TT;
    const int64_t u = blockIdx.x;  // tile: channel block fastest, then samples, batch row, tensor
    const int64_t cx = u % ncx;
    const int64_t r1 = u / ncx;
    const int64_t ty = r1 % nty;
    const int64_t z = r1 / nty;
    const int64_t b = z % a.B;
    const int s = (int)(z / a.B);
    const char* src = uniform_ptr(a.src[s]);
    const char* dst = uniform_ptr(a.dst[s]);
    const int64_t c0 = cx * TC, t0 = ty * TT;
    const int64_t row_base = ((b * N + t0) * d + c0) * 4;
    const int64_t run_base = ((b * d + c0) * N + t0) * 4;
    const __amdgpu_buffer_rsrc_t rrow = rsrc_of((TO_COLS ? src : dst) + row_base);
    const __amdgpu_buffer_rsrc_t rrun = rsrc_of((TO_COLS ? dst : src) + run_base);
    float x[PER];
    float g[GATED ? PER : 1];
    if constexpr (GATED) {
        const __amdgpu_buffer_rsrc_t rg = rsrc_of(uniform_ptr(a.gate) + row_base);
#pragma unroll
        for (int k = 0; k < PER; ++k)
            g[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, row_lane, (int)(k * row_k), 0));
    }
#pragma unroll
    for (int k = 0; k < PER; ++k)
        x[k] = __builtin_bit_cast(float, TO_COLS
            ? __builtin_amdgcn_raw_buffer_load_b32(rrow, row_lane, (int)(k * row_k), 0)
            : __builtin_amdgcn_raw_buffer_load_b32(rrun, run_lane, (int)(k * run_k), 0));
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if constexpr (TO_COLS) tile[rwc * RSC + rtr + RROWS * k] = x[k];
        else tile[uj * RST + uc + RCH * k] = x[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k)
        x[k] = TO_COLS ? tile[(uc + RCH * k) * RSC + uj] : tile[(rtr + RROWS * k) * RST + rwc];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if constexpr (TO_COLS) {
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x[k]), rrun, run_lane,
                                                  (int)(k * run_k), 0);
        } else {
            const float y = GATED ? x[k] * g[k] : x[k];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, y), rrow, row_lane,
                                                  (int)(k * row_k), 0);
        }
    }
}

hyena_status stage32_full_launch(const StageArgs& a, int ntensors, bool to_cols, hipStream_t s)
{
    const unsigned grid = (unsigned)(a.cols / 32 * (a.N / kStageTT) * a.B * (int64_t)ntensors);
    if (to_cols)
        HY_LAUNCH(kernel_label("hyena_stage32_full", true, false), (hyena_stage32_full<true, false>),
                  dim3(grid), dim3(256), 0, s, a);
    else if (a.gate)
        HY_LAUNCH(kernel_label("hyena_stage32_full", false, true), (hyena_stage32_full<false, true>),
                  dim3(grid), dim3(256), 0, s, a);
    else
        HY_LAUNCH(kernel_label("hyena_stage32_full", false, false), (hyena_stage32_full<false, false>),
                  dim3(grid), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

hyena_status stage_bf16_launch(const StageArgs& a, int ntensors, bool to_cols, hipStream_t s)
{
    const dim3 grid((unsigned)((a.cols + 63) / 64), (unsigned)((a.N + kStageTT - 1) / kStageTT),
                    (unsigned)(a.B * ntensors));
    if (to_cols)
        HY_LAUNCH(kernel_label("hyena_stage_bf16", true), (hyena_stage_bf16<true>), grid, dim3(256),
                  0, s, a);
    else
        HY_LAUNCH(kernel_label("hyena_stage_bf16", false), (hyena_stage_bf16<false>), grid,
                  dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

template <typename E>
const char* elem_label();
template <>
const char* elem_label<float>() { return "float"; }
template <>
const char* elem_label<uint16_t>() { return "unsigned short"; }

template <typename E>
hyena_status stage_launch(const StageArgs& a, int ntensors, bool to_cols, hipStream_t s)
{
    constexpr int TP = 128 / (int)sizeof(E);
    const dim3 grid((unsigned)((a.cols + TP - 1) / TP), (unsigned)((a.N + kStageTT - 1) / kStageTT),
                    (unsigned)(a.B * ntensors));
    if constexpr (sizeof(E) == 4) {
        if (a.gate) {
            HY_LAUNCH(kernel_label("hyena_stage", elem_label<E>(), false, true),
                      (hyena_stage<E, false, true>), grid, dim3(256), 0, s, a);
            const hipError_t e = hipGetLastError();
            return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
        }
    }
    if (to_cols)
        HY_LAUNCH(kernel_label("hyena_stage", elem_label<E>(), true, false), (hyena_stage<E, true>),
                  grid, dim3(256), 0, s, a);
    else
        HY_LAUNCH(kernel_label("hyena_stage", elem_label<E>(), false, false), (hyena_stage<E, false>),
                  grid, dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

// Stage u and the gates (to_cols) or y (back) channel-major.
hyena_status stage_plan(const Plan& p, const StageArgs& a, int ntensors, bool to_cols, hipStream_t s)
{
    StageArgs b = a;
    b.cols = p.d;
    // full tiles: the forms with scalar-based buffer accesses
    if (p.io_dtype == HYENA_F32 && p.d % 32 == 0 && p.N % kStageTT == 0 && p.d < (int64_t(1) << 22))
        return stage32_full_launch(b, ntensors, to_cols, s);
    if (p.io_dtype == HYENA_F32) return stage_launch<float>(b, ntensors, to_cols, s);
    if (p.d % kS16TC == 0 && p.N % kS16TT == 0 && p.d < (int64_t(1) << 22))
        return stage16_full_launch(b, ntensors, to_cols, s);
    if (p.d % 2 == 0) return stage_bf16_launch(b, ntensors, to_cols, s);
    return stage_launch<uint16_t>(b, ntensors, to_cols, s);
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
    a.B = p.B;
    a.nblocks = p.B * p.npairs;
    a.twm = static_cast<const float2*>(ws) + p.seg[4].off;
    const bool staged = p.lds_io == IO_REAL;
    if (staged) a.nblocks = p.B * p.d;
    StageArgs st{};
    if (staged) {
        const size_t esz = p.io_dtype == HYENA_F32 ? 4 : 2;
        const size_t tensor = (size_t)p.B * p.N * p.d * esz;
        char* base = const_cast<char*>(static_cast<const char*>(ws)) + p.stage_offset;
        st.B = p.B;
        st.N = p.N;
        // float32 storage: the last gate is applied on the way back out
        // (same single multiply, one tensor fewer staged)
        a.last_gate_out = p.io_dtype == HYENA_F32;
        const int staged_gates = p.order - a.last_gate_out;
        st.src[0] = u;
        st.dst[0] = base;
        for (int n = 0; n < staged_gates; ++n) {
            st.src[1 + n] = gates[n];
            st.dst[1 + n] = base + (size_t)(1 + n) * tensor;
        }
        a.u = base;
        for (int n = 0; n < p.order; ++n) a.gates[n] = base + (size_t)(1 + n) * tensor;
        a.y = base + (size_t)(1 + p.order) * tensor;
        const hyena_status r = stage_plan(p, st, 1 + staged_gates, true, s);
        if (r != HYENA_OK) return r;
    }
    const hyena_status r = by_storage(p, [&](auto io, auto sp) {
        using IO = typename decltype(io)::type;
        using SP = typename decltype(sp)::type;
        return staged ? real_fwd_by_l<IO, SP>(p.M / 2, p.circular != 0, a, s)
                      : fwd_by_m<IO, SP>(p.M, a, s);
    });
    if (r != HYENA_OK || !staged) return r;
    StageArgs out{};
    out.B = p.B;
    out.N = p.N;
    out.src[0] = a.y;
    out.dst[0] = y;
    out.gate = a.last_gate_out ? gates[p.order - 1] : nullptr;
    return stage_plan(p, out, 1, false, s);
}

Lds1dSpecArgs lds1d_spec_args(const Plan& p, void* H, const void* ws)
{
    Lds1dSpecArgs a{};
    a.spec = H;
    a.tw = static_cast<const float2*>(ws);
    a.N = p.N;
    a.d = p.d;
    a.npairs = p.npairs;
    a.nblocks = (int64_t)p.order * p.npairs;
    a.tw_off = lds1d_offsets(p);
    if (p.lds_io == IO_REAL) {
        a.nblocks = (int64_t)p.order * p.d;
        a.twm = static_cast<const float2*>(ws) + p.seg[4].off;
    }
    return a;
}

hyena_status launch_lds1d_spectrum(const Plan& p, const void* h, void* H, const void* ws,
                                   void* stream)
{
    Lds1dSpecArgs a = lds1d_spec_args(p, H, ws);
    a.h = h;
    const hipStream_t s = (hipStream_t)stream;
    const bool real = p.lds_io == IO_REAL;
    return by_storage(p, [&](auto io, auto sp) {
        using IO = typename decltype(io)::type;
        using SP = typename decltype(sp)::type;
        return real ? real_spec_by_l<IO, SP>(p.M / 2, p.circular != 0, a, s)
                    : spec_by_m<IO, SP>(p.M, a, s);
    });
}

}  // namespace hy
