// lds1d_kernels.h -- single-workgroup FFT convolution chain for transforms of
// length M <= 16384 (sequence length N <= 8192).
//
// One workgroup owns one (batch row b, channel pair c, c+1); the two real
// channels ride in one complex signal, and the whole order-N chain stays in
// registers and LDS:
//   load u (first N samples; the zero-padded half is never loaded)
//   for n = 1..order:
//     forward transform  (R0 pass with half-zero input, R1 pass, RL pass)
//     spectral product   Y[k] = Z[k] P[k] + conj(Z[M-k]) Q[k], feedthrough folded
//     inverse transform  (RL pass in registers, R1 pass, R0 pass keeping t < M/2)
//     gate               z <- gate_n . z   (samples t >= N are zeroed)
//   store y
// Chain and gate order: "Week 11: Hyena, Long Convolution, and Linear
// Attention", section "The Hyena operator", and "Hyena -- Long Convolutions
// Math", section "The Toeplitz picture" (gate after each convolution); the
// feedthrough D is the delta tap of the FFTConv equation ([P1] "FFTConv"),
// i.e. D added to every bin of the filter's transfer function.
#pragma once

#include "stockham.h"

namespace hy {

struct Lds1dFwdArgs {
    const void* u;
    const void* gates[kMaxOrder];
    void* y;
    const void* spec;
    const float* D;
    const float2* tw;
    int64_t N, d, npairs, nblocks;
    int32_t order;
    TwOffsets tw_off;
};

struct Lds1dSpecArgs {
    const void* h;
    void* spec;
    const float2* tw;
    int64_t N, d, npairs, nblocks;
    TwOffsets tw_off;
};

// FULL: N == M/2 (no sample of the live half is past the end of the sequence).
// EVEN: d is even (channel pairs are aligned wide accesses).
template <int M, typename IO, typename SP, bool FAST>
__global__ void __launch_bounds__(FftShape<M>::T, 2)
hyena_lds1d_forward(Lds1dFwdArgs a)
{
    using S = FftShape<M>;
    constexpr int T = S::T, PTS = S::PTS, R0 = S::R0;
    constexpr bool EVEN = FAST;
    __shared__ float sre[S::LW];
    __shared__ float sim[S::LW];
    __shared__ float sxs[4 * S::RL];

    const int tau = threadIdx.x;
    const int64_t lin = xcd_remap(blockIdx.x, a.nblocks);
    const int64_t b = lin / a.npairs;
    const int64_t p = lin - b * a.npairs;
    const int64_t c0 = 2 * p;
    const bool has_b = c0 + 1 < a.d;
    const int64_t row0 = b * a.N * a.d + c0;  // element offset of (b, t = 0, c0)
    const uint32_t dd = (uint32_t)a.d;
    const uint32_t N = (uint32_t)a.N;
    const int j1 = tau, j2 = tau ? 2 * T - tau : T;
    const float inv2M = 0.5f / (float)M;

    // Sample t = tau + q T + r (M/R0) of channel pair (c0, c0+1) of row b.
    // FAST: the row offset splits into a per-lane part (tau + q T) d and a
    // uniform part r (M/R0) d, so every access is scalar base + 32-bit offset.
    const IO* ubase = static_cast<const IO*>(a.u) + row0;
    float2 v[PTS];
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) {
        const uint32_t lane_off = (uint32_t)(tau + q * T) * dd * (uint32_t)sizeof(IO);
#pragma unroll
        for (int r = 0; r < R0 / 2; ++r) {
            if constexpr (FAST) {
                v[q * R0 + r] = widen_pair<IO>(load_pair_raw(ubase + (size_t)r * (M / R0) * dd, lane_off));
            } else {
                const uint32_t t = tau + q * T + r * (M / R0);
                v[q * R0 + r] = t < N ? load_pair<IO, EVEN>(ubase + (size_t)t * dd, has_b)
                                      : make_float2(0.0f, 0.0f);
            }
        }
    }

    for (int n = 0; n < a.order; ++n) {
        const SP* spec = static_cast<const SP*>(a.spec) +
                         ((int64_t)n * a.npairs + p) * (int64_t)(M / 2) * kEntryElems;
        typename EntryRaw<SP>::type ent[S::RL];
        fwd_transform<M>(v, sre, sim, a.tw, a.tw_off, tau, j1, j2, n > 0,
                         [&] { load_entries<M, SP>(ent, spec, tau); });

        const float Da = a.D[(int64_t)n * a.d + c0];
        const float Db = has_b ? a.D[(int64_t)n * a.d + c0 + 1] : 0.0f;
        spectral_product<M, SP>(v, ent, tau, (Da + Db) * inv2M, (Da - Db) * inv2M, sxs);

        const IO* g = static_cast<const IO*>(a.gates[n]) + row0;
        typename PairRaw<IO>::type graw[S::Q0][R0 / 2];
        float2 gv[S::Q0][R0 / 2];
        inv_transform<M>(v, sre, sim, a.tw, a.tw_off, tau, j1, j2, [&] {
#pragma unroll
            for (int q = 0; q < S::Q0; ++q) {
                const uint32_t lane_off = (uint32_t)(tau + q * T) * dd * (uint32_t)sizeof(IO);
#pragma unroll
                for (int r = 0; r < R0 / 2; ++r) {
                    if constexpr (FAST) {
                        graw[q][r] = load_pair_raw(g + (size_t)r * (M / R0) * dd, lane_off);
                    } else {
                        const uint32_t t = tau + q * T + r * (M / R0);
                        gv[q][r] = t < N ? load_pair<IO, EVEN>(g + (size_t)t * dd, has_b)
                                         : make_float2(0.0f, 0.0f);
                    }
                }
            }
        });
#pragma unroll
        for (int q = 0; q < S::Q0; ++q)
#pragma unroll
            for (int r = 0; r < R0 / 2; ++r) {
                const float2 gg = FAST ? widen_pair<IO>(graw[q][r]) : gv[q][r];
                float2& x = v[q * R0 + r];
                x = make_float2(x.x * gg.x, x.y * gg.y);
            }
    }

    IO* ybase = static_cast<IO*>(a.y) + row0;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) {
        const uint32_t lane_off = (uint32_t)(tau + q * T) * dd * (uint32_t)sizeof(IO);
#pragma unroll
        for (int r = 0; r < R0 / 2; ++r) {
            if constexpr (FAST) {
                store_pair_at(ybase + (size_t)r * (M / R0) * dd, lane_off, v[q * R0 + r]);
            } else {
                const uint32_t t = tau + q * T + r * (M / R0);
                if (t < N) store_pair<IO, EVEN>(ybase + (size_t)t * dd, v[q * R0 + r], has_b);
            }
        }
    }
}

// Filter spectrum: one workgroup per (filter n, channel pair).
// Z = DFT_M(pad(h_a + i h_b)); entries ((Ha + Hb), (Ha - Hb)) / (2M), the
// 1/M of the unscaled inverse transform folded in.
template <int M, typename IO, typename SP>
__global__ void __launch_bounds__(FftShape<M>::T, 2)
hyena_lds1d_spectrum(Lds1dSpecArgs a)
{
    using S = FftShape<M>;
    constexpr int T = S::T, PTS = S::PTS, R0 = S::R0;
    __shared__ float sre[S::LW];
    __shared__ float sim[S::LW];

    const int tau = threadIdx.x;
    const int64_t lin = blockIdx.x;  // n * npairs + p
    const int64_t n = lin / a.npairs;
    const int64_t p = lin - n * a.npairs;
    const int64_t c0 = 2 * p;
    const bool has_b = c0 + 1 < a.d;
    const IO* ha = static_cast<const IO*>(a.h) + (n * a.d + c0) * a.N;
    const IO* hb = ha + a.N;
    const int j1 = tau, j2 = tau ? 2 * T - tau : T;

    float2 v[PTS];
#pragma unroll
    for (int q = 0; q < S::Q0; ++q)
#pragma unroll
        for (int r = 0; r < R0 / 2; ++r) {
            const int64_t t = tau + q * T + r * (M / R0);
            const bool live = t < a.N;
            v[q * R0 + r] = make_float2(live ? ld1<IO>(ha + t) : 0.0f,
                                        (live && has_b) ? ld1<IO>(hb + t) : 0.0f);
        }
    fwd_transform<M>(v, sre, sim, a.tw, a.tw_off, tau, j1, j2, false, [] {});
    SP* spec = static_cast<SP*>(a.spec) + lin * (int64_t)(M / 2) * kEntryElems;
    store_spectrum_entries<M, SP>(v, spec, tau, 0.5f / (float)M);
}

template <int M, typename IO, typename SP>
hyena_status lds1d_forward_launch(const Lds1dFwdArgs& a, bool fast, hipStream_t s)
{
    const dim3 grid((unsigned)a.nblocks), block(FftShape<M>::T);
    if (fast) hipLaunchKernelGGL((hyena_lds1d_forward<M, IO, SP, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((hyena_lds1d_forward<M, IO, SP, false>), grid, block, 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

template <int M, typename IO, typename SP>
hyena_status lds1d_spectrum_launch(const Lds1dSpecArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL((hyena_lds1d_spectrum<M, IO, SP>), dim3((unsigned)a.nblocks),
                       dim3(FftShape<M>::T), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

#define HY_LDS1D_SIZES(X, IO, SP) \
    X(8, IO, SP) X(16, IO, SP) X(32, IO, SP) X(64, IO, SP) X(128, IO, SP) X(256, IO, SP) \
    X(512, IO, SP) X(1024, IO, SP) X(2048, IO, SP) X(4096, IO, SP) X(8192, IO, SP)       \
    X(16384, IO, SP)

#define HY_LDS1D_INSTANTIATE(M, IO, SP)                                                      \
    template hyena_status lds1d_forward_launch<M, IO, SP>(const Lds1dFwdArgs&, bool,         \
                                                          hipStream_t);                      \
    template hyena_status lds1d_spectrum_launch<M, IO, SP>(const Lds1dSpecArgs&, hipStream_t);

#define HY_LDS1D_EXTERN(M, IO, SP)                                                               \
    extern template hyena_status lds1d_forward_launch<M, IO, SP>(const Lds1dFwdArgs&, bool,      \
                                                                 hipStream_t);                   \
    extern template hyena_status lds1d_spectrum_launch<M, IO, SP>(const Lds1dSpecArgs&,          \
                                                                  hipStream_t);

}  // namespace hy
