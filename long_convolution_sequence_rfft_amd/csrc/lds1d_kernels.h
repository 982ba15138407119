// lds1d_kernels.h -- single-workgroup FFT convolution chain for transforms of
// length M <= 16384 (sequence length N <= 8192), in two forms: one real
// channel per half-length complex transform (N = M/2, and periodic plans;
// hyena_lds1d_real_*), or a channel pair per full-length complex transform
// (any other N; hyena_lds1d_forward / hyena_lds1d_spectrum).
//
// Channel-pair form: one workgroup owns one (batch row b, channel pair c,
// c+1); the two real channels ride in one complex signal, and the whole
// order-N chain stays in registers and LDS:
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
    const float2* twm;  // single-channel kernels: exp(-2 pi i k / M), k < M/2
    int64_t N, d, npairs, nblocks, B;
    int32_t order;
    int32_t last_gate_out;  // single-channel kernels: the last gate is applied by the stage-out
    TwOffsets tw_off;
};

struct Lds1dSpecArgs {
    const void* h;
    void* spec;
    const float2* tw;
    const float2* twm;
    int64_t N, d, npairs, nblocks;
    TwOffsets tw_off;
};

// How the forward pass reaches the activations (channels last in memory).
//   IO_PAIR: channel-pair kernel (hyena_lds1d_forward), each lane loading its
//            own channel pair from the channels-last rows.  The general form:
//            any N (including lengths below M/2) and any d.
//   IO_REAL: single-channel kernels (hyena_lds1d_real_forward) on u, gates and
//            y staged channel-major ([B][d][N]) in the workspace; used when
//            N = M/2.
enum Lds1dIo { IO_PAIR = 0, IO_REAL = 3 };

// Channel-pair form: one workgroup owns one (batch row b, channel pair c,
// c+1) and reads and writes the channels-last rows directly, masking the
// samples past N and a missing partner channel.
template <int M, typename IO, typename SP>
__global__ void __launch_bounds__(FftShape<M>::T, 2) hyena_lds1d_forward(Lds1dFwdArgs a)
{
    using S = FftShape<M>;
    constexpr int T = S::T, PTS = S::PTS, R0 = S::R0, LW = S::LW;
    // [re block | im block]: real and imaginary parts of an element are LW
    // words apart and share one base address
    __shared__ float smem[2 * LW];

    const int tau = threadIdx.x;
    const int64_t lin = xcd_remap(blockIdx.x, a.nblocks);
    // batch row fastest: the B workgroups of one channel pair run back to
    // back on one XCD, so the pair's spectrum is fetched from HBM once and
    // then found in that XCD's L2
    const int64_t pc = lin / a.B;
    const int64_t b = lin - pc * a.B;
    const int64_t c0 = 2 * pc;
    const bool has_b = c0 + 1 < a.d;
    const uint32_t dd = (uint32_t)a.d;
    const uint32_t N = (uint32_t)a.N;
    const int j1 = tau, j2 = tau ? 2 * T - tau : T;
    const float inv2M = 0.5f / (float)M;
    float* re = smem;
    float* im = smem + LW;
    const int64_t row0 = b * a.N * a.d + c0;

    float2 v[PTS];
    const IO* ubase = static_cast<const IO*>(a.u) + row0;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q)
#pragma unroll
        for (int r = 0; r < R0 / 2; ++r) {
            const uint32_t t = tau + q * T + r * (M / R0);
            v[q * R0 + r] = t < N ? load_pair<IO, false>(ubase + (size_t)t * dd, has_b)
                                  : make_float2(0.0f, 0.0f);
        }

    for (int n = 0; n < a.order; ++n) {
        const SP* spec = static_cast<const SP*>(a.spec) +
                         ((int64_t)n * a.npairs + pc) * (int64_t)(M / 2) * kEntryElems;
        typename EntryRaw<SP>::type ent[S::RL];
        fwd_transform<M>(v, re, im, a.tw, a.tw_off, tau, j1, j2, n > 0,
                         [&] { load_entries<M, SP>(ent, spec, tau); });

        const float Da = a.D[(int64_t)n * a.d + c0];
        const float Db = has_b ? a.D[(int64_t)n * a.d + c0 + 1] : 0.0f;
        spectral_product<M, SP>(v, ent, tau, (Da + Db) * inv2M, (Da - Db) * inv2M);

        const IO* g = static_cast<const IO*>(a.gates[n]) + row0;
        float2 gv[S::Q0][R0 / 2];
        inv_transform<M>(v, re, im, a.tw, a.tw_off, tau, j1, j2, [&] {
#pragma unroll
            for (int q = 0; q < S::Q0; ++q)
#pragma unroll
                for (int r = 0; r < R0 / 2; ++r) {
                    const uint32_t t = tau + q * T + r * (M / R0);
                    gv[q][r] = t < N ? load_pair<IO, false>(g + (size_t)t * dd, has_b)
                                     : make_float2(0.0f, 0.0f);
                }
        });
#pragma unroll
        for (int q = 0; q < S::Q0; ++q)
#pragma unroll
            for (int r = 0; r < R0 / 2; ++r) {
                float2& x = v[q * R0 + r];
                x = make_float2(x.x * gv[q][r].x, x.y * gv[q][r].y);
            }
    }

    IO* ybase = static_cast<IO*>(a.y) + row0;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q)
#pragma unroll
        for (int r = 0; r < R0 / 2; ++r) {
            const uint32_t t = tau + q * T + r * (M / R0);
            if (t < N) store_pair<IO, false>(ybase + (size_t)t * dd, v[q * R0 + r], has_b);
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
    __shared__ float smem[2 * S::LW];
    float* sre = smem;
    float* sim = smem + S::LW;

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

// ---------------------------------------------------------------------------
// Single-channel forms (transform length L = M/2, one real channel per
// workgroup; see real_product).  Half the LDS of the channel-pair kernel, so
// twice as many workgroups share a CU and one's exchanges and barriers
// overlap another's arithmetic.  Activations are staged channel-major
// ([B][d][N]); sample pair (2m, 2m+1) is one aligned PairRaw element.
// ---------------------------------------------------------------------------
// CIRC: periodic boundary -- the transform is the sequence itself (M = N,
// no zero padding), so every sample is loaded and every output kept.
template <int L, typename IO, typename SP, bool CIRC>
__global__ void __launch_bounds__(FftShape<L>::T, 2) hyena_lds1d_real_forward(Lds1dFwdArgs a)
{
    using S = FftShape<L>;
    constexpr int T = S::T, PTS = S::PTS, R0 = S::R0, LW = S::LW;
    constexpr int RIN = CIRC ? R0 : R0 / 2;  // live R0-pass samples per butterfly
    __shared__ float smem[2 * LW];
    float* re = smem;
    float* im = smem + LW;

    const int tau = threadIdx.x;
    const int64_t lin = xcd_remap(blockIdx.x, a.nblocks);
    // batch row fastest: the B workgroups of a channel share its spectrum in L2
    const int64_t c = lin / a.B;
    const int64_t b = lin - c * a.B;
    const int j1 = tau, j2 = tau ? 2 * T - tau : T;
    const int64_t row = (b * a.d + c) * a.N;  // this (b, c)'s run in the staged tensors
    const float2 wbase = a.twm[tau ? tau : T];
    const float invL = 1.0f / (float)L;

    float2 v[PTS];
    const IO* ubase = static_cast<const IO*>(a.u) + row;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) {
        const uint32_t lane_off = (uint32_t)(tau + q * T) * 2u * (uint32_t)sizeof(IO);
#pragma unroll
        for (int r = 0; r < RIN; ++r)
            v[q * R0 + r] = widen_pair<IO>(load_pair_raw(ubase + (size_t)r * (L / R0) * 2, lane_off));
    }

    for (int n = 0; n < a.order; ++n) {
        const SP* spec = static_cast<const SP*>(a.spec) +
                         ((int64_t)n * a.d + c) * (int64_t)(L / 2) * kEntryElems;
        typename EntryRaw<SP>::type ent[S::RL];
        fwd_transform<L, !CIRC>(v, re, im, a.tw, a.tw_off, tau, j1, j2, n > 0,
                         [&] { load_entries<L, SP>(ent, spec, tau); });
        real_product<L, SP>(v, ent, tau, a.D[(int64_t)n * a.d + c] * invL, wbase);

        const IO* g = static_cast<const IO*>(a.gates[n]) + row;
        // the last gate may be left to the stage-out kernel (uniform)
        const bool gate_here = n + 1 < a.order || !a.last_gate_out;
        typename PairRaw<IO>::type graw[S::Q0][RIN];
        inv_transform<L, !CIRC>(v, re, im, a.tw, a.tw_off, tau, j1, j2, [&] {
            if (!gate_here) return;
#pragma unroll
            for (int q = 0; q < S::Q0; ++q) {
                const uint32_t lane_off = (uint32_t)(tau + q * T) * 2u * (uint32_t)sizeof(IO);
#pragma unroll
                for (int r = 0; r < RIN; ++r)
                    graw[q][r] = load_pair_raw(g + (size_t)r * (L / R0) * 2, lane_off);
            }
        });
        if (gate_here) {
#pragma unroll
            for (int q = 0; q < S::Q0; ++q)
#pragma unroll
                for (int r = 0; r < RIN; ++r) {
                    const float2 gg = widen_pair<IO>(graw[q][r]);
                    float2& x = v[q * R0 + r];
                    x = make_float2(x.x * gg.x, x.y * gg.y);
                }
        }
    }

    IO* ybase = static_cast<IO*>(a.y) + row;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) {
        const uint32_t lane_off = (uint32_t)(tau + q * T) * 2u * (uint32_t)sizeof(IO);
#pragma unroll
        for (int r = 0; r < RIN; ++r)
            store_pair_at(ybase + (size_t)r * (L / R0) * 2, lane_off, v[q * R0 + r]);
    }
}

// Filter spectrum, single-channel form: one workgroup per (filter n, channel
// c); entries (S, Dl) / L, the 1/L of the unscaled inverse transform folded in.
// CIRC: periodic boundary (N = M taps, no zero padding).
template <int L, typename IO, typename SP, bool CIRC>
__global__ void __launch_bounds__(FftShape<L>::T, 2) hyena_lds1d_real_spectrum(Lds1dSpecArgs a)
{
    using S = FftShape<L>;
    constexpr int T = S::T, PTS = S::PTS, R0 = S::R0;
    constexpr int RIN = CIRC ? R0 : R0 / 2;
    __shared__ float smem[2 * S::LW];
    const int tau = threadIdx.x;
    const int64_t lin = blockIdx.x;  // n * d + c
    const int j1 = tau, j2 = tau ? 2 * T - tau : T;

    float2 v[PTS];
    const IO* h = static_cast<const IO*>(a.h) + lin * a.N;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) {
        const uint32_t lane_off = (uint32_t)(tau + q * T) * 2u * (uint32_t)sizeof(IO);
#pragma unroll
        for (int r = 0; r < RIN; ++r)
            v[q * R0 + r] = widen_pair<IO>(load_pair_raw(h + (size_t)r * (L / R0) * 2, lane_off));
    }
    fwd_transform<L, !CIRC>(v, smem, smem + S::LW, a.tw, a.tw_off, tau, j1, j2, false, [] {});
    SP* spec = static_cast<SP*>(a.spec) + lin * (int64_t)(L / 2) * kEntryElems;
    store_real_entries<L, SP>(v, spec, tau, 1.0f / (float)L, a.twm[tau ? tau : T]);
}

template <int L, typename IO, typename SP, bool CIRC>
hyena_status lds1d_real_forward_launch(const Lds1dFwdArgs& a, hipStream_t s)
{
    HY_LAUNCH(kernel_label("hyena_lds1d_real_forward", L, type_label<IO>(), type_label<SP>(), CIRC),
              (hyena_lds1d_real_forward<L, IO, SP, CIRC>), dim3((unsigned)a.nblocks),
              dim3(FftShape<L>::T), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

template <int L, typename IO, typename SP, bool CIRC>
hyena_status lds1d_real_spectrum_launch(const Lds1dSpecArgs& a, hipStream_t s)
{
    HY_LAUNCH(kernel_label("hyena_lds1d_real_spectrum", L, type_label<IO>(), type_label<SP>(), CIRC),
              (hyena_lds1d_real_spectrum<L, IO, SP, CIRC>), dim3((unsigned)a.nblocks),
              dim3(FftShape<L>::T), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

template <int M, typename IO, typename SP>
hyena_status lds1d_forward_launch(const Lds1dFwdArgs& a, hipStream_t s)
{
    HY_LAUNCH(kernel_label("hyena_lds1d_forward", M, type_label<IO>(), type_label<SP>()),
              (hyena_lds1d_forward<M, IO, SP>), dim3((unsigned)a.nblocks), dim3(FftShape<M>::T), 0,
              s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

template <int M, typename IO, typename SP>
hyena_status lds1d_spectrum_launch(const Lds1dSpecArgs& a, hipStream_t s)
{
    HY_LAUNCH(kernel_label("hyena_lds1d_spectrum", M, type_label<IO>(), type_label<SP>()),
              (hyena_lds1d_spectrum<M, IO, SP>), dim3((unsigned)a.nblocks), dim3(FftShape<M>::T), 0, s,
              a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

// Spectrum-launch arguments of a plan (everything but the taps pointer).
Lds1dSpecArgs lds1d_spec_args(const Plan& p, void* H, const void* ws);

#define HY_LDS1D_SIZES(X, IO, SP) \
    X(8, IO, SP) X(16, IO, SP) X(32, IO, SP) X(64, IO, SP) X(128, IO, SP) X(256, IO, SP) \
    X(512, IO, SP) X(1024, IO, SP) X(2048, IO, SP) X(4096, IO, SP) X(8192, IO, SP)       \
    X(16384, IO, SP)

#define HY_LDS1D_REAL_SIZES(X, IO, SP) \
    X(8, IO, SP) X(16, IO, SP) X(32, IO, SP) X(64, IO, SP) X(128, IO, SP) X(256, IO, SP) \
    X(512, IO, SP) X(1024, IO, SP) X(2048, IO, SP) X(4096, IO, SP) X(8192, IO, SP)

#define HY_LDS1D_INSTANTIATE(M, IO, SP)                                                      \
    template hyena_status lds1d_forward_launch<M, IO, SP>(const Lds1dFwdArgs&, hipStream_t);    \
    template hyena_status lds1d_spectrum_launch<M, IO, SP>(const Lds1dSpecArgs&, hipStream_t);

#define HY_LDS1D_EXTERN(M, IO, SP)                                                               \
    extern template hyena_status lds1d_forward_launch<M, IO, SP>(const Lds1dFwdArgs&,            \
                                                                 hipStream_t);                   \
    extern template hyena_status lds1d_spectrum_launch<M, IO, SP>(const Lds1dSpecArgs&,          \
                                                                  hipStream_t);

// single-channel kernels: (L, IO, SP) x {zero-padded, periodic}
#define HY_LDS1D_REAL_INST_B(L, IO, SP, CIRC, EXT)                                                 \
    EXT template hyena_status lds1d_real_forward_launch<L, IO, SP, CIRC>(const Lds1dFwdArgs&,      \
                                                                        hipStream_t);             \
    EXT template hyena_status lds1d_real_spectrum_launch<L, IO, SP, CIRC>(const Lds1dSpecArgs&,    \
                                                                         hipStream_t);

#define HY_LDS1D_REAL_INSTANTIATE(L, IO, SP) HY_LDS1D_REAL_INST_B(L, IO, SP, false, )
#define HY_LDS1D_CIRC_INSTANTIATE(L, IO, SP) HY_LDS1D_REAL_INST_B(L, IO, SP, true, )
#define HY_LDS1D_REAL_EXTERN(L, IO, SP)                 \
    HY_LDS1D_REAL_INST_B(L, IO, SP, false, extern)      \
    HY_LDS1D_REAL_INST_B(L, IO, SP, true, extern)

}  // namespace hy
