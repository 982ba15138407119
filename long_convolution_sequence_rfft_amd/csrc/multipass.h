// multipass.h -- transforms too long for one workgroup, split into passes
// that exchange data through a workspace in device memory.
//
//   1D (four-step, "Bailey"): M = M1 M2, sample t = M2 n1 + n2, bin
//     k = k1 + M1 k2.  DFT_M = length-M1 column DFTs over n1, a twiddle
//     W_M^{n2 k1}, length-M2 row DFTs over n2.
//   2D (row-column): a P1 x P2 (= 2X x 2Y) periodic grid; length-P2 DFTs
//     along q for every grid row p, then length-P1 DFTs along p.
//   3D: a P1 x P2 x P3 (= 2X x 2Y x 2Z) grid; length-P3 DFTs along z (the
//     outer pass, rows (x, y)), length-P2 DFTs along y (a middle pass between
//     two intermediates), then length-P1 DFTs along x (the inner pass, whose
//     outer index is the composite bin (ky, kz)).
// ("Hyena -- Long Convolutions Math", section "The convolution theorem";
// "How HyenaND works", section "The convolution theorem (FFT)": the ND
// transform on the native grid, here as 1D transforms along each axis.)
//
// Both share one structure.  The "outer" axis (n1 / q) is the one the
// channels-last activations are read and written along; the "inner" axis
// (n2 / p) is transformed in a separate pass.  The workspace holds, per
// channel pair, F[o][a]: outer spectral index a (k1 / kq) fastest, inner
// index o (n2 / p).  An order-N chain over one chunk of channel pairs is
//
//   OUTER_IN   activations u -> forward outer DFTs (-> twiddle) -> F
//   INNER      F rows -> forward inner DFT -> x (P, Q) -> inverse inner DFT -> F
//   OUTER_MID  F -> (conj twiddle ->) inverse outer DFT -> gate_n -> forward -> F
//   ...
//   OUTER_OUT  F -> (conj twiddle ->) inverse outer DFT -> gate_N -> y
//
// so each transform costs one workspace round trip.  Outer-pass workgroups
// own KP channel pairs x C outer columns and move activations in full
// 128-byte rows through LDS (the channel pair of one workgroup would
// otherwise use 4-8 bytes of every cache line it touches).  Inner-pass
// workgroups own one pair x U mirror-paired units.
//
// The transforms here keep every pass on the regular butterfly assignment
// and leave spectra in natural order in LDS; the mirror pairing of the
// channel-pair product (bin k with bin -k) is then plain index arithmetic.
#pragma once

#include "stockham.h"

namespace hy {

// ---------------------------------------------------------------------------
// One transform of length L in an LDS region, T = L/32 threads, registers in
// the R0-pass layout: v[q R0 + r] is sample tau + q T + r L/R0.
// ---------------------------------------------------------------------------

// Forward transform from registers (R0-pass inputs; HALF_IN: only r < R0/2
// hold data, the rest is zero padding) to natural-order bins in the region.
// The caller provides the WAR barrier before the first write when needed.
// TO_REGS: stop after the last pass's arithmetic; v[q RL + s] then holds bin
// (tau + q T) + s L/RL (lanes of one transform hold consecutive bins).
template <int L, bool HALF_IN, bool TO_REGS = false>
__device__ __forceinline__ void fwd_regs_to_lds(float2* v, float* sre, float* sim, const float2* tw,
                                                TwOffsets o, int tau)
{
    using S = FftShape<L>;
    constexpr int T = S::T, R0 = S::R0, R1 = S::R1, RL = S::RL;
    constexpr int QL = S::PTS / RL;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) dft<R0, -1, HALF_IN, false>(&v[q * R0]);
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) lds_write<R0, 1>(sre, sim, &v[q * R0], tau + q * T);
    if constexpr (R1 > 1) {
        float2 w1[R1 - 1];
        load_tw<R1, R0>(w1, tw + o.f1, tau & (R0 - 1));
        __syncthreads();
#pragma unroll
        for (int q = 0; q < S::Q1; ++q) lds_read<R1, L>(sre, sim, &v[q * R1], tau + q * T);
#pragma unroll
        for (int q = 0; q < S::Q1; ++q) {
            apply_tw<R1, -1>(&v[q * R1], w1);
            dft<R1, -1>(&v[q * R1]);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < S::Q1; ++q) lds_write<R1, R0>(sre, sim, &v[q * R1], tau + q * T);
    }
    constexpr int NSL = L / RL;
    float2 wl[QL][RL - 1];
#pragma unroll
    for (int q = 0; q < QL; ++q) load_tw<RL, NSL>(wl[q], tw + o.fL, tau + q * T);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QL; ++q) {
        lds_read<RL, L>(sre, sim, &v[q * RL], tau + q * T);
        apply_tw<RL, -1>(&v[q * RL], wl[q]);
        dft<RL, -1>(&v[q * RL]);
    }
    if constexpr (TO_REGS) return;
    __syncthreads();
    // last pass: NS = L/RL, so output s of butterfly j lands at j + s L/RL
#pragma unroll
    for (int q = 0; q < QL; ++q) lds_write<RL, NSL>(sre, sim, &v[q * RL], tau + q * T);
}

// Inverse (unscaled) transform from natural-order bins in the region to the
// R0-pass register layout.  HALF_OUT: only samples < L/2 are produced
// (v[q R0 + s], s < R0/2).  The caller provides the RAW barrier before.
// FROM_REGS: the bins are already in registers, v[q RL + r] = bin
// (tau + q T) + r L/RL (the layout fwd_regs_to_lds<..., true> leaves).
template <int L, bool HALF_OUT, bool FROM_REGS = false>
__device__ __forceinline__ void inv_lds_to_regs(float2* v, float* sre, float* sim, const float2* tw,
                                                TwOffsets o, int tau)
{
    using S = FftShape<L>;
    constexpr int T = S::T, R0 = S::R0, R1 = S::R1, RL = S::RL;
    constexpr int QL = S::PTS / RL;
#pragma unroll
    for (int q = 0; q < QL; ++q) {
        if constexpr (!FROM_REGS) lds_read<RL, L>(sre, sim, &v[q * RL], tau + q * T);
        dft<RL, +1>(&v[q * RL]);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QL; ++q) lds_write<RL, 1>(sre, sim, &v[q * RL], tau + q * T);
    if constexpr (R1 > 1) {
        float2 w1[R1 - 1];
        load_tw<R1, RL>(w1, tw + o.i1, tau & (RL - 1));
        __syncthreads();
#pragma unroll
        for (int q = 0; q < S::Q1; ++q) lds_read<R1, L>(sre, sim, &v[q * R1], tau + q * T);
#pragma unroll
        for (int q = 0; q < S::Q1; ++q) {
            apply_tw<R1, +1>(&v[q * R1], w1);
            dft<R1, +1>(&v[q * R1]);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < S::Q1; ++q) lds_write<R1, RL>(sre, sim, &v[q * R1], tau + q * T);
    }
    constexpr int NS0 = L / R0;
    float2 w0[S::Q0][R0 - 1];
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) load_tw<R0, NS0>(w0[q], tw + o.i0, tau + q * T);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) {
        lds_read<R0, L>(sre, sim, &v[q * R0], tau + q * T);
        apply_tw<R0, +1>(&v[q * R0], w0[q]);
        dft<R0, +1, false, HALF_OUT>(&v[q * R0]);
    }
}

// R0-pass registers <-> natural order in the region (for the live half only
// when HALF).  No barrier inside.
template <int L, bool HALF>
__device__ __forceinline__ void regs_to_lds(const float2* v, float* sre, float* sim, int tau)
{
    using S = FftShape<L>;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q)
#pragma unroll
        for (int r = 0; r < (HALF ? S::R0 / 2 : S::R0); ++r) {
            const int i = lpad(tau + q * S::T + r * (L / S::R0));
            sre[i] = v[q * S::R0 + r].x;
            sim[i] = v[q * S::R0 + r].y;
        }
}

template <int L, bool HALF>
__device__ __forceinline__ void lds_to_regs(float2* v, const float* sre, const float* sim, int tau)
{
    using S = FftShape<L>;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q)
#pragma unroll
        for (int r = 0; r < (HALF ? S::R0 / 2 : S::R0); ++r) {
            const int i = lpad(tau + q * S::T + r * (L / S::R0));
            v[q * S::R0 + r] = make_float2(sre[i], sim[i]);
        }
}

// ---------------------------------------------------------------------------
// geometry shared by the passes
// ---------------------------------------------------------------------------
struct MpGeom {
    int64_t N, d, npairs, B;
    int32_t four_step;  // 1: 1D four-step, 0: 2D row-column
    int32_t full;       // periodic plan: unpadded columns (every sample live)
    // sample index of (outer-axis position a, inner position o):
    //   four-step t = M2 a + o ;  2D t = Y o + a
    int64_t sa, so;
    int32_t La, Lb;        // outer / inner transform lengths (M1, M2 or P2, P1)
    int32_t Lb_live;       // inner positions held in F (M2, or X for 2D)
    int32_t kp_log2;       // pairs per outer workgroup (power of two)
    int32_t groups_per_b;  // pair groups per batch row = ceil(npairs / KP)
    int64_t group0;        // first pair group of this chunk (flattened b * G + g)
    int64_t ngroups;       // pair groups in this chunk
    int64_t pair_bytes;    // workspace bytes per pair slot
    int32_t order_n;       // filter index for INNER and the gate index for OUTER_MID/OUT
    TwOffsets tw_a, tw_b;  // twiddle tables of the outer / inner lengths
    int64_t tw_step;       // float2 offset of the W_M^{n2 k1} table (four-step)
    // 3D: grid sides (outer pass: filter tap placement and rows (x, y)) and,
    // for the inner pass, the length P3 of the composite outer index
    // a = ky P3 + kz
    int32_t three_d;
    int32_t gx, gy, gz;
    int32_t Lc;
};

__device__ __forceinline__ void pair_of_slot(const MpGeom& g, int64_t group, int kp, int64_t& b,
                                             int64_t& p, bool& live)
{
    b = group / g.groups_per_b;
    p = (group - b * g.groups_per_b) * ((int64_t)1 << g.kp_log2) + kp;
    live = p < g.npairs;
}

}  // namespace hy
