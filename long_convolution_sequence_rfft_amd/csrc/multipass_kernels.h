// multipass_kernels.h -- the outer, inner and (3D) middle passes of the
// four-step (1D) and row-column (2D, 3D) paths; see multipass.h for the
// structure.
#pragma once

#include "multipass.h"

namespace hy {

// OUTER_IN3 / OUTER_OUT3: OUTER_IN / OUTER_OUT with the HyenaND mixer's
// 3x3x3 short convolutions of a 3D grid (kept apart so that the plain passes
// compile without that code)
// OUTER_SPEC_IMP: OUTER_SPEC with the taps evaluated from an implicit
// filter's hidden features (four-step path)
enum OuterMode { OUTER_IN = 0, OUTER_MID = 1, OUTER_OUT = 2, OUTER_SPEC = 3, OUTER_IN3 = 4,
                 OUTER_OUT3 = 5, OUTER_SPEC_IMP = 6 };
enum InnerMode { INNER_CHAIN = 0, INNER_SPEC = 1 };

// Workgroup of kMpThreads threads, one length-L transform per
// FftShape<L>::T threads.  256 threads and 16384 points (68 KB of LDS) per
// workgroup let two workgroups share a CU, so one's barriers and memory
// waits overlap the other's arithmetic.
// Regions are RS = LW rounded up to an odd word count apart, so the staging
// loops (adjacent lanes -> same position of adjacent transforms) spread
// over the LDS banks.
constexpr int kMpThreads = 256;
// widest hidden layer of an implicit filter (W3 rows staged by OUTER_SPEC_IMP)
constexpr int kImpHidden = 256;
template <int L>
struct MpShape {
    static constexpr int T = FftShape<L>::T;
    static constexpr int NF = kMpThreads / T;
    static constexpr int LW = FftShape<L>::LW | 1;
};

// HyenaND mixer inputs ("How HyenaND works", section "Putting it together:
// the HyenaND operator"): with `on`, OUTER_IN reads q . SiLU(k) and OUTER_OUT
// gates with SiLU(v), where q, k, v first pass a depthwise short convolution
// with zero padding: 3x3 on an X x Y grid, 3x3x3 on an X x Y x Z grid.
struct BlockArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* sw;  // [3][d][3][3] (2D) or [3][d][3][3][3] (3D) taps of q, k, v
    const float* sb;  // [3][d] biases, or NULL
    int32_t on;
};

// Implicit filter's output layer for OUTER_SPEC_IMP: taps of filter row
// o = n d + c at sample t are exp(-alpha[o] t) (b3[o] + W3[o] . z2[t]).
struct ImpOuter {
    const float* z2;  // hidden features [N][hp] (row-major)
    const float* W3;  // [order d][H]
    const float* b3;
    const float* alpha;
    int32_t H, hp;
    int32_t n;  // filter index
};

struct OuterArgs {
    MpGeom g;
    const void* act;   // u (IN), gate (MID, OUT)
    void* out;         // y (OUT)
    const void* filt;  // filter taps (SPEC), this filter index
    float2* F;         // workspace intermediate of this chunk
    const float2* tw;
    BlockArgs blk;
    ImpOuter imp;
};

struct InnerArgs {
    MpGeom g;
    float2* F;
    const void* spec;  // spectrum of this filter index, entries [pair][unit][e] (CHAIN)
    void* spec_out;    // same layout, written (SPEC)
    const float* D;    // feedthrough of this filter index [d]
    const float2* tw;
};

// Streams read once per forward (activations, gates, spectrum entries):
// plain loads, or carrying the nontemporal hint with HY_STREAM_NT, fixed at
// build time.
#ifndef HY_STREAM_NT
#define HY_STREAM_NT 0
#endif
template <typename T>
__device__ __forceinline__ T stream_load(const T* p)
{
    if constexpr (HY_STREAM_NT != 0 && sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)));
    } else if constexpr (HY_STREAM_NT != 0 && sizeof(T) == 8) {
        typedef unsigned u2v __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u2v*>(p)));
    } else if constexpr (HY_STREAM_NT != 0 && sizeof(T) == 16) {
        typedef unsigned u4v __attribute__((ext_vector_type(4)));
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p)));
    } else {
        return *p;
    }
}

// Sample of channel pair (c0, c0+1) at activation row `row` (element offset).
template <typename IO>
__device__ __forceinline__ float2 act_load(const IO* base, int64_t row, int64_t c0, int64_t d)
{
    const IO* r = base + row * d + c0;
    if (c0 + 1 < d) {
        if ((d & 1) == 0)
            return widen_pair<IO>(stream_load(reinterpret_cast<const typename PairRaw<IO>::type*>(r)));
        return make_float2(ld1<IO>(r), ld1<IO>(r + 1));
    }
    return make_float2(ld1<IO>(r), 0.0f);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Short-conv taps of one channel pair (c0, c0 + 1) of tensor j (0 q, 1 k,
// 2 v): NT = 9 (3x3) or 27 (3x3x3) taps per channel.
template <int NT>
struct PairTaps {
    float w[2][NT];
    float b[2];
};

template <int NT>
__device__ __forceinline__ PairTaps<NT> pair_taps(const BlockArgs& k, int j, int64_t c0, int64_t d)
{
    PairTaps<NT> t;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bool live = c0 + h < d;
        const int64_t c = live ? c0 + h : c0;
#pragma unroll
        for (int i = 0; i < NT; ++i) t.w[h][i] = live ? k.sw[((int64_t)j * d + c) * NT + i] : 0.0f;
        t.b[h] = (live && k.sb) ? k.sb[(int64_t)j * d + c] : 0.0f;
    }
    return t;
}

// Depthwise 3x3 short convolution of one channel pair at grid point (p, q)
// of batch row b: row = b X Y + p Y + q is the point's activation row.
template <typename IO>
__device__ __forceinline__ float2 short_conv(const IO* x, const PairTaps<9>& t, int64_t row,
                                             int64_t p, int64_t q, int64_t X, int64_t Y,
                                             int64_t c0, int64_t d)
{
    float2 acc = make_float2(t.b[0], t.b[1]);
#pragma unroll
    for (int a = -1; a <= 1; ++a)
#pragma unroll
        for (int e = -1; e <= 1; ++e) {
            if (p + a < 0 || p + a >= X || q + e < 0 || q + e >= Y) continue;
            const float2 xv = act_load<IO>(x, row + a * Y + e, c0, d);
            acc.x = fmaf(t.w[0][(a + 1) * 3 + e + 1], xv.x, acc.x);
            acc.y = fmaf(t.w[1][(a + 1) * 3 + e + 1], xv.y, acc.y);
        }
    return acc;
}

// Depthwise 3x3x3 short convolution of one channel pair at grid point
// (p, q, r) of batch row b: row = b X Y Z + (p Y + q) Z + r.
template <typename IO>
__device__ __forceinline__ float2 short_conv3(const IO* x, const PairTaps<27>& t, int64_t row,
                                              int64_t p, int64_t q, int64_t r, int64_t X,
                                              int64_t Y, int64_t Z, int64_t c0, int64_t d)
{
    float2 acc = make_float2(t.b[0], t.b[1]);
#pragma unroll
    for (int a = -1; a <= 1; ++a)
#pragma unroll
        for (int e = -1; e <= 1; ++e)
#pragma unroll
            for (int f = -1; f <= 1; ++f) {
                if (p + a < 0 || p + a >= X || q + e < 0 || q + e >= Y || r + f < 0 || r + f >= Z)
                    continue;
                const float2 xv = act_load<IO>(x, row + (a * Y + e) * Z + f, c0, d);
                const int i = ((a + 1) * 3 + e + 1) * 3 + f + 1;
                acc.x = fmaf(t.w[0][i], xv.x, acc.x);
                acc.y = fmaf(t.w[1][i], xv.y, acc.y);
            }
    return acc;
}

template <typename IO>
__device__ __forceinline__ void act_store(IO* base, int64_t row, int64_t c0, int64_t d, float2 v)
{
    IO* r = base + row * d + c0;
    if (c0 + 1 < d) {
        if ((d & 1) == 0) {
            store_pair<IO, true>(r, v, true);
        } else {
            st1<IO>(r, v.x);
            st1<IO>(r + 1, v.y);
        }
    } else {
        st1<IO>(r, v.x);
    }
}

// Accesses to the intermediate F: plain, or carrying the nontemporal hint
// (HY_F_NT bit 0 on loads, bit 1 on stores), fixed at build time.
#ifndef HY_F_NT
#define HY_F_NT 0
#endif
typedef float f2vec __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 f_load(const float2* p)
{
    if constexpr ((HY_F_NT & 1) != 0) {
        const f2vec t = __builtin_nontemporal_load(reinterpret_cast<const f2vec*>(p));
        return make_float2(t.x, t.y);
    } else {
        return *p;
    }
}
__device__ __forceinline__ void f_store(float2* p, float2 v)
{
    if constexpr ((HY_F_NT & 2) != 0) {
        f2vec t;
        t.x = v.x;
        t.y = v.y;
        __builtin_nontemporal_store(t, reinterpret_cast<f2vec*>(p));
    } else {
        *p = v;
    }
}

// One outer column of F in the last-pass register layout of a length-L
// transform: v[q RL + r] <-> bin (tau + q T) + r L/RL, in natural bin order
// (the 3D path, whose middle pass reads these rows).  With `tw`, bins are
// multiplied by the four-step twiddle twstep[bin] (conjugated for DIR = +1,
// the inverse direction).  All loads are issued before any is used.
template <int L, int DIR>
__device__ __forceinline__ void load_column(float2* v, const float2* Fcol, const float2* twstep,
                                            int tau, bool live, bool tw)
{
    using S = FftShape<L>;
    constexpr int T = S::T, RL = S::RL, QL = S::PTS / RL;
    if (!live) {
#pragma unroll
        for (int i = 0; i < S::PTS; ++i) v[i] = make_float2(0.0f, 0.0f);
        return;
    }
#pragma unroll
    for (int q = 0; q < QL; ++q)
#pragma unroll
        for (int r = 0; r < RL; ++r) v[q * RL + r] = f_load(&Fcol[tau + q * T + r * (L / RL)]);
    if (tw) {
        float2 w[S::PTS];
#pragma unroll
        for (int q = 0; q < QL; ++q)
#pragma unroll
            for (int r = 0; r < RL; ++r) w[q * RL + r] = twstep[tau + q * T + r * (L / RL)];
#pragma unroll
        for (int i = 0; i < S::PTS; ++i) v[i] = ctw<DIR>(v[i], w[i]);
    }
}

template <int L>
__device__ __forceinline__ void store_column(const float2* v, float2* Fcol, const float2* twstep,
                                             int tau, bool tw)
{
    using S = FftShape<L>;
    constexpr int T = S::T, RL = S::RL, QL = S::PTS / RL;
    if (tw) {
        float2 w[S::PTS];
#pragma unroll
        for (int q = 0; q < QL; ++q)
#pragma unroll
            for (int r = 0; r < RL; ++r) w[q * RL + r] = twstep[tau + q * T + r * (L / RL)];
#pragma unroll
        for (int q = 0; q < QL; ++q)
#pragma unroll
            for (int r = 0; r < RL; ++r)
                f_store(&Fcol[tau + q * T + r * (L / RL)], ctw<-1>(v[q * RL + r], w[q * RL + r]));
    } else {
#pragma unroll
        for (int q = 0; q < QL; ++q)
#pragma unroll
            for (int r = 0; r < RL; ++r) f_store(&Fcol[tau + q * T + r * (L / RL)], v[q * RL + r]);
    }
}

// ---------------------------------------------------------------------------
// Mirror-paired F rows (1D and 2D paths).  An F row holds the L outer bins of
// one inner position with every bin beside its mirror (L - a) mod L: bins 0
// and L/2 at positions 0 and 1, and for 0 < a < L/2 bin a at 2a, bin L - a
// at 2a + 1.  The inner pass takes each bin with its mirror, so its
// workgroups read and write whole cache lines (in natural order the mirrors
// of an aligned run of columns straddle two lines, each shared with another
// workgroup).  The outer pass runs its last forward pass (and the inverse's
// first) on butterflies j1 = tau, j2 = 2T - tau (j2 = T for tau = 0), as the
// single-workgroup kernels do, so each thread holds bin pairs and moves each
// pair as one 16-byte access.
//
// Registers: v[s] = bin j1 + s L/RL, v[RL + s] = bin j2 + s L/RL.  Slot s of
// thread tau > 0 pairs v[s] (bin a = tau + s L/RL) with v[2RL-1-s] (bin
// L - a), at position 2a (s < RL/2, lower bin first) or 2 (L - a) (mirror
// first).  Thread 0 holds the self-mirrored butterflies 0 and T: slot
// s < RL/2 pairs v[RL+s] with v[2RL-1-s] (bins T + s L/RL and its mirror),
// slot RL/2 packs bins 0 and L/2 (v[0], v[RL/2]) at position 0, slots
// s > RL/2 pair v[RL-s] with v[s].  Every lane runs the same instructions;
// thread 0 differs only through selects.
// ---------------------------------------------------------------------------
template <int L>
struct PairSlot {
    float2 lo, hi;  // the two values as stored: position p and p + 1
    int pos;        // float2 position of lo
};

template <int L>
__device__ __forceinline__ PairSlot<L> pair_slot(const float2* v, int tau, int s)
{
    using S = FftShape<L>;
    constexpr int T = S::T, RL = S::RL, NSL = L / RL, H = RL / 2;
    const bool t0 = tau == 0;
    PairSlot<L> r;
    if (s < H) {
        const float2 A = t0 ? v[RL + s] : v[s];
        r.lo = A;
        r.hi = v[2 * RL - 1 - s];
        r.pos = 2 * ((t0 ? T : tau) + s * NSL);
    } else {
        const float2 B = t0 ? (s == H ? v[0] : v[RL - s]) : v[2 * RL - 1 - s];
        r.lo = B;
        r.hi = v[s];
        r.pos = (t0 && s == H) ? 0 : 2 * (L - tau - s * NSL);
    }
    return r;
}

// Bin index of the value stored at pos + k (k = 0, 1) of slot s: for the
// four-step twiddles, which depend on the bin.
template <int L>
__device__ __forceinline__ void pair_bins(int tau, int s, int& bin_lo, int& bin_hi)
{
    using S = FftShape<L>;
    constexpr int T = S::T, RL = S::RL, NSL = L / RL, H = RL / 2;
    const bool t0 = tau == 0;
    if (s < H) {
        bin_lo = (t0 ? T : tau) + s * NSL;
        bin_hi = L - bin_lo;
    } else if (t0 && s == H) {
        bin_lo = 0;
        bin_hi = L / 2;
    } else {
        bin_hi = tau + s * NSL;
        bin_lo = L - bin_hi;
    }
}

typedef float f4vec __attribute__((ext_vector_type(4)));

// Store the forward transform's outputs (registers as above) to an F row,
// times the four-step twiddle of each bin when `tw`.
// Frow and the twiddle table never overlap (the table lives at the start of
// the workspace, the rows after it), so twiddle loads may move ahead of the
// stores.
template <int L>
__device__ __forceinline__ void store_pairs(const float2* v, float2* __restrict__ Frow,
                                            const float2* __restrict__ twstep, int tau, bool tw)
{
    constexpr int RL = FftShape<L>::RL;
    // slots in groups of G: the group's twiddle loads are all issued before
    // its first store, so their latencies overlap (per slot they would not:
    // the compiler keeps loads behind earlier stores)
    constexpr int G = RL < 8 ? RL : 8;
#pragma unroll
    for (int s0 = 0; s0 < RL; s0 += G) {
        float2 wlo[G], whi[G];
        if (tw) {
#pragma unroll
            for (int i = 0; i < G; ++i) {
                int blo, bhi;
                pair_bins<L>(tau, s0 + i, blo, bhi);
                wlo[i] = twstep[blo];
                whi[i] = twstep[bhi];
            }
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            PairSlot<L> p = pair_slot<L>(v, tau, s0 + i);
            if (tw) {
                p.lo = ctw<-1>(p.lo, wlo[i]);
                p.hi = ctw<-1>(p.hi, whi[i]);
            }
            f4vec t;
            t.x = p.lo.x;
            t.y = p.lo.y;
            t.z = p.hi.x;
            t.w = p.hi.y;
            if constexpr ((HY_F_NT & 2) != 0)
                __builtin_nontemporal_store(t, reinterpret_cast<f4vec*>(Frow + p.pos));
            else
                *reinterpret_cast<f4vec*>(Frow + p.pos) = t;
        }
    }
}

// Load an F row into the inverse's first-pass registers (the layout
// store_pairs reads), times the conjugate four-step twiddle when `tw`.
template <int L>
__device__ __forceinline__ void load_pairs(float2* v, const float2* Frow, const float2* twstep,
                                           int tau, bool live, bool tw)
{
    using S = FftShape<L>;
    constexpr int RL = S::RL, H = RL / 2;
    const bool t0 = tau == 0;
    float2 lo[RL], hi[RL];
#pragma unroll
    for (int s = 0; s < RL; ++s) {
        int pos;
        if (s < H) pos = 2 * ((t0 ? S::T : tau) + s * (L / RL));
        else pos = (t0 && s == H) ? 0 : 2 * (L - tau - s * (L / RL));
        f4vec t = {0.0f, 0.0f, 0.0f, 0.0f};
        if (live) {
            if constexpr ((HY_F_NT & 1) != 0)
                t = __builtin_nontemporal_load(reinterpret_cast<const f4vec*>(Frow + pos));
            else
                t = *reinterpret_cast<const f4vec*>(Frow + pos);
        }
        lo[s] = make_float2(t.x, t.y);
        hi[s] = make_float2(t.z, t.w);
    }
    if (tw && live) {
#pragma unroll
        for (int s = 0; s < RL; ++s) {
            int blo, bhi;
            pair_bins<L>(tau, s, blo, bhi);
            lo[s] = ctw<+1>(lo[s], twstep[blo]);
            hi[s] = ctw<+1>(hi[s], twstep[bhi]);
        }
    }
    // general: v[s] = A of slot s (hi for s >= RL/2, lo below), v[2RL-1-s] =
    // the other.  Thread 0: v[0] = lo of slot RL/2, v[s] (0 < s < RL/2) = lo
    // of slot RL - s, v[RL + s] (s < RL/2) = lo of slot s.
#pragma unroll
    for (int s = 0; s < H; ++s) {
        v[s] = t0 ? (s == 0 ? lo[H] : lo[RL - s]) : lo[s];
        v[RL + s] = t0 ? lo[s] : lo[RL - 1 - s];
        v[H + s] = hi[H + s];
        v[2 * RL - 1 - s] = hi[s];
    }
}

// ---------------------------------------------------------------------------
// Outer pass.  Workgroup = KP pair slots x C outer columns (C KP = NF).
// blockIdx.x = column block * ngroups + group-in-chunk.
// ---------------------------------------------------------------------------
// PAIRED: the 1D and 2D paths, whose F rows hold mirror pairs (load_pairs);
// the 3D path keeps natural bin order for its middle pass.
template <int LA, typename IO, int MODE, bool HALF_SPEC, bool PAIRED>
__global__ void __launch_bounds__(kMpThreads, 2) hyena_mp_outer(OuterArgs a)
{
    using S = FftShape<LA>;
    using X = MpShape<LA>;
    constexpr int TA = X::T, NF = X::NF, LW = X::LW, R0 = S::R0;
    // HALF_SPEC: zero-padded transforms (only the first LA/2 samples of a
    // column are live, and the inverse keeps only those).  false: the
    // periodic plans' unpadded transforms on the chain modes, and the 2D
    // spectrum.  The 3D and implicit-filter modes are always padded.
    constexpr bool HALF_IN = (MODE == OUTER_SPEC || MODE == OUTER_IN || MODE == OUTER_MID ||
                              MODE == OUTER_OUT) ? HALF_SPEC : true;
    constexpr int NHALF = HALF_IN ? 1 : 2;  // column halves the activation tiles cover
    __shared__ float sre[NF * LW];
    __shared__ float sim[NF * LW];

    const MpGeom& g = a.g;
    const int KP = 1 << g.kp_log2;
    const int C = NF >> g.kp_log2;
    const int f = threadIdx.x / TA;
    const int tau = threadIdx.x - f * TA;
    const int gi = blockIdx.x % g.ngroups;
    const int cb = blockIdx.x / g.ngroups;
    const int kp = f & (KP - 1);
    const int o = cb * C + (f >> g.kp_log2);  // this transform's outer column
    // 1D and 2D: F rows hold mirror pairs, and the last forward / first
    // inverse pass runs on butterflies tau and 2T - tau (see load_pairs)
    constexpr bool paired = PAIRED;
    static_assert(!PAIRED || (MODE != OUTER_IN3 && MODE != OUTER_OUT3), "3D modes keep natural rows");
    const int j1 = tau, j2 = tau ? 2 * TA - tau : TA;
    constexpr bool IN = MODE == OUTER_IN || MODE == OUTER_IN3;
    constexpr bool OUT = MODE == OUTER_OUT || MODE == OUTER_OUT3;
    const int n_outer = (MODE == OUTER_SPEC || MODE == OUTER_SPEC_IMP) ? g.Lb : g.Lb_live;
    const bool col_live = o < n_outer;
    float* re = sre + f * LW;
    float* im = sim + f * LW;
    const int64_t group = g.group0 + gi;
    int64_t b, p;
    bool live;
    pair_of_slot(g, group, kp, b, p, live);
    float2* Fcol = a.F + ((int64_t)gi * KP + kp) * (g.pair_bytes / 8) + (int64_t)o * LA;
    const float2* twstep = a.tw + g.tw_step + (int64_t)(o - 1) * LA;  // W_M^{o a'}, o >= 1

    // cooperative move of activation rows between memory and the regions:
    // index -> (pair kp', outer sample s, column c'); KP consecutive lanes
    // cover one row's KP channel pairs (one cache line for KP = 16 f32).
    // Half hf of the column: samples s in [hf LA/2, (hf + 1) LA/2).
    // A thread's pair slot is the same in every element (KP divides the
    // thread count), so each call works it out once, outside the element
    // loop -- except in the 3D mixer modes, whose short convolutions leave
    // too few registers for it (they spill that way) and which recompute it
    // per element.
    constexpr bool SLOT_PER_ELEMENT = MODE == OUTER_IN3 || MODE == OUTER_OUT3;
    auto tile_rows_half = [&](int hf, auto&& fn) {
        constexpr int total = (LA / 2) * NF;  // = (LA/2) C KP
        static_assert(total % kMpThreads == 0 && kMpThreads % 16 == 0, "tile split");
        const int kq_t = (int)threadIdx.x & (KP - 1);
        int64_t bq_t = 0, pq_t = 0;
        bool lq_t = false;
        if constexpr (!SLOT_PER_ELEMENT) pair_of_slot(g, group, kq_t, bq_t, pq_t, lq_t);
#pragma unroll
        for (int it = 0; it < total / kMpThreads; ++it) {
            const int rest = ((int)threadIdx.x >> g.kp_log2) + it * (kMpThreads >> g.kp_log2);
            const int s = hf * (LA / 2) + rest % (LA / 2);
            const int cq = rest / (LA / 2);
            const int fq = cq * KP + kq_t;
            int64_t bq = bq_t, pq = pq_t;
            bool lq = lq_t;
            if constexpr (SLOT_PER_ELEMENT) pair_of_slot(g, group, kq_t, bq, pq, lq);
            const int oq = cb * C + cq;
            const int64_t t = g.sa * s + g.so * (int64_t)oq;
            fn(it, fq, s, pq, lq && oq < n_outer && t < g.N, bq * g.N + t);
        }
    };
    auto tile_rows = [&](auto&& fn) { tile_rows_half(0, fn); };

    // tile elements per thread in tile_rows
    constexpr int GT = (LA / 2) * NF / kMpThreads;
    float2 v[S::PTS];
    if constexpr (IN) {
        // all tile loads are issued before the first LDS store, so their
        // latencies overlap instead of adding up
        const IO* u = static_cast<const IO*>(a.act);
        float2 xin[GT];
        if constexpr (MODE == OUTER_IN3) {
            // the mixer on a 3D grid: rows o = x Y + y, samples s = z; q and
            // k are convolved one after the other so only one tap set is live
            int64_t bq0, pq0;
            bool l0;
            pair_of_slot(g, group, (int)(threadIdx.x & (KP - 1)), bq0, pq0, l0);
            const IO* qx = static_cast<const IO*>(a.blk.q);
            const IO* kx = static_cast<const IO*>(a.blk.k);
            auto conv3 = [&](const IO* x, const PairTaps<27>& t, int s, int64_t pq, int64_t row) {
                const int64_t o3 = (row % g.N) / g.so;
                const int64_t px = o3 / g.gy, py = o3 - px * g.gy;
                return short_conv3<IO>(x, t, row, px, py, s, g.gx, g.gy, g.gz, 2 * pq, g.d);
            };
            {
                const PairTaps<27> tq = pair_taps<27>(a.blk, 0, 2 * pq0, g.d);
                tile_rows([&](int it, int, int s, int64_t pq, bool ok, int64_t row) {
                    xin[it] = ok ? conv3(qx, tq, s, pq, row) : make_float2(0.0f, 0.0f);
                });
            }
            {
                const PairTaps<27> tk = pair_taps<27>(a.blk, 1, 2 * pq0, g.d);
                tile_rows([&](int it, int, int s, int64_t pq, bool ok, int64_t row) {
                    if (ok) {
                        const float2 kv = conv3(kx, tk, s, pq, row);
                        xin[it] = make_float2(xin[it].x * silu(kv.x), xin[it].y * silu(kv.y));
                    }
                });
            }
        } else if (a.blk.on) {
            // HyenaND mixer input q . SiLU(k) after the short convolutions;
            // this thread's channel pair is the same in every tile element
            int64_t bq0, pq0;
            bool l0;
            pair_of_slot(g, group, (int)(threadIdx.x & (KP - 1)), bq0, pq0, l0);
            const PairTaps<9> tq = pair_taps<9>(a.blk, 0, 2 * pq0, g.d);
            const PairTaps<9> tk = pair_taps<9>(a.blk, 1, 2 * pq0, g.d);
            const IO* qx = static_cast<const IO*>(a.blk.q);
            const IO* kx = static_cast<const IO*>(a.blk.k);
            tile_rows([&](int it, int, int s, int64_t pq, bool ok, int64_t row) {
                float2 z = make_float2(0.0f, 0.0f);
                if (ok) {
                    const int64_t pp = (row % g.N) / g.so, qq = s;
                    const float2 qv = short_conv<IO>(qx, tq, row, pp, qq, g.Lb_live, g.so, 2 * pq, g.d);
                    const float2 kv = short_conv<IO>(kx, tk, row, pp, qq, g.Lb_live, g.so, 2 * pq, g.d);
                    z = make_float2(qv.x * silu(kv.x), qv.y * silu(kv.y));
                }
                xin[it] = z;
            });
        } else {
            tile_rows([&](int it, int, int, int64_t pq, bool ok, int64_t row) {
                xin[it] = ok ? act_load<IO>(u, row, 2 * pq, g.d) : make_float2(0.0f, 0.0f);
            });
        }
        tile_rows([&](int it, int fq, int s, int64_t, bool, int64_t) {
            sre[fq * LW + lpad(s)] = xin[it].x;
            sim[fq * LW + lpad(s)] = xin[it].y;
        });
        if constexpr (!HALF_IN) {
            // unpadded (periodic) column: the second half of the samples
            static_assert(MODE == OUTER_IN, "unpadded columns on the plain chain only");
            tile_rows_half(1, [&](int it, int, int, int64_t pq, bool ok, int64_t row) {
                xin[it] = ok ? act_load<IO>(u, row, 2 * pq, g.d) : make_float2(0.0f, 0.0f);
            });
            tile_rows_half(1, [&](int it, int fq, int s, int64_t, bool, int64_t) {
                sre[fq * LW + lpad(s)] = xin[it].x;
                sim[fq * LW + lpad(s)] = xin[it].y;
            });
        }
        __syncthreads();
        lds_to_regs<LA, HALF_IN>(v, re, im, tau);
        __syncthreads();
    } else if constexpr (MODE == OUTER_SPEC_IMP) {
        // Taps of an implicit filter, four-step layout: transform f holds
        // pair kp at column o, samples s = tau + q T + r LA/R0 (r < R0/2),
        // t = M2 s + o.  Per column of the workgroup, the hidden features of
        // its samples are staged in sre feature-major (HC features at a
        // time, rows of LA/2 + 1 words), the pairs' W3 rows in sim.
        static_assert(HALF_IN, "four-step spectra read the live half");
        const ImpOuter& im = a.imp;
        constexpr int HS = LA / 2 + 1;  // staged row length (odd: no bank conflicts)
        constexpr int HC = 16 * HS <= NF * LW ? 16 : 8;  // features per staging round
        static_assert(HC * HS <= NF * LW, "implicit staging fits the transform's LDS");
        static_assert(16 * 2 * kImpHidden <= NF * LW, "W3 rows fit the transform's LDS");
        float* zs = sre;  // [HC][HS]
        float* sw = sim;  // [KP][2][hp]
        const int hh = HC;
        for (int e = threadIdx.x; e < KP * 2 * im.hp; e += kMpThreads) {
            const int j = e % im.hp, rc = e / im.hp, kq = rc >> 1, ch = rc & 1;
            int64_t bq, pq;
            bool lq;
            pair_of_slot(g, group, kq, bq, pq, lq);
            const int64_t c = 2 * pq + ch;
            sw[e] = (lq && c < g.d && j < im.H) ? im.W3[((int64_t)im.n * g.d + c) * im.H + j] : 0.0f;
        }
        constexpr int NSAMP = S::Q0 * (R0 / 2);
        float2 acc[NSAMP];
#pragma unroll
        for (int i = 0; i < NSAMP; ++i) acc[i] = make_float2(0.0f, 0.0f);
        const float* w0 = sw + (kp * 2 + 0) * im.hp;
        const float* w1 = sw + (kp * 2 + 1) * im.hp;
        for (int ci = 0; ci < C; ++ci) {
            const int oc = cb * C + ci;  // column staged in this round
            for (int j0 = 0; j0 < im.hp; j0 += hh) {
                __syncthreads();  // previous half consumed (and W3 rows written)
                // rows t = M2 s + oc, s < LA/2: lane -> (s, 4-feature chunk)
                const int nch = hh / 4;
                for (int e = threadIdx.x; e < (LA / 2) * nch; e += kMpThreads) {
                    const int sx = e / nch, jc = e - sx * nch;
                    const int64_t t = g.sa * sx + g.so * oc;
                    float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    if (oc < n_outer && t < g.N)
                        z = *reinterpret_cast<const float4*>(im.z2 + t * im.hp + j0 + 4 * jc);
                    zs[(4 * jc + 0) * HS + sx] = z.x;
                    zs[(4 * jc + 1) * HS + sx] = z.y;
                    zs[(4 * jc + 2) * HS + sx] = z.z;
                    zs[(4 * jc + 3) * HS + sx] = z.w;
                }
                __syncthreads();
                if ((f >> g.kp_log2) == ci) {
                    for (int j = 0; j < hh; ++j) {
                        const float wa = w0[j0 + j], wb = w1[j0 + j];
                        const float* zr = zs + j * HS;
#pragma unroll
                        for (int q = 0; q < S::Q0; ++q)
#pragma unroll
                            for (int r = 0; r < R0 / 2; ++r) {
                                const float z = zr[tau + q * TA + r * (LA / R0)];
                                float2& c = acc[q * (R0 / 2) + r];
                                c = make_float2(fmaf(wa, z, c.x), fmaf(wb, z, c.y));
                            }
                    }
                }
            }
        }
        const int64_t ca = 2 * p, cbb = 2 * p + 1;
        const bool has_b = cbb < g.d;
        const int64_t oa = (int64_t)im.n * g.d + (live ? ca : 0);
        const int64_t ob = has_b && live ? oa + 1 : oa;
        const float ala = im.alpha[oa], alb = im.alpha[ob], ba = im.b3[oa], bb = im.b3[ob];
#pragma unroll
        for (int q = 0; q < S::Q0; ++q)
#pragma unroll
            for (int r = 0; r < R0; ++r) {
                float2 x = make_float2(0.0f, 0.0f);
                if (r < R0 / 2) {
                    const int sx = tau + q * TA + r * (LA / R0);
                    const int64_t t = g.sa * sx + g.so * o;
                    const float2 c = acc[q * (R0 / 2) + r];
                    if (live && col_live && t < g.N) {
                        x.x = expf(-ala * (float)t) * (ba + c.x);
                        if (has_b) x.y = expf(-alb * (float)t) * (bb + c.y);
                    }
                }
                v[q * R0 + r] = x;
            }
        __syncthreads();  // the staging area becomes the transform's LDS
    } else if constexpr (MODE == OUTER_SPEC) {
        // filter taps straight from their channel-major layout (not timed)
        const IO* h = static_cast<const IO*>(a.filt);
        const int64_t c0 = 2 * p;
#pragma unroll
        for (int q = 0; q < S::Q0; ++q)
#pragma unroll
            for (int r = 0; r < (HALF_IN ? R0 / 2 : R0); ++r) {
                const int s = tau + q * TA + r * (LA / R0);
                float2 x = make_float2(0.0f, 0.0f);
                if (live && col_live) {
                    int64_t idx = -1, stride = 0;
                    if (g.four_step) {
                        const int64_t t = g.sa * s + g.so * o;
                        if (t < g.N) idx = t;
                        stride = g.N;
                    } else if (g.three_d) {
                        // row o = (x, y) of the P1 x P2 periodic grid, column s = z;
                        // offset (i, j, l) sits at (i mod P1, j mod P2, l mod P3)
                        const int64_t X2 = g.gx, Y2 = g.gy, Z2 = g.gz;
                        const int64_t xr = o / (2 * Y2), yr = o - xr * (2 * Y2);
                        const int64_t i = xr < X2 ? xr : xr - 2 * X2;
                        const int64_t j = yr < Y2 ? yr : yr - 2 * Y2;
                        const int64_t l = s < Z2 ? s : s - 2 * Z2;
                        if (xr != X2 && yr != Y2 && s != Z2)
                            idx = ((i + X2 - 1) * (2 * Y2 - 1) + (j + Y2 - 1)) * (2 * Z2 - 1) +
                                  (l + Z2 - 1);
                        stride = (2 * X2 - 1) * (2 * Y2 - 1) * (2 * Z2 - 1);
                    } else {
                        // periodic placement: tap offset (i, j) sits at (i mod P1, j mod P2);
                        // row o = i mod P1, column s = j mod P2
                        const int64_t X2 = g.Lb / 2, Y2 = LA / 2;
                        const int64_t i = o < X2 ? o : o - g.Lb;
                        const int64_t j = s < Y2 ? s : s - LA;
                        if (o != X2 && s != Y2) idx = (i + X2 - 1) * (2 * Y2 - 1) + (j + Y2 - 1);
                        stride = (2 * X2 - 1) * (2 * Y2 - 1);
                    }
                    if (idx >= 0) {
                        x.x = ld1<IO>(h + c0 * stride + idx);
                        if (c0 + 1 < g.d) x.y = ld1<IO>(h + (c0 + 1) * stride + idx);
                    }
                }
                v[q * R0 + r] = x;
            }
    } else {
        // MID / OUT.  F column -> (conj twiddle) -> registers in the layout
        // of the inverse's first pass (lanes of a transform read consecutive
        // bins).  The gate tile is fetched next, so its latency overlaps the
        // inverse outer DFT.
        static_assert(GT >= 1 && (LA / 2) * NF % kMpThreads == 0, "gate tile");
        if (paired) load_pairs<LA>(v, Fcol, twstep, tau, col_live, g.four_step && o > 0);
        else load_column<LA, +1>(v, Fcol, twstep, tau, col_live, g.four_step && o > 0);
        const IO* gate = static_cast<const IO*>(a.act);
        float2 gval[GT];
        if constexpr (MODE == OUTER_OUT3) {
            // HyenaND outer gate SiLU(v) after the 3x3x3 short convolution
            int64_t bq0, pq0;
            bool l0;
            pair_of_slot(g, group, (int)(threadIdx.x & (KP - 1)), bq0, pq0, l0);
            const PairTaps<27> tv = pair_taps<27>(a.blk, 2, 2 * pq0, g.d);
            const IO* vx = static_cast<const IO*>(a.blk.v);
            tile_rows([&](int it, int, int s, int64_t pq, bool ok, int64_t row) {
                float2 gv = make_float2(0.0f, 0.0f);
                if (ok) {
                    const int64_t o3 = (row % g.N) / g.so;
                    const int64_t px = o3 / g.gy, py = o3 - px * g.gy;
                    const float2 vv = short_conv3<IO>(vx, tv, row, px, py, s, g.gx, g.gy, g.gz,
                                                      2 * pq, g.d);
                    gv = make_float2(silu(vv.x), silu(vv.y));
                }
                gval[it] = gv;
            });
        } else if (MODE == OUTER_OUT && a.blk.on) {
            // HyenaND outer gate SiLU(v) after the short convolution
            int64_t bq0, pq0;
            bool l0;
            pair_of_slot(g, group, (int)(threadIdx.x & (KP - 1)), bq0, pq0, l0);
            const PairTaps<9> tv = pair_taps<9>(a.blk, 2, 2 * pq0, g.d);
            const IO* vx = static_cast<const IO*>(a.blk.v);
            tile_rows([&](int it, int, int s, int64_t pq, bool ok, int64_t row) {
                float2 gv = make_float2(0.0f, 0.0f);
                if (ok) {
                    const int64_t pp = (row % g.N) / g.so;
                    const float2 vv = short_conv<IO>(vx, tv, row, pp, s, g.Lb_live, g.so, 2 * pq, g.d);
                    gv = make_float2(silu(vv.x), silu(vv.y));
                }
                gval[it] = gv;
            });
        } else {
            tile_rows([&](int it, int, int, int64_t pq, bool ok, int64_t row) {
                gval[it] = ok ? act_load<IO>(gate, row, 2 * pq, g.d) : make_float2(0.0f, 0.0f);
            });
        }
        if (paired) inv_transform<LA, HALF_IN>(v, re, im, a.tw, g.tw_a, tau, j1, j2, [] {});
        else inv_lds_to_regs<LA, true, true>(v, re, im, a.tw, g.tw_a, tau);
        __syncthreads();
        tile_rows([&](int it, int fq, int s, int64_t, bool, int64_t) {
            sre[fq * LW + lpad(s)] = gval[it].x;
            sim[fq * LW + lpad(s)] = gval[it].y;
        });
        if constexpr (!HALF_IN) {
            // unpadded (periodic) column: the gates of the second half
            static_assert(MODE == OUTER_MID || MODE == OUTER_OUT, "unpadded columns on the plain chain only");
            tile_rows_half(1, [&](int it, int, int, int64_t pq, bool ok, int64_t row) {
                gval[it] = ok ? act_load<IO>(gate, row, 2 * pq, g.d) : make_float2(0.0f, 0.0f);
            });
            tile_rows_half(1, [&](int it, int fq, int s, int64_t, bool, int64_t) {
                sre[fq * LW + lpad(s)] = gval[it].x;
                sim[fq * LW + lpad(s)] = gval[it].y;
            });
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < S::Q0; ++q)
#pragma unroll
            for (int r = 0; r < (HALF_IN ? R0 / 2 : R0); ++r) {
                const int i = lpad(tau + q * TA + r * (LA / R0));
                float2& x = v[q * R0 + r];
                x = make_float2(x.x * re[i], x.y * im[i]);
            }
        __syncthreads();
        if constexpr (OUT) {
            regs_to_lds<LA, HALF_IN>(v, re, im, tau);
            __syncthreads();
            IO* y = static_cast<IO*>(a.out);
#pragma unroll
            for (int hf = 0; hf < NHALF; ++hf)
                tile_rows_half(hf, [&](int, int fq, int s, int64_t pq, bool ok, int64_t row) {
                    if (ok) act_store<IO>(y, row, 2 * pq, g.d,
                                          make_float2(sre[fq * LW + lpad(s)], sim[fq * LW + lpad(s)]));
                });
            return;
        }
    }

    // forward outer DFT -> (twiddle) -> F column, straight from the last
    // pass's registers (lanes of a transform hold consecutive bins)
    if (paired) {
        fwd_transform<LA, HALF_IN>(v, re, im, a.tw, g.tw_a, tau, j1, j2, false, [] {});
        if (col_live) store_pairs<LA>(v, Fcol, twstep, tau, g.four_step && o > 0);
    } else {
        fwd_regs_to_lds<LA, HALF_IN, true>(v, re, im, a.tw, g.tw_a, tau);
        if (col_live) store_column<LA>(v, Fcol, twstep, tau, g.four_step && o > 0);
    }
}

// ---------------------------------------------------------------------------
// Inner pass.  Unit kk (1 <= kk < La/2) = outer columns (kk, La - kk): their
// bins are each other's mirrors.  Unit 0 = outer columns 0 and La/2, each
// mirrored onto itself.  Workgroup = one pair slot x U = NF/2 units;
// transform f = 2u + side (side 0: column kk, side 1: its partner).
// blockIdx.x = unit block * (pair slots in chunk) + slot.
//
// Mirror of inner bin e (length LB):
//   four-step (t = M2 n1 + n2, k = k1 + M1 k2):
//     unit kk > 0:  (kk, e)      <-> (La - kk, LB - 1 - e)
//     column 0:     (0, e)       <-> (0, -e mod LB)
//     column La/2:  (La/2, e)    <-> (La/2, LB - 1 - e)
//   2D (bin (kp, kq), kq outer):
//     unit kk > 0:  (kq=kk, e)   <-> (La - kk, -e mod LB)
//     columns 0 and La/2: (kq, e) <-> (kq, -e mod LB)
// Entry e of a unit (entries [pair][unit][e], e < LB):
//   unit kk > 0: primary bin (kk, e).
//   unit 0, four-step: e = 0 packs the real bins (0,0) and (0,LB/2);
//     0 < e < LB/2: primary (0, e); e >= LB/2: primary (La/2, e - LB/2).
//   unit 0, 2D: e = 0 packs (0,0),(0,LB/2) of column 0; 0 < e < LB/2:
//     primary (0, e); e = LB/2 packs (La/2: 0, LB/2); e > LB/2: primary
//     (La/2, e - LB/2).
// ---------------------------------------------------------------------------
// Outer columns (side 0, side 1) of unit kk; `self` when both are mirrored
// onto themselves (2D: unit 0 = columns 0 and La/2).  3D (composite outer
// index a = ky P3 + kz, mirror ((-ky) mod P2, (-kz) mod P3)):
//   units 0, 1:           the self-mirrored columns (ky, 0) and (ky, P3/2) of
//                         ky = 0 and ky = P2/2;
//   next 2 (P3/2 - 1):    (ky, kz) <-> (ky, P3 - kz), 0 < kz < P3/2, for
//                         ky = 0 and ky = P2/2;
//   the rest:             (ky, kz) <-> (P2 - ky, (-kz) mod P3), 0 < ky < P2/2.
__device__ __forceinline__ void unit_columns(const MpGeom& g, int kk, int& c0, int& c1, bool& self)
{
    if (!g.three_d) {
        self = kk == 0;
        c0 = kk;
        c1 = kk == 0 ? g.La / 2 : g.La - kk;
        return;
    }
    const int P3 = g.Lc, H3 = P3 / 2, P2 = g.La / P3, H2 = P2 / 2;
    if (kk < 2) {
        self = true;
        c0 = kk * H2 * P3;
        c1 = c0 + H3;
        return;
    }
    self = false;
    int u = kk - 2;
    if (u < 2 * (H3 - 1)) {
        const int row = u / (H3 - 1), kz = 1 + u % (H3 - 1);
        const int base = row * H2 * P3;
        c0 = base + kz;
        c1 = base + P3 - kz;
        return;
    }
    u -= 2 * (H3 - 1);
    const int ky = 1 + u / P3, kz = u % P3;
    c0 = ky * P3 + kz;
    c1 = (P2 - ky) * P3 + ((P3 - kz) & (P3 - 1));
}

__device__ __forceinline__ void unit_pairing(bool four_step, bool self_unit, int e, int LB, int& fa,
                                             int& ka, int& fb, int& kb, int& self)
{
    // fa/fb: side (0 or 1), ka/kb: bin index; self: 0 = pair, 1 = packed self bins (ka, kb in side fa)
    self = 0;
    if (!self_unit) {
        fa = 0;
        ka = e;
        fb = 1;
        kb = four_step ? LB - 1 - e : (LB - e) & (LB - 1);
        return;
    }
    if (four_step) {
        if (e == 0) {
            fa = fb = 0;
            ka = 0;
            kb = LB / 2;
            self = 1;
        } else if (e < LB / 2) {
            fa = fb = 0;
            ka = e;
            kb = LB - e;
        } else {
            fa = fb = 1;
            ka = e - LB / 2;
            kb = LB - 1 - ka;
        }
    } else {
        if (e == 0 || e == LB / 2) {
            fa = fb = e == 0 ? 0 : 1;
            ka = 0;
            kb = LB / 2;
            self = 1;
        } else if (e < LB / 2) {
            fa = fb = 0;
            ka = e;
            kb = LB - e;
        } else {
            fa = fb = 1;
            ka = e - LB / 2;
            kb = LB - ka;
        }
    }
}

template <int LB, typename SP, int MODE, bool HALF_B>
__global__ void __launch_bounds__(kMpThreads, 2) hyena_mp_inner(InnerArgs a)
{
    using S = FftShape<LB>;
    using X = MpShape<LB>;
    constexpr int TB = X::T, NF = X::NF, LW = X::LW, U = NF / 2;
    __shared__ float sre[NF * LW];
    __shared__ float sim[NF * LW];

    const MpGeom& g = a.g;
    const int KP = 1 << g.kp_log2;
    const int64_t nslots = g.ngroups * KP;
    const int64_t slot = blockIdx.x % nslots;
    const int ub = blockIdx.x / nslots;
    const int kk0 = ub * U;
    const int f = threadIdx.x / TB;
    const int tau = threadIdx.x - f * TB;
    float* re = sre + f * LW;
    float* im = sim + f * LW;
    const int La = g.La;
    const int nlive = MODE == INNER_SPEC ? LB : g.Lb_live;
    const int64_t group = g.group0 + slot / KP;
    int64_t b, p;
    bool live;
    pair_of_slot(g, group, (int)(slot % KP), b, p, live);
    float2* Fp = a.F + slot * (g.pair_bytes / 8);

    // units of this workgroup: kk0 .. kk0 + nu - 1 (nu <= U)
    const int nu = min(U, La / 2 - kk0);
    // F position of (unit, side): on the 1D and 2D paths the outer pass
    // stores a bin next to its mirror (fpos), so unit kk sits at 2 kk and
    // 2 kk + 1; 3D intermediates keep the composite bins in natural order
    auto col_of = [&](int u, int side) {
        if (!g.three_d) return 2 * (kk0 + u) + side;
        int c0, c1;
        bool sf;
        unit_columns(g, kk0 + u, c0, c1, sf);
        return side == 0 ? c0 : c1;
    };

    // this thread's share of the mirror-paired product: unit u, entries
    // e = tu + i 2TB
    constexpr int EPT = LB / (2 * TB);
    const int u_me = f >> 1;
    const int tu = (f & 1) * TB + tau;  // 0 .. 2 TB - 1
    const int kk_me = kk0 + u_me;
    const bool unit_ok = u_me < nu && live;
    bool self_me;
    {
        int c0, c1;
        unit_columns(g, kk_me, c0, c1, self_me);
    }
    const int64_t ebase = p * (int64_t)(La / 2) * LB + (int64_t)kk_me * LB;
    typename EntryRaw<SP>::type ent[EPT];
    if constexpr (MODE == INNER_CHAIN) {
        // entries first: their latency overlaps the F load and the forward DFT
        if (unit_ok) {
            using Raw = typename EntryRaw<SP>::type;
#pragma unroll
            for (int i = 0; i < EPT; ++i)
                ent[i] = stream_load(&reinterpret_cast<const Raw*>(a.spec)[ebase + tu + i * 2 * TB]);
        }
    }

    // F[o][column] -> region of (u, side) at inner position o.  With all U
    // units present (the usual case) the per-thread element count is a
    // compile-time constant and every load is issued before the first use.
    constexpr int NLIVE = MODE == INNER_SPEC ? LB : (HALF_B ? LB / 2 : LB);
    constexpr int PER = NLIVE * 2 * U / kMpThreads;
    static_assert(NLIVE * 2 * U % kMpThreads == 0, "inner tile split");
    // fast path: 2U divides the thread count, so a thread's (unit, side) --
    // hence its column -- is the same in every iteration; inner positions
    // step by kMpThreads / (2U).  Neighbouring lanes take the two sides of a
    // unit, then the next unit: consecutive F positions on the 1D and 2D
    // paths, and consecutive LDS regions.
    static_assert(kMpThreads % (2 * U) == 0, "inner tile rows");
    constexpr int OPS = kMpThreads / (2 * U);
    const int u_t = ((int)threadIdx.x >> 1) % U;
    const int side_t = (int)threadIdx.x & 1;
    const int op_t = (int)threadIdx.x / (2 * U);
    const int fq_t = 2 * u_t + side_t;
    if (nu == U) {
        const float2* src = Fp + col_of(u_t, side_t);
        float2 xin[PER];
#pragma unroll
        for (int it = 0; it < PER; ++it) xin[it] = f_load(&src[(int64_t)(op_t + it * OPS) * La]);
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            sre[fq_t * LW + lpad(op_t + it * OPS)] = xin[it].x;
            sim[fq_t * LW + lpad(op_t + it * OPS)] = xin[it].y;
        }
    } else {
        const int total = nlive * nu * 2;
        for (int idx = threadIdx.x; idx < total; idx += kMpThreads) {
            const int u = (idx >> 1) % nu;
            const int side = idx & 1;
            const int op = idx / (2 * nu);
            const float2 x = f_load(&Fp[(int64_t)op * La + col_of(u, side)]);
            const int fq = 2 * u + side;
            sre[fq * LW + lpad(op)] = x.x;
            sim[fq * LW + lpad(op)] = x.y;
        }
    }
    __syncthreads();
    constexpr bool HALF_LOAD = (MODE == INNER_CHAIN) && HALF_B;
    float2 v[S::PTS];
    lds_to_regs<LB, HALF_LOAD>(v, re, im, tau);
    __syncthreads();
    fwd_regs_to_lds<LB, HALF_LOAD>(v, re, im, a.tw, g.tw_b, tau);
    __syncthreads();

    // mirror-paired product (CHAIN) or entry computation (SPEC)
    if (unit_ok) {
        float* ure = sre + (2 * u_me) * LW;
        float* uim = sim + (2 * u_me) * LW;
        float dp = 0.0f, dq = 0.0f;
        if constexpr (MODE == INNER_CHAIN) {
            const int64_t c0 = 2 * p;
            const float Da = a.D[c0];
            const float Db = c0 + 1 < g.d ? a.D[c0 + 1] : 0.0f;
            // entries hold (Ha +- Hb) / (2M); the feedthrough adds D to every bin
            const float inv2M = 0.5f / ((float)La * (float)LB);
            dp = (Da + Db) * inv2M;
            dq = (Da - Db) * inv2M;
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tu + i * 2 * TB;
            int fa, ka, fb, kb, self;
            unit_pairing(g.four_step != 0, self_me, e, LB, fa, ka, fb, kb, self);
            const int ia = fa * LW + lpad(ka), ib = fb * LW + lpad(kb);
            float2 za = make_float2(ure[ia], uim[ia]);
            float2 zb = make_float2(ure[ib], uim[ib]);
            if constexpr (MODE == INNER_CHAIN) {
                float2 P, Q;
                widen_entry<SP>(ent[i], P, Q);
                if (self) {
                    za = self_product(za, P.x + dp, Q.x + dq);
                    zb = self_product(zb, P.y + dp, Q.y + dq);
                } else {
                    P.x += dp;
                    Q.x += dq;
                    pair_product(za, zb, P, Q);
                }
                ure[ia] = za.x;
                uim[ia] = za.y;
                ure[ib] = zb.x;
                uim[ib] = zb.y;
            } else {
                const float sc = 0.5f / ((float)La * (float)LB);
                float2 P, Q;
                if (self) {
                    P = make_float2((za.x + za.y) * sc, (zb.x + zb.y) * sc);
                    Q = make_float2((za.x - za.y) * sc, (zb.x - zb.y) * sc);
                } else {
                    entry_from_pair(za, zb, sc, P, Q);
                }
                store_entry(static_cast<SP*>(a.spec_out), ebase + e, P, Q);
            }
        }
    }
    if constexpr (MODE == INNER_SPEC) return;

    __syncthreads();
    inv_lds_to_regs<LB, HALF_B>(v, re, im, a.tw, g.tw_b, tau);
    __syncthreads();
    regs_to_lds<LB, HALF_B>(v, re, im, tau);
    __syncthreads();
    if (nu == U) {
        float2* dst = Fp + col_of(u_t, side_t);
        float2 xout[PER];
#pragma unroll
        for (int it = 0; it < PER; ++it)
            xout[it] = make_float2(sre[fq_t * LW + lpad(op_t + it * OPS)],
                                   sim[fq_t * LW + lpad(op_t + it * OPS)]);
#pragma unroll
        for (int it = 0; it < PER; ++it) f_store(&dst[(int64_t)(op_t + it * OPS) * La], xout[it]);
    } else {
        const int total_out = g.Lb_live * nu * 2;
        for (int idx = threadIdx.x; idx < total_out; idx += kMpThreads) {
            const int u = (idx >> 1) % nu;
            const int side = idx & 1;
            const int op = idx / (2 * nu);
            const int fq = 2 * u + side;
            f_store(&Fp[(int64_t)op * La + col_of(u, side)],
                    make_float2(sre[fq * LW + lpad(op)], sim[fq * LW + lpad(op)]));
        }
    }
}

// ---------------------------------------------------------------------------
// Middle pass (3D): length-LY transforms along y between the two
// intermediates of a pair slot, F1 [x][y][kz] (y < ylen1) and F2
// [x][ky][kz].  Transform j = x P3 + kz of the slot; a workgroup takes NF
// consecutive j, with transform f = threadIdx % NF and lane tau = threadIdx /
// NF, so the lanes of one register slot touch consecutive kz.
//   MID_FWD: F1 -> F2; HALF: only y < LY/2 hold data (the zero padding).
//   MID_INV: F2 -> F1 (unscaled inverse), keeping y < LY/2.
// ---------------------------------------------------------------------------
enum MidMode { MID_FWD = 0, MID_INV = 1 };

struct MidArgs {
    const float2* src;
    float2* dst;
    const float2* tw;
    TwOffsets tw_y;
    int64_t f1_pair, f2_pair;  // float2 elements per pair slot of F1 / F2
    int64_t ncols;             // transforms per slot: x rows times P3
    int64_t nslots;            // pair slots in this chunk
    int32_t P3;
    int32_t ylen1;             // y extent of F1 (Y in the chain, P2 for spectra)
};

template <int LY, int MODE, bool HALF>
__global__ void __launch_bounds__(kMpThreads, 2) hyena_mp_mid(MidArgs a)
{
    using S = FftShape<LY>;
    using X = MpShape<LY>;
    constexpr int T = X::T, NF = X::NF, LW = X::LW, R0 = S::R0, RL = S::RL, QL = S::PTS / RL;
    constexpr int RIN = HALF ? R0 / 2 : R0;
    __shared__ float sre[NF * LW];
    __shared__ float sim[NF * LW];
    const int f = (int)threadIdx.x % NF;
    const int tau = (int)threadIdx.x / NF;
    const int64_t slot = blockIdx.x % a.nslots;
    const int64_t j = (int64_t)(blockIdx.x / a.nslots) * NF + f;
    const bool live = j < a.ncols;
    const int64_t x = live ? j / a.P3 : 0;
    const int64_t kz = live ? j - x * a.P3 : 0;
    float* re = sre + f * LW;
    float* im = sim + f * LW;
    const int64_t e1 = slot * a.f1_pair + x * a.ylen1 * a.P3 + kz;  // F1 (x, 0, kz)
    const int64_t e2 = slot * a.f2_pair + x * (int64_t)LY * a.P3 + kz;  // F2 (x, 0, kz)
    float2 v[S::PTS];
    if constexpr (MODE == MID_FWD) {
        // R0-pass layout: v[q R0 + r] = sample y = tau + q T + r LY/R0
#pragma unroll
        for (int q = 0; q < S::Q0; ++q)
#pragma unroll
            for (int r = 0; r < RIN; ++r) {
                const int y = tau + q * T + r * (LY / R0);
                v[q * R0 + r] = live ? a.src[e1 + (int64_t)y * a.P3] : make_float2(0.0f, 0.0f);
            }
        fwd_regs_to_lds<LY, HALF, true>(v, re, im, a.tw, a.tw_y, tau);
        if (live) {
#pragma unroll
            for (int q = 0; q < QL; ++q)
#pragma unroll
                for (int r = 0; r < RL; ++r) {
                    const int ky = tau + q * T + r * (LY / RL);
                    a.dst[e2 + (int64_t)ky * a.P3] = v[q * RL + r];
                }
        }
    } else {
        // the inverse's first pass reads bins ky = tau + q T + r LY/RL
#pragma unroll
        for (int q = 0; q < QL; ++q)
#pragma unroll
            for (int r = 0; r < RL; ++r) {
                const int ky = tau + q * T + r * (LY / RL);
                v[q * RL + r] = live ? a.src[e2 + (int64_t)ky * a.P3] : make_float2(0.0f, 0.0f);
            }
        inv_lds_to_regs<LY, true, true>(v, re, im, a.tw, a.tw_y, tau);
        if (live) {
#pragma unroll
            for (int q = 0; q < S::Q0; ++q)
#pragma unroll
                for (int r = 0; r < R0 / 2; ++r) {
                    const int y = tau + q * T + r * (LY / R0);
                    a.dst[e1 + (int64_t)y * a.P3] = v[q * R0 + r];
                }
        }
    }
}

}  // namespace hy

namespace hy {

template <int LA, typename IO, int MODE, bool HALF_SPEC, bool PAIRED>
hyena_status mp_outer_launch(const OuterArgs& a, int64_t nblocks, hipStream_t s)
{
    if (PAIRED == (a.g.three_d != 0))
        return fail(HYENA_ERR_UNSUPPORTED, "multi-pass: outer row layout does not match the path");
    HY_LAUNCH(kernel_label("hyena_mp_outer", LA, type_label<IO>(), MODE, HALF_SPEC, PAIRED),
              (hyena_mp_outer<LA, IO, MODE, HALF_SPEC, PAIRED>), dim3((unsigned)nblocks), dim3(kMpThreads),
              0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

template <int LB, typename SP, int MODE, bool HALF_B>
hyena_status mp_inner_launch(const InnerArgs& a, int64_t nblocks, hipStream_t s)
{
    HY_LAUNCH(kernel_label("hyena_mp_inner", LB, type_label<SP>(), MODE, HALF_B),
              (hyena_mp_inner<LB, SP, MODE, HALF_B>), dim3((unsigned)nblocks), dim3(kMpThreads), 0,
              s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

template <int LY, int MODE, bool HALF>
hyena_status mp_mid_launch(const MidArgs& a, int64_t nblocks, hipStream_t s)
{
    HY_LAUNCH(kernel_label("hyena_mp_mid", LY, MODE, HALF), (hyena_mp_mid<LY, MODE, HALF>),
              dim3((unsigned)nblocks), dim3(kMpThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

#define HY_MP_LENGTHS(X, A, B) X(8, A, B) X(16, A, B) X(32, A, B) X(64, A, B) X(128, A, B) \
    X(256, A, B) X(512, A, B) X(1024, A, B)
// inner (F-facing) passes also come in 2048 and 4096 points: four-step
// transforms up to 1024 x 4096
#define HY_MP_INNER_LENGTHS(X, A, B) HY_MP_LENGTHS(X, A, B) X(2048, A, B) X(4096, A, B)
// outer passes also come in 2048 points: 2D grids with sides up to 1024
// (transforms of 2048 points along either axis)
#define HY_MP_OUTER_LENGTHS(X, A, B) HY_MP_LENGTHS(X, A, B) X(2048, A, B)

// unpadded (periodic) chain modes on the four-step column lengths of
// periodic plans (N >= 32768: 512 or 1024 samples)
#define HY_MP_OUTER_CIRC_LENGTHS(X, A, B) X(512, A, B) X(1024, A, B)
#define HY_MP_OUTER_CIRC_INST(L, IO, EXT)                  \
    HY_MP_OUTER_ONE(L, IO, OUTER_IN, false, true, EXT)     \
    HY_MP_OUTER_ONE(L, IO, OUTER_MID, false, true, EXT)    \
    HY_MP_OUTER_ONE(L, IO, OUTER_OUT, false, true, EXT)

// the implicit-filter spectrum pass reads no storage-typed input: float only;
// four-step column lengths (32 .. 1024)
#define HY_MP_OUTER_IMP_LENGTHS(X, A, B) X(32, A, B) X(64, A, B) X(128, A, B) X(256, A, B) \
    X(512, A, B) X(1024, A, B)
#define HY_MP_OUTER_IMP_INST(L, A_, EXT) \
    EXT template hyena_status mp_outer_launch<L, float, OUTER_SPEC_IMP, true, true>(const OuterArgs&, int64_t, hipStream_t);
#define HY_MP_OUTER_ONE(L, IO, MODE, HS, PR, EXT) \
    EXT template hyena_status mp_outer_launch<L, IO, MODE, HS, PR>(const OuterArgs&, int64_t, hipStream_t);
// 1D / 2D (mirror-paired rows) and 3D (natural rows, and the mixer's modes)
#define HY_MP_OUTER_INST(L, IO, EXT)                   \
    HY_MP_OUTER_ONE(L, IO, OUTER_IN, true, true, EXT)    \
    HY_MP_OUTER_ONE(L, IO, OUTER_MID, true, true, EXT)   \
    HY_MP_OUTER_ONE(L, IO, OUTER_OUT, true, true, EXT)   \
    HY_MP_OUTER_ONE(L, IO, OUTER_SPEC, true, true, EXT)  \
    HY_MP_OUTER_ONE(L, IO, OUTER_SPEC, false, true, EXT) \
    HY_MP_OUTER_ONE(L, IO, OUTER_IN, true, false, EXT)   \
    HY_MP_OUTER_ONE(L, IO, OUTER_MID, true, false, EXT)  \
    HY_MP_OUTER_ONE(L, IO, OUTER_OUT, true, false, EXT)  \
    HY_MP_OUTER_ONE(L, IO, OUTER_SPEC, false, false, EXT) \
    HY_MP_OUTER_ONE(L, IO, OUTER_IN3, true, false, EXT)  \
    HY_MP_OUTER_ONE(L, IO, OUTER_OUT3, true, false, EXT)

#define HY_MP_MID_INST(L, A_, EXT)                                                            \
    EXT template hyena_status mp_mid_launch<L, MID_FWD, true>(const MidArgs&, int64_t,        \
                                                              hipStream_t);                   \
    EXT template hyena_status mp_mid_launch<L, MID_FWD, false>(const MidArgs&, int64_t,       \
                                                               hipStream_t);                  \
    EXT template hyena_status mp_mid_launch<L, MID_INV, true>(const MidArgs&, int64_t,        \
                                                              hipStream_t);

#define HY_MP_INNER_INST(L, SP, EXT)                                                          \
    EXT template hyena_status mp_inner_launch<L, SP, INNER_CHAIN, true>(const InnerArgs&,     \
                                                                        int64_t, hipStream_t); \
    EXT template hyena_status mp_inner_launch<L, SP, INNER_CHAIN, false>(const InnerArgs&,    \
                                                                         int64_t, hipStream_t); \
    EXT template hyena_status mp_inner_launch<L, SP, INNER_SPEC, false>(const InnerArgs&,     \
                                                                        int64_t, hipStream_t);

}  // namespace hy
