// implicit.hip -- filter spectra from an implicit filter ("Hyena -- Long
// Convolutions Math", sections "Implicit filters: an MLP over positions" and
// "The decay window"): taps exp(-alpha t) FFN(gamma(t)) with FFN a two-layer
// sine MLP shared over positions.
//
//   hyena_implicit_hidden: z2[t] = sin(omega (W2 sin(omega (W1 gamma(t) + b1))
//                          + b2)) for every position t, into the scratch
//                          (the only buffer the call needs besides H).
//   The spectrum kernels then evaluate every tap where the transform needs
//   it, h = window . (W3 z2 + b3), in registers, straight into their forward
//   transform, so the taps never exist in memory:
//     hyena_implicit_real_spectrum   single-channel form, two or three filter
//                                    rows per workgroup sharing each z2 load;
//     hyena_implicit_pair_spectrum   channel-pair form (a pair per workgroup);
//     four-step path: the outer pass's OUTER_SPEC_IMP mode, which stages the
//     z2 rows of its column in LDS for its 16 channel pairs.
#include "dispatch.h"
#include "lds1d_kernels.h"

namespace hy {

namespace {

constexpr int kImpMaxFreqs = 64;
constexpr int kImpMaxHidden = 256;
constexpr int kImpPos = 16;  // positions per workgroup of the hidden kernel
constexpr int kHiddenPad = 16;  // hidden width padded to a multiple of this

// hidden width padded with zero features: the contractions walk the features
// in pairs (single-channel spectrum) and in LDS rounds of 8 or 16 (four-step)
int64_t hidden_pad(int32_t H) { return (H + kHiddenPad - 1) / kHiddenPad * kHiddenPad; }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct HiddenArgs {
    const float* W1;
    const float* b1;
    const float* W2;
    const float* b2;
    float* z2;  // [N][hp], or [hp][N] when feature_major
    int64_t N;
    int32_t K, H, hp;
    int32_t feature_major;
    float omega;
};

// One workgroup: kImpPos positions; thread i < H computes hidden unit i.
__global__ void __launch_bounds__(kImpMaxHidden) hyena_implicit_hidden(HiddenArgs a)
{
    constexpr int P = kImpPos;
    __shared__ float g[P][2 * kImpMaxFreqs + 1];
    __shared__ float z1[P][kImpMaxHidden];
    const int m = 2 * a.K + 1;
    const int64_t t0 = (int64_t)blockIdx.x * P;
    // positional encoding: t/N, then cos and sin of 2 pi j t/N (argument
    // reduced exactly in integers: 2 j t mod 2N, then sinpi / cospi)
    for (int e = threadIdx.x; e < P * m; e += blockDim.x) {
        const int p = e / m, k = e - p * m;
        const int64_t t = t0 + p;
        float val = 0.0f;
        if (t < a.N) {
            if (k == 0) {
                val = (float)((double)t / (double)a.N);
            } else {
                const int64_t j = (k + 1) / 2;
                const int64_t r = (2 * j * t) % (2 * a.N);
                const float x = (float)((double)r / (double)a.N);
                val = (k & 1) ? cospif(x) : sinpif(x);
            }
        }
        g[p][k] = val;
    }
    __syncthreads();
    const int i = threadIdx.x;
    float acc[P];
    if (i < a.H) {
#pragma unroll
        for (int p = 0; p < P; ++p) acc[p] = a.b1[i];
        for (int k = 0; k < m; ++k) {
            const float w = a.W1[(int64_t)i * m + k];
#pragma unroll
            for (int p = 0; p < P; ++p) acc[p] = fmaf(w, g[p][k], acc[p]);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) z1[p][i] = sinf(a.omega * acc[p]);
    }
    __syncthreads();
    if (i < a.hp) {
        if (i < a.H) {
#pragma unroll
            for (int p = 0; p < P; ++p) acc[p] = a.b2[i];
            for (int k = 0; k < a.H; ++k) {
                const float w = a.W2[(int64_t)i * a.H + k];
#pragma unroll
                for (int p = 0; p < P; ++p) acc[p] = fmaf(w, z1[p][k], acc[p]);
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int64_t t = t0 + p;
            if (t < a.N) {
                const float zv = i < a.H ? sinf(a.omega * acc[p]) : 0.0f;
                if (a.feature_major) a.z2[(int64_t)i * a.N + t] = zv;
                else a.z2[t * a.hp + i] = zv;
            }
        }
    }
}

// Output layer of the implicit filter for the fused spectrum kernels.
struct ImpArgs {
    const float* z2;  // hidden features, [hp][N] (feature-major)
    const float* W3;  // [rows][H]
    const float* b3;
    const float* alpha;
    int64_t N, rows;  // rows = order d
    int32_t H, hp;
};

// exp(-alpha t) for the sample pair (t, t + 1): one exponential per pair, the
// second sample takes the one-step factor.
__device__ __forceinline__ float2 window_pair(float alpha, float step, int64_t t)
{
    const float e = expf(-alpha * (float)t);
    return make_float2(e, e * step);
}

// Single-channel spectrum (transform length L = M/2, one real channel per
// transform; CIRC: the periodic plan, M = N) with the taps evaluated in
// registers.  Workgroup = RPW consecutive filter rows o0 = RPW blockIdx ...:
// every z2 value a thread loads serves all of them, so the hidden features
// are read from L2 once per RPW rows (the contraction is bound by that
// traffic).  The accumulators of all RPW rows stay in registers through the
// rows' transforms, so RPW is what the register file leaves room for: three
// rows from L = 4096 up (spill-free; 8192 at 768 channels and order 2 then
// fills the GPU with exactly one round of workgroups, 23% faster than two
// rows), two below (three measured no faster at 2048), one for the periodic
// plans (twice as many live samples per thread).  The R0-pass input of
// thread tau, slot (q, r), is the sample pair (2m, 2m + 1), m = tau + q T +
// r L/R0; feature j of that pair is one aligned float2 of the feature-major
// z2.
template <int L, bool CIRC>
constexpr int kImpRows = CIRC ? 1 : L >= 4096 ? 3 : 2;

template <int L, typename SP, bool CIRC>
__global__ void __launch_bounds__(FftShape<L>::T, 2) hyena_implicit_real_spectrum(ImpArgs a, Lds1dSpecArgs s)
{
    using S = FftShape<L>;
    constexpr int T = S::T, PTS = S::PTS, R0 = S::R0;
    constexpr int RIN = CIRC ? R0 : R0 / 2;
    constexpr int NS = S::Q0 * RIN;  // sample pairs per thread
    constexpr int RPW = kImpRows<L, CIRC>;
    __shared__ float smem[2 * S::LW];
    __shared__ float sw[RPW][kImpMaxHidden];
    const int tau = threadIdx.x;
    const int64_t o0 = RPW * (int64_t)blockIdx.x;
    const int nrows = (int)(a.rows - o0 < RPW ? a.rows - o0 : RPW);  // rows of this workgroup
    const int j1 = tau, j2 = tau ? 2 * T - tau : T;
    for (int e = tau; e < RPW * a.hp; e += T) {
        const int r = e / a.hp, j = e - r * a.hp;
        const int64_t o = o0 + (r < nrows ? r : 0);
        sw[r][j] = j < a.H ? a.W3[o * a.H + j] : 0.0f;
    }
    __syncthreads();
    float2 acc[RPW][NS];
#pragma unroll
    for (int k = 0; k < RPW; ++k)
#pragma unroll
        for (int i = 0; i < NS; ++i) acc[k][i] = make_float2(0.0f, 0.0f);
    // features in pairs: both features' loads are issued before either is
    // used (hp is a multiple of 16), so L2 latencies overlap
    for (int j = 0; j < a.hp; j += 2) {
        float2 z[2][NS];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const float* zj = a.z2 + (int64_t)(j + jj) * a.N;
#pragma unroll
            for (int q = 0; q < S::Q0; ++q)
#pragma unroll
                for (int r = 0; r < RIN; ++r) {
                    const int64_t m = tau + q * T + r * (L / R0);
                    z[jj][q * RIN + r] = *reinterpret_cast<const float2*>(zj + 2 * m);
                }
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int k = 0; k < RPW; ++k) {
                const float w = sw[k][j + jj];
#pragma unroll
                for (int i = 0; i < NS; ++i) {
                    const float2 zz = z[jj][i];
                    float2& c = acc[k][i];
                    c = make_float2(fmaf(w, zz.x, c.x), fmaf(w, zz.y, c.y));
                }
            }
    }
    float2 v[PTS];
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
        if (k >= nrows) break;  // uniform
        const int64_t o = o0 + k;
        const float al = a.alpha[o], b3 = a.b3[o], step = expf(-al);
#pragma unroll
        for (int q = 0; q < S::Q0; ++q)
#pragma unroll
            for (int r = 0; r < R0; ++r) {
                if (r >= RIN) continue;
                const int64_t m = tau + q * T + r * (L / R0);
                const float2 w = window_pair(al, step, 2 * m);
                const float2 c = acc[k][q * RIN + r];
                v[q * R0 + r] = make_float2(w.x * (b3 + c.x), w.y * (b3 + c.y));
            }
        fwd_transform<L, !CIRC>(v, smem, smem + S::LW, s.tw, s.tw_off, tau, j1, j2, k > 0, [] {});
        SP* spec = static_cast<SP*>(s.spec) + o * (int64_t)(L / 2) * kEntryElems;
        store_real_entries<L, SP>(v, spec, tau, 1.0f / (float)L, s.twm[tau ? tau : T]);
    }
}

// Channel-pair spectrum (transform length M, any N < M/2 + 1) with the taps
// of the pair's two channels evaluated in registers: one workgroup per
// (filter n, channel pair); sample t = tau + q T + r M/R0, r < R0/2.
template <int M, typename SP>
__global__ void __launch_bounds__(FftShape<M>::T, 2) hyena_implicit_pair_spectrum(ImpArgs a, Lds1dSpecArgs s)
{
    using S = FftShape<M>;
    constexpr int T = S::T, PTS = S::PTS, R0 = S::R0;
    constexpr int NS = S::Q0 * (R0 / 2);
    __shared__ float smem[2 * S::LW];
    __shared__ float sw[2][kImpMaxHidden];
    const int tau = threadIdx.x;
    const int64_t lin = blockIdx.x;  // n * npairs + p
    const int64_t n = lin / s.npairs;
    const int64_t c0 = 2 * (lin - n * s.npairs);
    const bool has_b = c0 + 1 < s.d;
    const int64_t oa = n * s.d + c0, ob = has_b ? oa + 1 : oa;
    const int j1 = tau, j2 = tau ? 2 * T - tau : T;
    for (int e = tau; e < 2 * a.hp; e += T) {
        const int r = e / a.hp, j = e - r * a.hp;
        sw[r][j] = j < a.H ? a.W3[(r == 0 ? oa : ob) * a.H + j] : 0.0f;
    }
    __syncthreads();
    float2 acc[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) acc[i] = make_float2(0.0f, 0.0f);
    for (int j = 0; j < a.hp; ++j) {
        const float w0 = sw[0][j], w1 = sw[1][j];
        const float* zj = a.z2 + (int64_t)j * a.N;
#pragma unroll
        for (int q = 0; q < S::Q0; ++q)
#pragma unroll
            for (int r = 0; r < R0 / 2; ++r) {
                const int64_t t = tau + q * T + r * (M / R0);
                const float z = t < a.N ? zj[t] : 0.0f;
                float2& c = acc[q * (R0 / 2) + r];
                c = make_float2(fmaf(w0, z, c.x), fmaf(w1, z, c.y));
            }
    }
    const float ala = a.alpha[oa], alb = a.alpha[ob], ba = a.b3[oa], bb = a.b3[ob];
    float2 v[PTS];
#pragma unroll
    for (int q = 0; q < S::Q0; ++q)
#pragma unroll
        for (int r = 0; r < R0 / 2; ++r) {
            const int64_t t = tau + q * T + r * (M / R0);
            const float2 c = acc[q * (R0 / 2) + r];
            const bool live = t < a.N;
            v[q * R0 + r] = make_float2(live ? expf(-ala * (float)t) * (ba + c.x) : 0.0f,
                                        (live && has_b) ? expf(-alb * (float)t) * (bb + c.y) : 0.0f);
        }
    fwd_transform<M>(v, smem, smem + S::LW, s.tw, s.tw_off, tau, j1, j2, false, [] {});
    SP* spec = static_cast<SP*>(s.spec) + lin * (int64_t)(M / 2) * kEntryElems;
    store_spectrum_entries<M, SP>(v, spec, tau, 0.5f / (float)M);
}

template <int L, typename SP, bool CIRC>
hyena_status imp_real_launch(const ImpArgs& a, const Lds1dSpecArgs& s, hipStream_t st)
{
    constexpr int RPW = kImpRows<L, CIRC>;
    const int64_t nb = (a.rows + RPW - 1) / RPW;
    HY_LAUNCH(kernel_label("hyena_implicit_real_spectrum", L, type_label<SP>(), CIRC),
              (hyena_implicit_real_spectrum<L, SP, CIRC>), dim3((unsigned)nb), dim3(FftShape<L>::T),
              0, st, a, s);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

template <int M, typename SP>
hyena_status imp_pair_launch(const ImpArgs& a, const Lds1dSpecArgs& s, hipStream_t st)
{
    HY_LAUNCH(kernel_label("hyena_implicit_pair_spectrum", M, type_label<SP>()),
              (hyena_implicit_pair_spectrum<M, SP>), dim3((unsigned)s.nblocks), dim3(FftShape<M>::T),
              0, st, a, s);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? HYENA_OK : fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
}

template <typename SP>
hyena_status imp_lds1d(const Plan& p, const ImpArgs& a, const Lds1dSpecArgs& s, hipStream_t st)
{
    if (p.lds_io == IO_REAL) {
        const bool circ = p.circular != 0;
        switch (p.M / 2) {
#define HY_CASE(LL, I, S_)                                                            \
    case LL:                                                                          \
        return circ ? imp_real_launch<LL, SP, true>(a, s, st) : imp_real_launch<LL, SP, false>(a, s, st);
            HY_LDS1D_REAL_SIZES(HY_CASE, 0, 0)
#undef HY_CASE
            default: return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: unsupported length");
        }
    }
    switch (p.M) {
#define HY_CASE(MM, I, S_) \
    case MM: return imp_pair_launch<MM, SP>(a, s, st);
        HY_LDS1D_SIZES(HY_CASE, 0, 0)
#undef HY_CASE
        default: return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: unsupported length");
    }
}

}  // namespace

size_t implicit_scratch_bytes(const Plan& p, int32_t hidden)
{
    // the hidden features only: the taps are never stored
    return align256((size_t)p.N * (size_t)hidden_pad(hidden) * 4u);
}

hyena_status launch_implicit_spectrum(const Plan& p, const hyena_implicit_filter& f, void* H,
                                      void* ws, void* scratch, void* stream)
{
    const hipStream_t s = (hipStream_t)stream;
    if (f.n_freqs < 0 || f.n_freqs > kImpMaxFreqs)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: n_freqs must be in 0..64");
    if (f.hidden < 1 || f.hidden > kImpMaxHidden)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: hidden must be in 1..256");
    const bool four = p.path == HYENA_PATH_FOURSTEP1D;
    HiddenArgs h{};
    h.W1 = f.W1;
    h.b1 = f.b1;
    h.W2 = f.W2;
    h.b2 = f.b2;
    h.z2 = static_cast<float*>(scratch);
    h.N = p.N;
    h.K = f.n_freqs;
    h.H = f.hidden;
    h.hp = (int32_t)hidden_pad(f.hidden);
    // the four-step spectrum stages whole rows z2[t][:] of its column in LDS;
    // the single-workgroup kernels read one feature for many t at a time
    h.feature_major = four ? 0 : 1;
    h.omega = f.omega;
    HY_LAUNCH(kernel_label("hyena_implicit_hidden"), hyena_implicit_hidden,
              dim3((unsigned)((p.N + kImpPos - 1) / kImpPos)), dim3(kImpMaxHidden), 0, s, h);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));

    ImpArgs ia{};
    ia.z2 = h.z2;
    ia.W3 = f.W3;
    ia.b3 = f.b3;
    ia.alpha = f.alpha;
    ia.N = p.N;
    ia.rows = (int64_t)p.order * p.d;
    ia.H = f.hidden;
    ia.hp = h.hp;
    if (four) return launch_fourstep_spectrum_implicit(p, ia.z2, ia.W3, ia.b3, ia.alpha, ia.hp,
                                                       ia.H, H, ws, stream);
    Lds1dSpecArgs sa = lds1d_spec_args(p, H, ws);
    if (p.spec_dtype == HYENA_F32) return imp_lds1d<float>(p, ia, sa, s);
    return imp_lds1d<uint16_t>(p, ia, sa, s);
}

}  // namespace hy
