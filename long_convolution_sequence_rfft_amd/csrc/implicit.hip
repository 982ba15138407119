// implicit.hip -- filter spectra from an implicit filter ("Hyena -- Long
// Convolutions Math", sections "Implicit filters: an MLP over positions" and
// "The decay window"): taps exp(-alpha t) FFN(gamma(t)) with FFN a two-layer
// sine MLP shared over positions.
//
//   hyena_implicit_hidden: z2[t] = sin(omega (W2 sin(omega (W1 gamma(t) + b1))
//                          + b2)) for every position t, into the scratch.
//   single-channel path:   the spectrum kernel forms the taps from z2 itself
//                          (hyena_lds1d_real_spectrum<..., true>).
//   other paths:           hyena_implicit_taps writes the taps to the scratch
//                          in the plan's storage type, then the plan's usual
//                          spectrum launch transforms them.
#include "dispatch.h"
#include "lds1d_kernels.h"

namespace hy {

HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_EXTERN, float, float)
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_EXTERN, uint16_t, uint16_t)
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_EXTERN, uint16_t, float)
HY_LDS1D_REAL_SIZES(HY_LDS1D_REAL_EXTERN, _Float16, float)

namespace {

constexpr int kImpMaxFreqs = 64;
constexpr int kImpMaxHidden = 256;
constexpr int kImpPos = 16;  // positions per workgroup of the hidden kernel

int64_t hidden_pad(int32_t H) { return (H + 3) / 4 * 4; }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct HiddenArgs {
    const float* W1;
    const float* b1;
    const float* W2;
    const float* b2;
    float* z2;  // [N][hp]
    int64_t N;
    int32_t K, H, hp;
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
            if (t < a.N) a.z2[t * a.hp + i] = i < a.H ? sinf(a.omega * acc[p]) : 0.0f;
        }
    }
}

// Taps [order d][N] in the storage type, one thread per tap.
template <typename IO>
__global__ void __launch_bounds__(256) hyena_implicit_taps(ImplicitTaps im, IO* h, int64_t N)
{
    __shared__ float w3s[kImpMaxHidden];
    const int64_t o = blockIdx.y;
    for (int i = threadIdx.x; i < im.hp; i += blockDim.x)
        w3s[i] = i < im.H ? im.W3[o * im.H + i] : 0.0f;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= N) return;
    st1<IO>(h + o * N + t, implicit_tap(im, w3s, im.b3[o], im.alpha[o], t));
}

bool single_channel(const Plan& p) { return p.path == HYENA_PATH_LDS1D && p.lds_io == 3; }

}  // namespace

size_t implicit_scratch_bytes(const Plan& p, int32_t hidden)
{
    size_t b = align256((size_t)p.N * (size_t)hidden_pad(hidden) * 4u);
    if (!single_channel(p))
        b += align256((size_t)p.order * (size_t)p.d * (size_t)p.N *
                      (p.io_dtype == HYENA_F32 ? 4u : 2u));
    return b;
}

hyena_status launch_implicit_spectrum(const Plan& p, const hyena_implicit_filter& f, void* H,
                                      void* ws, void* scratch, void* stream)
{
    const hipStream_t s = (hipStream_t)stream;
    if (f.n_freqs < 0 || f.n_freqs > kImpMaxFreqs)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: n_freqs must be in 0..64");
    if (f.hidden < 1 || f.hidden > kImpMaxHidden)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: hidden must be in 1..256");
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
    h.omega = f.omega;
    HY_LAUNCH(kernel_label("hyena_implicit_hidden"), hyena_implicit_hidden,
              dim3((unsigned)((p.N + kImpPos - 1) / kImpPos)), dim3(kImpMaxHidden), 0, s, h);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));

    ImplicitTaps im{};
    im.z2 = h.z2;
    im.W3 = f.W3;
    im.b3 = f.b3;
    im.alpha = f.alpha;
    im.H = f.hidden;
    im.hp = h.hp;
    if (single_channel(p)) {
        Lds1dSpecArgs a{};
        a.spec = H;
        a.tw = static_cast<const float2*>(ws);
        a.twm = a.tw + p.seg[4].off;
        a.N = p.N;
        a.d = p.d;
        a.npairs = p.npairs;
        a.nblocks = (int64_t)p.order * p.d;
        a.tw_off = TwOffsets{(int32_t)p.seg[0].off, (int32_t)p.seg[1].off, (int32_t)p.seg[2].off,
                             (int32_t)p.seg[3].off};
        a.imp = im;
        const int64_t L = p.M / 2;
        return by_storage(p, [&](auto io, auto sp) -> hyena_status {
            using IO = typename decltype(io)::type;
            using SP = typename decltype(sp)::type;
            switch (L) {
#define HY_CASE(LL, I_, S_) \
    case LL:                                                                      \
        return p.circular ? lds1d_real_spectrum_launch<LL, IO, SP, true, true>(a, s) \
                          : lds1d_real_spectrum_launch<LL, IO, SP, true, false>(a, s);
                HY_LDS1D_REAL_SIZES(HY_CASE, 0, 0)
#undef HY_CASE
                default: return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: unsupported length");
            }
        });
    }
    char* taps = static_cast<char*>(scratch) + align256((size_t)p.N * (size_t)h.hp * 4u);
    const dim3 grid((unsigned)((p.N + 255) / 256), (unsigned)(p.order * p.d));
    if (p.io_dtype == HYENA_F32)
        HY_LAUNCH(kernel_label("hyena_implicit_taps", "float"), hyena_implicit_taps<float>, grid,
                  dim3(256), 0, s, im, reinterpret_cast<float*>(taps), p.N);
    else if (p.io_dtype == HYENA_F16)
        HY_LAUNCH(kernel_label("hyena_implicit_taps", "_Float16"), hyena_implicit_taps<_Float16>,
                  grid, dim3(256), 0, s, im, reinterpret_cast<_Float16*>(taps), p.N);
    else
        HY_LAUNCH(kernel_label("hyena_implicit_taps", "unsigned short"), hyena_implicit_taps<uint16_t>,
                  grid, dim3(256), 0, s, im, reinterpret_cast<uint16_t*>(taps), p.N);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
    if (p.path == HYENA_PATH_LDS1D) return launch_lds1d_spectrum(p, taps, H, ws, stream);
    return launch_fourstep_spectrum(p, taps, H, ws, stream);
}

}  // namespace hy
