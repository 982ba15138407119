// implicit.hip -- filter spectra from an implicit filter ("Hyena -- Long
// Convolutions Math", sections "Implicit filters: an MLP over positions" and
// "The decay window"): taps exp(-alpha t) FFN(gamma(t)) with FFN a two-layer
// sine MLP shared over positions.
//
//   hyena_implicit_hidden: z2[t] = sin(omega (W2 sin(omega (W1 gamma(t) + b1))
//                          + b2)) for every position t, into the scratch.
//   hyena_implicit_taps:   h = window . (W3 z2 + b3), a dense [order d] x [N]
//                          contraction over the hidden width, tiled through
//                          LDS, written to the scratch in the plan's storage
//                          type; then the plan's usual spectrum launch
//                          transforms the taps.
#include "dispatch.h"
#include "lds1d_kernels.h"

namespace hy {

namespace {

constexpr int kImpMaxFreqs = 64;
constexpr int kImpMaxHidden = 256;
constexpr int kImpPos = 16;  // positions per workgroup of the hidden kernel
constexpr int kTapTile = 64;  // taps tile: 64 filter rows x 64 positions
constexpr int kTapK = 16;     // hidden features per LDS chunk

// hidden width padded to whole chunks of the taps contraction (zero features)
int64_t hidden_pad(int32_t H) { return (H + kTapK - 1) / kTapK * kTapK; }
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

struct TapArgs {
    const float* z2;  // [N][hp]
    const float* W3;  // [rows][H]
    const float* b3;
    const float* alpha;
    void* h;  // [rows][N], storage type
    int64_t N, rows;
    int32_t H, hp;
};

// Taps h[o][t] = exp(-alpha[o] t) (b3[o] + sum_j W3[o][j] z2[t][j]) for one
// tile of 64 filter rows o = n d + c by 64 positions t.  256 threads, each
// accumulating a 4 x 4 block; the contraction over the hidden width runs in
// chunks of kTapK features, both operands staged through LDS transposed
// ([j][o] and [j][t]) so the inner loop reads one float4 of each.
template <typename IO>
__global__ void __launch_bounds__(256) hyena_implicit_taps(TapArgs a)
{
    constexpr int TT = kTapTile, KC = kTapK, LDW = TT + 4;
    __shared__ __align__(16) float ws[KC][LDW];
    __shared__ __align__(16) float zs[KC][LDW];
    const int e = threadIdx.x;
    const int tx = e & 15, ty = e >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * TT, o0 = (int64_t)blockIdx.y * TT;
    // staging roles: row (or position) e / 4 of the tile, features 4 (e % 4) ..
    const int sl = e >> 2, sj = (e & 3) * 4;
    const int64_t so = o0 + sl, st = t0 + sl;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] = 0.0f;

    for (int j0 = 0; j0 < a.hp; j0 += KC) {
        float wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + sj + i;
            wv[i] = (so < a.rows && j < a.H) ? a.W3[so * a.H + j] : 0.0f;
        }
        const float4 zv = st < a.N ? *reinterpret_cast<const float4*>(a.z2 + st * a.hp + j0 + sj)
                                   : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        __syncthreads();  // previous chunk fully consumed
#pragma unroll
        for (int i = 0; i < 4; ++i) ws[sj + i][sl] = wv[i];
        zs[sj + 0][sl] = zv.x;
        zs[sj + 1][sl] = zv.y;
        zs[sj + 2][sl] = zv.z;
        zs[sj + 3][sl] = zv.w;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            const float4 wa = *reinterpret_cast<const float4*>(&ws[k][4 * ty]);
            const float4 zb = *reinterpret_cast<const float4*>(&zs[k][4 * tx]);
            const float wr[4] = {wa.x, wa.y, wa.z, wa.w};
            const float zc[4] = {zb.x, zb.y, zb.z, zb.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[i][c] = fmaf(wr[i], zc[c], acc[i][c]);
        }
    }

    IO* h = static_cast<IO*>(a.h);
    const int64_t t = t0 + 4 * tx;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t o = o0 + 4 * ty + i;
        if (o >= a.rows) break;
        const float b3 = a.b3[o], al = a.alpha[o];
        float val[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) val[c] = expf(-al * (float)(t + c)) * (b3 + acc[i][c]);
        IO* row = h + o * a.N + t;
        if ((a.N & 3) == 0 && t + 3 < a.N) {
            // row start and t are multiples of 4: two aligned sample pairs
            using PR = typename PairRaw<IO>::type;
            reinterpret_cast<PR*>(row)[0] = narrow_pair<IO>(make_float2(val[0], val[1]));
            reinterpret_cast<PR*>(row)[1] = narrow_pair<IO>(make_float2(val[2], val[3]));
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (t + c < a.N) st1<IO>(row + c, val[c]);
        }
    }
}

}  // namespace

size_t implicit_scratch_bytes(const Plan& p, int32_t hidden)
{
    return align256((size_t)p.N * (size_t)hidden_pad(hidden) * 4u) +
           align256((size_t)p.order * (size_t)p.d * (size_t)p.N *
                    (p.io_dtype == HYENA_F32 ? 4u : 2u));
}

hyena_status launch_implicit_spectrum(const Plan& p, const hyena_implicit_filter& f, void* H,
                                      void* ws, void* scratch, void* stream)
{
    const hipStream_t s = (hipStream_t)stream;
    if (f.n_freqs < 0 || f.n_freqs > kImpMaxFreqs)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: n_freqs must be in 0..64");
    if (f.hidden < 1 || f.hidden > kImpMaxHidden)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: hidden must be in 1..256");
    if ((int64_t)p.order * p.d > 65535ll * kTapTile)
        return fail(HYENA_ERR_UNSUPPORTED, "implicit filter: order * d must be at most 4194240");
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

    TapArgs ta{};
    ta.z2 = h.z2;
    ta.W3 = f.W3;
    ta.b3 = f.b3;
    ta.alpha = f.alpha;
    ta.N = p.N;
    ta.rows = (int64_t)p.order * p.d;
    ta.H = f.hidden;
    ta.hp = h.hp;
    char* taps = static_cast<char*>(scratch) + align256((size_t)p.N * (size_t)h.hp * 4u);
    ta.h = taps;
    const dim3 grid((unsigned)((p.N + kTapTile - 1) / kTapTile),
                    (unsigned)((ta.rows + kTapTile - 1) / kTapTile));
    if (p.io_dtype == HYENA_F32)
        HY_LAUNCH(kernel_label("hyena_implicit_taps", "float"), hyena_implicit_taps<float>, grid,
                  dim3(256), 0, s, ta);
    else if (p.io_dtype == HYENA_F16)
        HY_LAUNCH(kernel_label("hyena_implicit_taps", "_Float16"), hyena_implicit_taps<_Float16>,
                  grid, dim3(256), 0, s, ta);
    else
        HY_LAUNCH(kernel_label("hyena_implicit_taps", "unsigned short"), hyena_implicit_taps<uint16_t>,
                  grid, dim3(256), 0, s, ta);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(HYENA_ERR_DEVICE, hipGetErrorString(e));
    if (p.path == HYENA_PATH_LDS1D) return launch_lds1d_spectrum(p, taps, H, ws, stream);
    return launch_fourstep_spectrum(p, taps, H, ws, stream);
}

}  // namespace hy
