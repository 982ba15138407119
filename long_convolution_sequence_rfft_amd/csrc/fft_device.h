// fft_device.h -- register-level FFT building blocks for gfx950 (wave64).
//
// The transforms are radix-2^k decimation-in-time networks evaluated on
// values held in VGPRs ("Hyena -- Long Convolutions Math", section "Counting
// the cost": a length-M transform as log2(M) radix-2 stages).  Several
// radix-2 stages are fused into one radix-R pass in registers; passes
// exchange data through LDS (see the kernels).  Everything is float32.
//
// Conventions: DIR = -1 is the forward transform X[k] = sum x[t] W^{kt},
// W = exp(-2 pi i / R); DIR = +1 is the unscaled inverse.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hy {

// ---------------------------------------------------------------------------
// complex helpers (float2 = re, im)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 w)
{
    return make_float2(fmaf(a.x, w.x, -a.y * w.y), fmaf(a.x, w.y, a.y * w.x));
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
// a * w for DIR = -1, a * conj(w) for DIR = +1 (twiddle tables hold forward roots)
template <int DIR>
__device__ __forceinline__ float2 ctw(float2 a, float2 w)
{
    if constexpr (DIR < 0) return cmul(a, w);
    else return make_float2(fmaf(a.x, w.x, a.y * w.y), fmaf(a.y, w.x, -a.x * w.y));
}

// ---------------------------------------------------------------------------
// Roots of unity of order 32, exact to float rounding: cos(2 pi m / 32)
// for m = 0..8 (the rest follow by symmetry).
// ---------------------------------------------------------------------------
struct Roots32 {
    static constexpr float c[9] = {
        1.0f,
        0.98078528040323044913f,
        0.92387953251128675613f,
        0.83146961230254523708f,
        0.70710678118654752440f,
        0.55557023301960222474f,
        0.38268343236508977173f,
        0.19509032201612826785f,
        0.0f};
};

__host__ __device__ constexpr float cos32(int m)
{
    m = ((m % 32) + 32) % 32;
    return m <= 8 ? Roots32::c[m] : m <= 16 ? -Roots32::c[16 - m]
                                  : m <= 24 ? -Roots32::c[m - 16] : Roots32::c[32 - m];
}
__host__ __device__ constexpr float sin32(int m) { return cos32(m - 8); }

// Radix-2 DIT butterfly with twiddle W = exp(DIR 2 pi i mq / 32):
//   a <- a + W b,  b <- a - W b.
// General twiddles use the fused form (a + W b via two FMAs per component,
// a - W b = 2a - (a + W b)): 6 VALU ops instead of 8.
template <int DIR>
__device__ __forceinline__ void bfly(float2& a, float2& b, int mq)
{
    mq &= 31;
    if (mq == 0) {
        const float2 t = b;
        b = csub(a, t);
        a = cadd(a, t);
    } else if (mq == 8) {  // W = DIR * i
        const float tx = DIR < 0 ? b.y : -b.y;
        const float ty = DIR < 0 ? -b.x : b.x;
        b = make_float2(a.x - tx, a.y - ty);
        a = make_float2(a.x + tx, a.y + ty);
    } else {
        const float wr = cos32(mq), wi = DIR < 0 ? -sin32(mq) : sin32(mq);
        const float ox = fmaf(wr, b.x, fmaf(-wi, b.y, a.x));
        const float oy = fmaf(wr, b.y, fmaf(wi, b.x, a.y));
        b.x = fmaf(2.0f, a.x, -ox);
        b.y = fmaf(2.0f, a.y, -oy);
        a.x = ox;
        a.y = oy;
    }
}

// Only the "a + W b" half of the butterfly (for pruned outputs).
template <int DIR>
__device__ __forceinline__ void bfly_top(float2& a, const float2& b, int mq)
{
    mq &= 31;
    if (mq == 0) {
        a = cadd(a, b);
    } else if (mq == 8) {
        a = make_float2(a.x + (DIR < 0 ? b.y : -b.y), a.y + (DIR < 0 ? -b.x : b.x));
    } else {
        const float wr = cos32(mq), wi = DIR < 0 ? -sin32(mq) : sin32(mq);
        const float ox = fmaf(wr, b.x, fmaf(-wi, b.y, a.x));
        const float oy = fmaf(wr, b.y, fmaf(wi, b.x, a.y));
        a.x = ox;
        a.y = oy;
    }
}

__host__ __device__ constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n >> 1); }
__host__ __device__ constexpr int bitrev(int i, int R)
{
    int r = 0;
    for (int b = 1; b < R; b <<= 1) r = (r << 1) | ((i & b) ? 1 : 0);
    return r;
}

// In-register DFT of length R (2 <= R <= 32) on v[0..R), natural order in
// and out.  HALF_IN: inputs v[R/2..R) are known to be zero (zero-padded
// signal), so the first radix-2 stage is a copy.  HALF_OUT: only outputs
// v[0..R/2) are needed; the last stage computes just those.
template <int R, int DIR, bool HALF_IN = false, bool HALF_OUT = false>
__device__ __forceinline__ void dft(float2* v)
{
    static_assert(R >= 2 && R <= 32 && (R & (R - 1)) == 0, "radix");
    float2 w[R];
#pragma unroll
    for (int i = 0; i < R; ++i) w[i] = v[bitrev(i, R)];
#pragma unroll
    for (int len = 2; len <= R; len <<= 1) {
        const int half = len >> 1;
#pragma unroll
        for (int start = 0; start < R; start += len) {
#pragma unroll
            for (int k = 0; k < half; ++k) {
                const int mq = k * (32 / len);
                if (HALF_IN && len == 2) {
                    // partner is a zero input: both outputs equal the live one
                    w[start + 1] = w[start];
                } else if (HALF_OUT && len == R) {
                    bfly_top<DIR>(w[start + k], w[start + k + half], mq);
                } else {
                    bfly<DIR>(w[start + k], w[start + k + half], mq);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < (HALF_OUT ? R / 2 : R); ++i) v[i] = w[i];
}

// LDS index padding: one spare word per 32, so power-of-two strides up to 32
// spread over distinct banks.
__device__ __forceinline__ int lpad(int i) { return i + (i >> 5); }
__host__ __device__ constexpr int lds_words(int M) { return M + (M >> 5); }

// ---------------------------------------------------------------------------
// bfloat16 storage (round to nearest even on store, exact widening on load)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    // the hardware conversion: round to nearest even, NaN stays a (quiet) NaN
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// XCD-aware block order: the dispatcher hands consecutive workgroup ids to
// the eight XCDs in turn, so id i runs on XCD i % 8.  Remap so that each XCD
// walks a contiguous range of work items; neighbouring channel pairs then
// share that XCD's L2 while they read the same channels-last cache lines.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks)
{
    if (nblocks % 8 != 0) return bid;
    return (bid % 8) * (nblocks / 8) + bid / 8;
}

}  // namespace hy
