// stockham.h -- one length-L complex transform held by a group of threads,
// radix passes in registers, exchanges through LDS (Stockham autosort: no
// bit-reversal pass), plus the spectral products of the channel-pair and the
// single-channel (packed real) forms.
//
// A radix-R pass with sub-transform length NS reads butterfly j's inputs at
// j + r L/R, multiplies input r by W_{NS R}^{r k} (k = j mod NS), takes a
// length-R DFT and writes output s to (j - k) R + k + s NS; after the last
// pass the transform is in natural order.  The passes are R0, R1 (optional),
// RL forward and RL, R1, R0 inverse, so the inverse's last pass leaves each
// thread holding exactly the time samples the next forward pass starts from.
//
// The convolution theorem and the 2N zero padding that keeps the cyclic
// product causal follow "Hyena -- Long Convolutions Math", sections "The
// convolution theorem" and "Linear vs circular".
#pragma once

#include "fft_device.h"
#include "plan.h"
#include "timing.h"

namespace hy {

template <int L>
struct FftShape {
    static constexpr int PTS = lds1d_pts(L);  // complex values per thread
    static constexpr int T = L / PTS;         // threads per transform
    static constexpr int RL = lds1d_rl(L);
    static constexpr int R0 = lds1d_r0(L);
    static constexpr int R1 = lds1d_r1(L);
    static constexpr int Q0 = PTS / R0;  // butterflies per thread in the R0 pass
    static constexpr int Q1 = PTS / R1;
    static constexpr int LW = lds_words(L);
    static_assert(R0 * R1 * RL == L, "radix plan");
    static_assert(RL * 2 == PTS, "last pass must give two butterflies per thread");
};

// ---------------------------------------------------------------------------
// storage access (float32, bfloat16 stored as uint16_t, or _Float16)
//
// Global accesses take a wave-uniform base pointer and a 32-bit per-lane byte
// offset, which maps onto the scalar-base + vector-offset addressing form
// (one VGPR per access instead of a 64-bit address pair).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ const T& at_bytes(const void* base, uint32_t off)
{
    return *reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}
template <typename T>
__device__ __forceinline__ T& at_bytes(void* base, uint32_t off)
{
    return *reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// Storage types: float (float32), uint16_t (bfloat16 bits) and _Float16
// (IEEE binary16).  Two 16-bit values travel as one dword, the first in the
// low half.
template <typename IO>
constexpr bool is_bf16() { return sizeof(IO) == 2 && !__is_same(IO, _Float16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f)
{
    // hardware conversion, round to nearest even; beyond 65504 gives +-inf
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <typename IO>
__device__ __forceinline__ float ld1(const IO* p)
{
    if constexpr (sizeof(IO) == 4) return *p;
    else if constexpr (is_bf16<IO>()) return bf16_to_f32(*p);
    else return (float)*p;
}

template <typename IO>
__device__ __forceinline__ void st1(IO* p, float v)
{
    if constexpr (sizeof(IO) == 4) *p = v;
    else if constexpr (is_bf16<IO>()) *p = f32_to_bf16(v);
    else *p = (_Float16)v;
}

// Raw channel-pair (or sample-pair) value as stored (float2 for f32, one
// dword for two 16-bit values); widened at use so prefetched values occupy as
// few VGPRs as possible.
template <typename IO>
struct PairRaw {
    using type = uint32_t;
};
template <>
struct PairRaw<float> {
    using type = float2;
};

template <typename IO>
__device__ __forceinline__ float2 widen_pair(const typename PairRaw<IO>::type& w)
{
    if constexpr (sizeof(IO) == 4) return w;
    else if constexpr (is_bf16<IO>())
        return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    else return make_float2(f16_bits_to_f32(w & 0xffffu), f16_bits_to_f32(w >> 16));
}

template <typename IO>
__device__ __forceinline__ typename PairRaw<IO>::type narrow_pair(float2 v)
{
    if constexpr (sizeof(IO) == 4) return v;
    else if constexpr (is_bf16<IO>())
        return (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    else return f32_to_f16_bits(v.x) | (f32_to_f16_bits(v.y) << 16);
}

// Channel pair (c, c+1) of a channels-last row.  EVEN: d is even, so the
// pair is one aligned 8-byte (f32) or 4-byte (16-bit types) access.
template <typename IO, bool EVEN>
__device__ __forceinline__ float2 load_pair(const IO* row, bool has_b)
{
    if constexpr (EVEN) {
        return widen_pair<IO>(*reinterpret_cast<const typename PairRaw<IO>::type*>(row));
    } else {
        return make_float2(ld1<IO>(row), has_b ? ld1<IO>(row + 1) : 0.0f);
    }
}

template <typename IO, bool EVEN>
__device__ __forceinline__ void store_pair(IO* row, float2 v, bool has_b)
{
    if constexpr (EVEN) {
        *reinterpret_cast<typename PairRaw<IO>::type*>(row) = narrow_pair<IO>(v);
    } else {
        st1<IO>(row, v.x);
        if (has_b) st1<IO>(row + 1, v.y);
    }
}

// EVEN pair at byte offset `off` from a uniform base.
template <typename IO>
__device__ __forceinline__ typename PairRaw<IO>::type load_pair_raw(const IO* base, uint32_t off)
{
    return at_bytes<typename PairRaw<IO>::type>(base, off);
}

template <typename IO>
__device__ __forceinline__ void store_pair_at(IO* base, uint32_t off, float2 v)
{
    at_bytes<typename PairRaw<IO>::type>(base, off) = narrow_pair<IO>(v);
}

// One spectrum entry (P, Q): a float4 for f32, four bfloat16 in 8 bytes.
template <typename SP>
__device__ __forceinline__ void load_entry(const SP* spec, int64_t e, float2& P, float2& Q)
{
    if constexpr (sizeof(SP) == 4) {
        const float4 r = reinterpret_cast<const float4*>(spec)[e];
        P = make_float2(r.x, r.y);
        Q = make_float2(r.z, r.w);
    } else {
        const uint2 r = reinterpret_cast<const uint2*>(spec)[e];
        P = make_float2(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u));
        Q = make_float2(__uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
    }
}

template <typename SP>
__device__ __forceinline__ void store_entry(SP* spec, int64_t e, float2 P, float2 Q)
{
    if constexpr (sizeof(SP) == 4) {
        reinterpret_cast<float4*>(spec)[e] = make_float4(P.x, P.y, Q.x, Q.y);
    } else {
        uint2 r;
        r.x = (uint32_t)f32_to_bf16(P.x) | ((uint32_t)f32_to_bf16(P.y) << 16);
        r.y = (uint32_t)f32_to_bf16(Q.x) | ((uint32_t)f32_to_bf16(Q.y) << 16);
        reinterpret_cast<uint2*>(spec)[e] = r;
    }
}

// Elements of one spectrum entry, in units of SP (four reals per entry).
constexpr int kEntryElems = 4;

// ---------------------------------------------------------------------------
// pass pieces
// ---------------------------------------------------------------------------
// Every access below is lpad(A + c) with a run-time A and a compile-time c.
// For these Stockham patterns A mod 32 + c mod 32 < 32 always holds (reads:
// A = j < L/R and c a multiple of L/R, L/R a power of two; writes: A is the
// output base and c = s NS, both aligned to NS R or to 32), so
// lpad(A + c) = lpad(A) + c + c/32 and c becomes an instruction offset.
template <int R, int NS>
__device__ __forceinline__ void lds_write(float* sre, float* sim, const float2* v, int j)
{
    const int k = j & (NS - 1);
    const int pb = lpad((j - k) * R + k);
#pragma unroll
    for (int s = 0; s < R; ++s) {
        const int c = s * NS;
        const int i = pb + c + (c >> 5);
        sre[i] = v[s].x;
        sim[i] = v[s].y;
    }
}

template <int R, int L>
__device__ __forceinline__ void lds_read(const float* sre, const float* sim, float2* v, int j)
{
    const int pb = lpad(j);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int c = r * (L / R);
        const int i = pb + c + (c >> 5);
        v[r] = make_float2(sre[i], sim[i]);
    }
}

// Natural positions j + r L/R for r < RN (RN <= R), j < L/R: the R0-pass
// sample layout.  Same carry-free addressing as lds_read.
template <int RN, int R, int L>
__device__ __forceinline__ void lds_read_first(const float* sre, const float* sim, float2* v, int j)
{
    const int pb = lpad(j);
#pragma unroll
    for (int r = 0; r < RN; ++r) {
        const int c = r * (L / R);
        const int i = pb + c + (c >> 5);
        v[r] = make_float2(sre[i], sim[i]);
    }
}

template <int RN, int R, int L>
__device__ __forceinline__ void lds_write_first(float* sre, float* sim, const float2* v, int j)
{
    const int pb = lpad(j);
#pragma unroll
    for (int r = 0; r < RN; ++r) {
        const int c = r * (L / R);
        const int i = pb + c + (c >> 5);
        sre[i] = v[r].x;
        sim[i] = v[r].y;
    }
}

// Twiddles of butterfly k of a pass with sub-transform length NS: input r
// takes tab[(r - 1) NS + k].  Loaded into registers ahead of the barrier that
// precedes the pass, so the load latency overlaps the LDS exchange.
// `tab` is wave-uniform.  Raw buffer loads: the table base sits in a scalar
// descriptor, the row offset (r - 1) NS in a scalar register and the lane
// offset in one VGPR, so no load needs address arithmetic of its own (a
// global load would need a 64-bit add per row, since the rows are further
// apart than its immediate offset reaches).
template <int R, int NS>
__device__ __forceinline__ void load_tw(float2* w, const float2* tab, uint32_t k)
{
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float2*>(tab), (short)0, 0x7fffffff, 0x00020000);
    const uint32_t koff = k * 8u;
#pragma unroll
    for (int r = 1; r < R; ++r) {
        typedef float f2v __attribute__((ext_vector_type(2)));
        const f2v t = __builtin_bit_cast(f2v, __builtin_amdgcn_raw_buffer_load_b64(rs, koff, (r - 1) * NS * 8, 0));
        w[r - 1] = make_float2(t.x, t.y);
    }
}

template <int R, int DIR>
__device__ __forceinline__ void apply_tw(float2* v, const float2* w)
{
#pragma unroll
    for (int r = 1; r < R; ++r) v[r] = ctw<DIR>(v[r], w[r - 1]);
}

// Twiddle-table offsets (float2 units) of one transform length.
struct TwOffsets {
    int32_t f1, fL, i1, i0;
};

// Forward transform.  On entry v holds the R0-pass inputs of butterflies
// tau + q T (values r < R0/2; the upper half is the zero padding and is never
// read).  On return v[0..RL) and v[RL..2RL) hold the outputs of last-pass
// butterflies j1 and j2: bins j1 + s L/RL and j2 + s L/RL.
// sync_first: LDS may still be read by the previous step (WAR barrier).
// `prefetch` runs after the last exchange's reads (global loads for the
// caller, whose latency then overlaps the last pass's arithmetic).
// Every pass with Q > 1 butterflies per thread shares one twiddle set in the
// R1 pass (T is a multiple of R0 whenever R1 > 1).
// HALF_IN = false: all R0 inputs per butterfly hold data (no zero padding).
template <int L, bool HALF_IN = true, typename F>
__device__ __forceinline__ void fwd_transform(float2* v, float* sre, float* sim, const float2* tw,
                                              TwOffsets o, int tau, int j1, int j2,
                                              bool sync_first, F&& prefetch)
{
    using S = FftShape<L>;
    constexpr int T = S::T, R0 = S::R0, R1 = S::R1, RL = S::RL;
    constexpr int NSL = L / RL;
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) dft<R0, -1, HALF_IN, false>(&v[q * R0]);
    if (sync_first) __syncthreads();
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) lds_write<R0, 1>(sre, sim, &v[q * R0], tau + q * T);
    if constexpr (R1 > 1) {
        static_assert(T % R0 == 0, "shared R1-pass twiddles");
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
    float2 wa[RL - 1], wb[RL - 1];
    load_tw<RL, NSL>(wa, tw + o.fL, j1);
    load_tw<RL, NSL>(wb, tw + o.fL, j2);
    __syncthreads();
    lds_read<RL, L>(sre, sim, &v[0], j1);
    lds_read<RL, L>(sre, sim, &v[RL], j2);
    apply_tw<RL, -1>(&v[0], wa);
    apply_tw<RL, -1>(&v[RL], wb);
    prefetch();
    dft<RL, -1>(&v[0]);
    dft<RL, -1>(&v[RL]);
}

// Inverse transform (unscaled) from the last-pass registers (butterflies j1,
// j2) back to the R0-pass layout: v[q R0 + s], s < R0/2, is sample
// tau + q T + s L/R0.  Only the first half of the samples is produced.
// `prefetch` runs after the last exchange's reads (global loads for the
// caller, e.g. the gate values, whose latency overlaps the last pass).
// HALF_OUT = false: all L samples are produced (v[q R0 + s], s < R0).
template <int L, bool HALF_OUT = true, typename F>
__device__ __forceinline__ void inv_transform(float2* v, float* sre, float* sim, const float2* tw,
                                              TwOffsets o, int tau, int j1, int j2, F&& prefetch)
{
    using S = FftShape<L>;
    constexpr int T = S::T, R0 = S::R0, R1 = S::R1, RL = S::RL;
    constexpr int NS0 = L / R0;
    dft<RL, +1>(&v[0]);
    dft<RL, +1>(&v[RL]);
    __syncthreads();
    lds_write<RL, 1>(sre, sim, &v[0], j1);
    lds_write<RL, 1>(sre, sim, &v[RL], j2);
    if constexpr (R1 > 1) {
        static_assert(T % RL == 0, "shared R1-pass twiddles");
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
    float2 w0[S::Q0][R0 - 1];
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) load_tw<R0, NS0>(w0[q], tw + o.i0, tau + q * T);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) {
        lds_read<R0, L>(sre, sim, &v[q * R0], tau + q * T);
        apply_tw<R0, +1>(&v[q * R0], w0[q]);
    }
    prefetch();
#pragma unroll
    for (int q = 0; q < S::Q0; ++q) dft<R0, +1, false, HALF_OUT>(&v[q * R0]);
}

// ---------------------------------------------------------------------------
// Channel-pair spectral product.  Two real channels a, b ride in one complex
// signal z = a + i b.  With Z = DFT(z), the spectrum of a*ha + i (b*hb) is
//   Y[k] = Z[k] P[k] + conj(Z[-k]) Q[k],  P = (Ha + Hb)/2,  Q = (Ha - Hb)/2,
// because DFT(a) = (Z[k] + conj Z[-k])/2 and DFT(b) = (Z[k] - conj Z[-k])/2i.
// A bin and its mirror are computed together from one (P, Q) entry:
//   Y[-k] = Z[-k] conj(P[k]) + conj(Z[k]) conj(Q[k]).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void pair_product(float2& zp, float2& zm, float2 P, float2 Q)
{
    const float ypx = fmaf(zp.x, P.x, fmaf(-zp.y, P.y, fmaf(zm.x, Q.x, zm.y * Q.y)));
    const float ypy = fmaf(zp.x, P.y, fmaf(zp.y, P.x, fmaf(zm.x, Q.y, -zm.y * Q.x)));
    const float ymx = fmaf(zm.x, P.x, fmaf(zm.y, P.y, fmaf(zp.x, Q.x, -zp.y * Q.y)));
    const float ymy = fmaf(zm.y, P.x, fmaf(-zm.x, P.y, fmaf(-zp.x, Q.y, -zp.y * Q.x)));
    zp = make_float2(ypx, ypy);
    zm = make_float2(ymx, ymy);
}

// A self-mirrored bin (k = -k): P and Q are real.
__device__ __forceinline__ float2 self_product(float2 z, float P, float Q)
{
    return make_float2(z.x * (P + Q), z.y * (P - Q));
}

// Filter side: from Z = DFT(ha + i hb) at a bin and its mirror, the entry
// ((Ha + Hb), (Ha - Hb)) * scale with Ha = (zp + conj zm)/2, Hb = (zp - conj zm)/2i.
__device__ __forceinline__ void entry_from_pair(float2 zp, float2 zm, float scale, float2& P,
                                                float2& Q)
{
    const float2 Ha = make_float2(0.5f * (zp.x + zm.x), 0.5f * (zp.y - zm.y));
    const float2 Hb = make_float2(0.5f * (zp.y + zm.y), -0.5f * (zp.x - zm.x));
    P = make_float2((Ha.x + Hb.x) * scale, (Ha.y + Hb.y) * scale);
    Q = make_float2((Ha.x - Hb.x) * scale, (Ha.y - Hb.y) * scale);
}

// Raw spectrum entry as loaded (widened at use): float4 or four bfloat16.
template <typename SP>
struct EntryRaw;
template <>
struct EntryRaw<float> {
    using type = float4;
};
template <>
struct EntryRaw<uint16_t> {
    using type = uint2;
};

template <typename SP>
__device__ __forceinline__ void widen_entry(const typename EntryRaw<SP>::type& r, float2& P,
                                            float2& Q)
{
    if constexpr (sizeof(SP) == 4) {
        P = make_float2(r.x, r.y);
        Q = make_float2(r.z, r.w);
    } else {
        P = make_float2(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u));
        Q = make_float2(__uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
    }
}

// Entries e = 0..RL-1 of thread tau of one length-L transform (entry index
// e T + tau: lanes read consecutive entries).  Raw buffer loads from the
// transform's (wave-uniform) entry base: the entry offset e T sits in a
// scalar register and the lane offset in one VGPR, where global loads would
// need a 64-bit address add for every entry beyond the immediate-offset
// range.  All offsets are below L/2 entries.
template <int L, typename SP>
__device__ __forceinline__ void load_entries(typename EntryRaw<SP>::type* ent, const SP* spec,
                                             int tau)
{
    using S = FftShape<L>;
    using Raw = typename EntryRaw<SP>::type;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<SP*>(spec), (short)0, 0x7fffffff, 0x00020000);
    const uint32_t off = (uint32_t)tau * (uint32_t)sizeof(Raw);
#pragma unroll
    for (int e = 0; e < S::RL; ++e) {
        const uint32_t soff = (uint32_t)(e * S::T) * (uint32_t)sizeof(Raw);
        if constexpr (sizeof(Raw) == 16) {
            typedef float v4 __attribute__((ext_vector_type(4)));
            const v4 t = __builtin_bit_cast(v4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, soff, 0));
            ent[e] = make_float4(t.x, t.y, t.z, t.w);
        } else {
            static_assert(sizeof(Raw) == 8, "entry width");
            typedef unsigned v2 __attribute__((ext_vector_type(2)));
            const v2 t = __builtin_bit_cast(v2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, soff, 0));
            ent[e] = make_uint2(t.x, t.y);
        }
    }
}

// Mirror-paired product on the last-pass registers of one length-L transform.
//   tau > 0: last-pass butterflies tau and 2T - tau; slot e pairs output e of
//            the first with output RL-1-e of the second; the bin <= L/2 is
//            the first's for e < RL/2, the second's otherwise.
//   tau = 0: butterflies 0 and T are their own mirrors.  Slots e < RL/2 pair
//            outputs (e, RL-1-e) of butterfly T, slots e > RL/2 outputs
//            (RL-e, e) of butterfly 0, and slot RL/2 packs the self-mirrored
//            bins 0 and L/2 (real P, Q).
// dp, dq: real offsets added to every P and Q (the folded feedthrough).
// Every lane runs the same instruction stream; thread 0's operands and
// results differ only through selects.
template <int L, typename SP>
__device__ __forceinline__ void spectral_product(float2* v, const typename EntryRaw<SP>::type* ent,
                                                 int tau, float dp, float dq)
{
    using S = FftShape<L>;
    constexpr int RL = S::RL, H = RL / 2;
    const bool t0 = tau == 0;
    float2 yp[RL], ym[RL];
#pragma unroll
    for (int e = 0; e < RL; ++e) {
        float2 P, Q;
        widen_entry<SP>(ent[e], P, Q);
        float2 y0, yh;
        if (e == H) {
            // thread 0: the self-mirrored bins 0 (v[0]) and L/2 (v[H])
            y0 = self_product(v[0], P.x + dp, Q.x + dq);
            yh = self_product(v[H], P.y + dp, Q.y + dq);
        }
        P.x += dp;
        Q.x += dq;
        const int ip = e < H ? e : 2 * RL - 1 - e;  // the bin <= L/2
        const int im = e < H ? 2 * RL - 1 - e : e;
        float2 p = v[ip];
        if (e < H) p = t0 ? v[RL + e] : p;
        if (e > H) p = t0 ? v[RL - e] : p;
        float2 m = v[im];
        pair_product(p, m, P, Q);
        if (e == H) {
            p = t0 ? y0 : p;
            m = t0 ? yh : m;
        }
        yp[e] = p;
        ym[e] = m;
    }
    // general: v[ip(e)] = yp[e], v[im(e)] = ym[e]; thread 0 writes butterfly
    // 0's low half and butterfly T's low half from its own slots
#pragma unroll
    for (int e = 0; e < H; ++e) {
        v[e] = t0 ? (e == 0 ? yp[H] : yp[RL - e]) : yp[e];
        v[RL + e] = t0 ? yp[e] : yp[RL - 1 - e];
        v[H + e] = ym[H + e];
        v[2 * RL - 1 - e] = ym[e];
    }
}

// Filter side of the same layout: write the entries of one transform.
template <int L, typename SP>
__device__ __forceinline__ void store_spectrum_entries(const float2* v, SP* spec, int tau,
                                                       float scale)
{
    using S = FftShape<L>;
    constexpr int T = S::T, RL = S::RL;
    float2 P, Q;
    if (tau != 0) {
#pragma unroll
        for (int e = 0; e < RL; ++e) {
            if (e < RL / 2) entry_from_pair(v[e], v[2 * RL - 1 - e], scale, P, Q);
            else entry_from_pair(v[2 * RL - 1 - e], v[e], scale, P, Q);
            store_entry(spec, e * T + tau, P, Q);
        }
    } else {
        // thread 0 in the product's slot order
        constexpr int H = RL / 2;
#pragma unroll
        for (int e = 0; e < H; ++e) {
            entry_from_pair(v[RL + e], v[2 * RL - 1 - e], scale, P, Q);
            store_entry(spec, e * T, P, Q);
        }
        const float2 z0 = v[0], zh = v[H];
        store_entry(spec, H * T, make_float2((z0.x + z0.y) * scale, (zh.x + zh.y) * scale),
                    make_float2((z0.x - z0.y) * scale, (zh.x - zh.y) * scale));
#pragma unroll
        for (int e = H + 1; e < RL; ++e) {
            entry_from_pair(v[RL - e], v[e], scale, P, Q);
            store_entry(spec, e * T, P, Q);
        }
    }
}

// ---------------------------------------------------------------------------
// Single-channel spectral product.  One real channel x of the length-M
// zero-padded sequence rides in z[m] = x[2m] + i x[2m+1], a complex signal of
// length L = M/2 with Z = DFT_L(z).  E and O, the transforms of the even and
// odd samples, are E[k] = (Z[k] + conj Z[L-k])/2 and
// O[k] = (Z[k] - conj Z[L-k])/2i, and X[k] = E[k] + W^k O[k],
// X[k+L] = E[k] - W^k O[k] with W = exp(-2 pi i/M).  Multiplying X by the
// filter's transfer function H and packing the product the same way gives
//   Z'[k]   = (S - s Dl) Z[k] + i c Dl conj Z[L-k]
//   Z'[L-k] = conj(S + s Dl) Z[L-k] + i c conj(Dl) conj Z[k]
// with S = (H[k] + conj H[L-k])/2, Dl = (H[k] - conj H[L-k])/2 and
// W^k = c - i s; the inverse DFT_L of Z' then holds y[2m] + i y[2m+1].  One
// entry (S, Dl) serves a bin and its mirror.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void real_pair_product(float2& zk, float2& zm, float2 S, float2 Dl,
                                                  float c, float s)
{
    const float2 U = make_float2(Dl.x * s, Dl.y * s);
    const float2 V = make_float2(Dl.x * c, Dl.y * c);
    const float2 A = make_float2(S.x - U.x, S.y - U.y);   // coefficient of Z[k]
    const float2 Ap = make_float2(S.x + U.x, S.y + U.y);  // conj of the coefficient of Z[L-k]
    const float ykx = fmaf(A.x, zk.x, fmaf(-A.y, zk.y, fmaf(-V.y, zm.x, V.x * zm.y)));
    const float yky = fmaf(A.x, zk.y, fmaf(A.y, zk.x, fmaf(V.x, zm.x, V.y * zm.y)));
    const float ymx = fmaf(Ap.x, zm.x, fmaf(Ap.y, zm.y, fmaf(V.y, zk.x, V.x * zk.y)));
    const float ymy = fmaf(Ap.x, zm.y, fmaf(-Ap.y, zm.x, fmaf(V.x, zk.x, -V.y * zk.y)));
    zk = make_float2(ykx, yky);
    zm = make_float2(ymx, ymy);
}

// Filter side: the entry (S, Dl) * scale of bin k from Z = DFT_L of the packed
// filter at k and L-k: S = E[k], Dl = W^k O[k].
__device__ __forceinline__ void entry_from_real(float2 zk, float2 zm, float c, float s, float scale,
                                                float2& S, float2& Dl)
{
    S = make_float2(0.5f * (zk.x + zm.x) * scale, 0.5f * (zk.y - zm.y) * scale);
    // O = (Z[k] - conj Z[L-k]) / 2i
    const float ox = 0.5f * (zk.y + zm.y), oy = -0.5f * (zk.x - zm.x);
    Dl = make_float2((c * ox + s * oy) * scale, (c * oy - s * ox) * scale);
}

// exp(-2 pi i e / (2 RL)), the step between a thread's last-pass outputs.
template <int RL>
__device__ __forceinline__ float2 out_step_root(int e)
{
    const int m = e * (32 / (2 * RL));
    return make_float2(cos32(m), -sin32(m));
}

// W^k of output e of a thread's first last-pass butterfly (bin base + e L/RL),
// from W^base: cos and sin of 2 pi k / M.
template <int RL>
__device__ __forceinline__ void bin_cs(float2 wbase, int e, float& c, float& s)
{
    const float2 r = out_step_root<RL>(e);
    const float2 w = cmul(wbase, r);
    c = w.x;
    s = -w.y;
}

// Single-channel product on the last-pass registers of one length-L
// transform.  Thread tau holds butterflies tau and 2T - tau (0 and T for
// tau = 0); slot e = 0..RL-1 is one bin k and its mirror L - k:
//   tau > 0: k = tau + e L/RL (output e of butterfly tau), mirror output
//            RL-1-e of butterfly 2T - tau.
//   tau = 0: butterflies 0 and T are their own mirrors.  Slots e < RL/2:
//            k = T + e L/RL, outputs (e, RL-1-e) of butterfly T; slots
//            e > RL/2: k = e L/RL, outputs (e, RL-e) of butterfly 0; slot
//            RL/2 packs the self-mirrored bins 0 and L/2 as
//            ((S0, Re H[L/2]), (Dl0, Im H[L/2])).
// Every lane runs the same instruction stream: thread 0's operands, twiddles
// and results differ from the others' only through selects, so the wave that
// holds thread 0 does no extra pass of its own.
// wbase = W^tau (tau > 0) or W^T (tau = 0); dp = D/L (folded feedthrough).
template <int L, typename SP>
__device__ __forceinline__ void real_product(float2* v, const typename EntryRaw<SP>::type* ent,
                                             int tau, float dp, float2 wbase)
{
    using S = FftShape<L>;
    constexpr int RL = S::RL, H = RL / 2;
    const bool t0 = tau == 0;
    float2 ya[RL], yb[RL];
    // W^k of slot e + RL/2 is -i W^k of slot e: (c, s) -> (-s, c)
    float cs_c[H], cs_s[H];
#pragma unroll
    for (int e = 0; e < RL; ++e) {
        float2 Sv, Dv;
        widen_entry<SP>(ent[e], Sv, Dv);
        Sv.x += dp;
        float c, s;
        if (e < H) {
            bin_cs<RL>(wbase, e, c, s);
            cs_c[e] = c;
            cs_s[e] = s;
        } else {
            c = -cs_s[e - H];
            s = cs_c[e - H];
        }
        float2 a = v[e], b = v[2 * RL - 1 - e];
        if (e < H) {
            a = t0 ? v[RL + e] : a;
        } else if (e > H) {
            const float2 r = out_step_root<RL>(e);
            b = t0 ? v[RL - e] : b;
            c = t0 ? r.x : c;
            s = t0 ? -r.y : s;
        }
        float2 z0h, z00;
        if (e == H) {
            // thread 0: bin L/2 (zh = v[H]) and bin 0 (z0 = v[0])
            const float2 zh = v[H], z0 = v[0];
            const float Hr = Sv.y + dp, Hi = Dv.y;
            z0h = make_float2(fmaf(Hr, zh.x, Hi * zh.y), fmaf(Hr, zh.y, -Hi * zh.x));
            z00 = make_float2(fmaf(Sv.x, z0.x, Dv.x * z0.y), fmaf(Sv.x, z0.y, Dv.x * z0.x));
        }
        real_pair_product(a, b, Sv, Dv, c, s);
        if (e == H) {
            a = t0 ? z0h : a;
            b = t0 ? z00 : b;
        }
        ya[e] = a;
        yb[e] = b;
    }
#pragma unroll
    for (int e = 0; e < H; ++e) {
        v[e] = t0 ? (e == 0 ? yb[H] : yb[RL - e]) : ya[e];
        v[RL + e] = t0 ? ya[e] : yb[RL - 1 - e];
        v[H + e] = ya[H + e];
        v[2 * RL - 1 - e] = yb[e];
    }
}

// Filter side of the single-channel layout: write the entries of one transform.
template <int L, typename SP>
__device__ __forceinline__ void store_real_entries(const float2* v, SP* spec, int tau, float scale,
                                                   float2 wbase)
{
    using S = FftShape<L>;
    constexpr int T = S::T, RL = S::RL;
    float2 Sv, Dv;
    float c, s;
    if (tau != 0) {
#pragma unroll
        for (int e = 0; e < RL; ++e) {
            bin_cs<RL>(wbase, e, c, s);
            entry_from_real(v[e], v[2 * RL - 1 - e], c, s, scale, Sv, Dv);
            store_entry(spec, e * T + tau, Sv, Dv);
        }
    } else {
        // thread 0 in the product's slot order
        constexpr int H = RL / 2;
#pragma unroll
        for (int e = 0; e < H; ++e) {
            bin_cs<RL>(wbase, e, c, s);
            entry_from_real(v[RL + e], v[2 * RL - 1 - e], c, s, scale, Sv, Dv);
            store_entry(spec, e * T, Sv, Dv);
        }
        // bins 0 and L/2: S0 = Re Z[0], Dl0 = Im Z[0], H[L/2] = conj Z[L/2]
        const float2 z0 = v[0], zh = v[H];
        store_entry(spec, H * T, make_float2(z0.x * scale, zh.x * scale),
                    make_float2(z0.y * scale, -zh.y * scale));
#pragma unroll
        for (int e = H + 1; e < RL; ++e) {
            const float2 r = out_step_root<RL>(e);
            entry_from_real(v[e], v[RL - e], r.x, -r.y, scale, Sv, Dv);
            store_entry(spec, e * T, Sv, Dv);
        }
    }
}

// Bin k of single-channel entry (tau, e); its mirror is L - k.  Entry
// (0, RL/2) holds bins 0 and L/2 instead.
__host__ __device__ inline int64_t real_entry_bin(int64_t L, int64_t T, int64_t tau, int64_t e)
{
    const int64_t RL = L / (2 * T);
    if (tau == 0) return e < RL / 2 ? T + e * 2 * T : e * 2 * T;
    return tau + e * 2 * T;
}

// Bin (<= L/2) of entry (tau, e) of a length-L transform; entry (0, RL/2)
// holds bins 0 and L/2 instead.
__host__ __device__ inline int64_t entry_bin(int64_t L, int64_t T, int64_t tau, int64_t e)
{
    const int64_t RL = L / (2 * T);
    if (tau == 0) return e < RL / 2 ? T + e * 2 * T : (RL - e) * 2 * T;
    return e < RL / 2 ? tau + e * 2 * T : (2 * T - tau) + (RL - 1 - e) * 2 * T;
}

}  // namespace hy
