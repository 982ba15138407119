// plan.h -- host-side plan shared by the C-ABI layer and the kernel launchers.
//
// The plan is plain data: shape, dtypes, the resolved path, the radix
// decomposition of each transform and the byte layout of the spectrum and of
// the workspace.  Building it needs no GPU (plan.cpp has no HIP calls).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "hyena.h"

namespace hy {

constexpr int kMaxOrder = 8;
constexpr int kMaxTwSegments = 12;
constexpr int64_t kLdsMaxM = 16384;       // largest transform held in one workgroup's LDS
constexpr int64_t kFourStepMaxM = 1 << 22;  // largest 1D transform (N = 2097152): 1024 x 4096
// Multi-pass paths walk the channel pairs in chunks whose intermediate is
// about this large (at least 16 pairs).  Chains of two or more chunks run
// them on two streams, so two chunks' intermediates are live at a time:
// 64 MiB each (128 MiB together) measured fastest at 64K tokens (32, 48, 64,
// 80, 96, 128, 192, 256 MiB: 1245, 1206, 1202-1212, 1251-1258, 1240-1256,
// 1285-1294, 1270-1304, 1302-1304 us) and on the 256 x 256 grid (523-530
// us against 545-557 at 96 and 192 MiB).
#ifndef HY_CHUNK_MIB
#define HY_CHUNK_MIB 64
#endif
constexpr int64_t kChunkBytes = (int64_t)HY_CHUNK_MIB << 20;

// Radix plan of the single-workgroup transform of length M (8 <= M <= 16384):
// 32 complex values per thread (M >= 64), forward passes R0, R1, RL with
// RL = 16 so that the last pass gives each thread two butterflies.
constexpr int lds1d_pts(int M) { return M >= 64 ? 32 : M; }
constexpr int lds1d_rl(int M) { return lds1d_pts(M) / 2; }
constexpr int lds1d_rest(int M) { return M / lds1d_rl(M); }
constexpr int lds1d_r0(int M)
{
    return lds1d_rest(M) <= 32 ? lds1d_rest(M) : lds1d_rest(M) <= 512 ? lds1d_rest(M) / 16 : 32;
}
constexpr int lds1d_r1(int M)
{
    return lds1d_rest(M) <= 32 ? 1 : lds1d_rest(M) <= 512 ? 16 : 32;
}

// One twiddle table, lane-coalesced: tw[off + (r - 1) * ns + k] =
// exp(-2 pi i r k / (ns * radix)), r = 1..radix-1, k = 0..ns-1.  Neighbouring
// lanes hold neighbouring k, so each load instruction reads one contiguous run.
struct TwSegment {
    int64_t off;    // in float2 elements from the workspace base
    int32_t ns;
    int32_t radix;
};

struct Plan {
    // shape
    int64_t B = 0, N = 0, d = 0;
    int32_t order = 0;
    int32_t ndims = 1;
    int64_t X = 0, Y = 0, Z = 0;  // 2D / 3D grid sides
    int32_t io_dtype = HYENA_F32, spec_dtype = HYENA_F32;
    int32_t path = HYENA_PATH_AUTO;
    int32_t circular = 0;  // periodic boundary: transform length N, no padding

    int64_t M = 0;       // 1D transform length (power of two >= 2N)
    int64_t npairs = 0;  // channel pairs (two real channels per complex transform)

    // LDS1D: forward radices R0, R1 (1 if absent), RL of the transform the
    // kernels run (length M, or M/2 for the single-channel form); the inverse
    // runs them reversed.
    int32_t R0 = 0, R1 = 1, RL = 0;
    // LDS1D form: 0 channel pairs on channels-last rows, 3 single channels on
    // activations staged channel-major in the workspace (N = M/2)
    int32_t lds_io = 0;
    size_t stage_offset = 0, stage_bytes = 0;  // channel-major staging in the workspace

    // FOURSTEP1D: M = M1 * M2; columns of length M1 (time index t = M2 n1 + n2),
    // rows of length M2.  ROWCOL2D: P1 = 2X (columns), P2 = 2Y (rows).
    // ROWCOL3D: P1 = 2X, P2 = 2Y, P3 = 2Z.
    int64_t M1 = 0, M2 = 0;
    int64_t P1 = 0, P2 = 0, P3 = 0;
    int64_t chunk_pairs = 0;      // channel-pair slots per pass over the intermediate buffer
    int64_t fwd_pair_bytes = 0;   // intermediate bytes per pair slot, forward chain
    int64_t spec_pair_bytes = 0;  // intermediate bytes per pair slot, filter spectrum
    // ROWCOL3D: a second intermediate (after the transform along y) per pair
    // slot, placed after the first one's chunk in the workspace
    int64_t fwd_pair_bytes2 = 0, spec_pair_bytes2 = 0;
    size_t inter2_offset = 0;

    // twiddle tables
    TwSegment seg[kMaxTwSegments];
    int32_t nseg = 0;
    int64_t tw_elems = 0;  // float2 elements

    // byte layout
    size_t spec_entry_bytes = 0;  // one (P, Q) entry: 16 (f32) or 8 (bf16)
    int64_t spec_entries_per_pair = 0;
    size_t spectrum_bytes = 0;
    size_t tw_bytes = 0;
    size_t inter_offset = 0;  // workspace offset of the intermediate buffer
    size_t inter_bytes = 0;   // its size (F, and F2 on 3D grids; chain and spectrum)
    // copies of the intermediate for the forward chain: 2 when the chain
    // walks two or more chunks, which then alternate between the caller's
    // stream and a second one (copy i % 2 for chunk i), so passes of
    // neighbouring chunks overlap.  Copy 0 is the buffer above; copy 1, sized
    // for the chain alone, follows it.  fwd_offset / fwd2_offset: F (F1) and
    // F2 of each copy.
    int32_t inter_copies = 1;
    size_t fwd_offset[2] = {0, 0};
    size_t fwd2_offset[2] = {0, 0};
    size_t workspace_bytes = 0;

    // identifies the plan in the workspace record (unique in the process)
    uint64_t token = 0;
};

// Implemented in plan.cpp (pure host code).
hyena_status plan_build(Plan& p, int64_t B, int64_t N, int64_t d, int32_t order,
                        const int64_t* dims, int32_t ndims, int32_t io_dtype,
                        int32_t spec_dtype, int32_t path, int32_t flags);
void set_error(const std::string& msg);
hyena_status fail(hyena_status s, const std::string& msg);

// HYENA_LOG: with the environment variable HYENA_LOG set to a non-empty value
// other than "0", the host side reports plan decisions, workspace records and
// every kernel launch on stderr.  Read once per process.
bool log_on();
void log_msg(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

// Process-wide record of which plan's twiddle tables each workspace holds
// (implemented in plan.cpp, pure host code, internally locked).  A workspace
// is recorded by its first byte and the byte count the plan uses.
//   ws_record_init:    `token`'s tables were written at ws; every record whose
//                      bytes overlap [ws, ws + bytes) is dropped first (the
//                      write clobbered them).
//   ws_record_use:     true when ws holds `token`'s tables; then every other
//                      record overlapping [ws, ws + bytes) is dropped (the call
//                      about to run writes its intermediates there).
//   ws_record_release: drop the record of ws if `token` made it; returns
//                      whether one was dropped.
//   ws_record_drop:    drop every record of `token` (plan destroyed).
void ws_record_init(const void* ws, size_t bytes, uint64_t token);
bool ws_record_use(const void* ws, size_t bytes, uint64_t token);
bool ws_record_release(const void* ws, uint64_t token);
void ws_record_drop(uint64_t token);
size_t ws_record_count();

// api.hip: the checks and dispatch shared by hyena_forward and the
// allocation-free hyena_forward_noalloc (static_scratch.hip).
hyena_status check_forward_args(const Plan& p, const void* u, const void* const* gates,
                                const void* H, const float* D, const void* y, const void* ws);
// While one of these lives on a thread, the multi-pass chains run every
// chunk on the caller's stream and create no stream or event (for the
// allocation-free entry point).
struct SingleStreamScope {
    SingleStreamScope();
    ~SingleStreamScope();
};
hyena_status run_forward(const Plan& p, const void* u, const void* const* gates, const void* H,
                         const float* D, void* y, void* ws, void* stream);
const Plan* plan_of(hyena_plan_t plan);

// Implemented in the .hip launchers.
hyena_status launch_tw_init(const Plan& p, void* ws, void* stream);
hyena_status launch_lds1d_spectrum(const Plan& p, const void* h, void* H, const void* ws, void* stream);
hyena_status launch_lds1d_forward(const Plan& p, const void* u, const void* const* gates,
                                  const void* H, const float* D, void* y, const void* ws,
                                  void* stream);
hyena_status launch_lds1d_export(const Plan& p, const void* H, void* out, void* stream);

hyena_status launch_fourstep_spectrum(const Plan& p, const void* h, void* H, void* ws, void* stream);
hyena_status launch_fourstep_forward(const Plan& p, const void* u, const void* const* gates,
                                     const void* H, const float* D, void* y, void* ws,
                                     void* stream);
hyena_status launch_fourstep_export(const Plan& p, const void* H, void* out, void* stream);
// taps of an implicit filter evaluated in the spectrum's first pass from its
// hidden features z2 [N][hp] (the output layer W3, b3 and the window alpha)
hyena_status launch_fourstep_spectrum_implicit(const Plan& p, const float* z2, const float* W3,
                                               const float* b3, const float* alpha, int32_t hp,
                                               int32_t hidden, void* H, void* ws, void* stream);

hyena_status launch_rowcol2d_spectrum(const Plan& p, const void* h, void* H, void* ws, void* stream);
hyena_status launch_rowcol2d_forward(const Plan& p, const void* u, const void* const* gates,
                                     const void* H, const float* D, void* y, void* ws,
                                     void* stream);
hyena_status launch_rowcol2d_export(const Plan& p, const void* H, void* out, void* stream);
hyena_status launch_rowcol2d_block(const Plan& p, const hyena_nd_mixer& m, const void* H,
                                   const float* D, void* y, void* ws, void* stream);

hyena_status launch_rowcol3d_spectrum(const Plan& p, const void* h, void* H, void* ws, void* stream);
hyena_status launch_rowcol3d_forward(const Plan& p, const void* u, const void* const* gates,
                                     const void* H, const float* D, void* y, void* ws,
                                     void* stream);
hyena_status launch_rowcol3d_export(const Plan& p, const void* H, void* out, void* stream);
hyena_status launch_rowcol3d_block(const Plan& p, const hyena_nd_mixer& m, const void* H,
                                   const float* D, void* y, void* ws, void* stream);

// implicit.hip
size_t implicit_scratch_bytes(const Plan& p, int32_t hidden);
hyena_status launch_implicit_spectrum(const Plan& p, const hyena_implicit_filter& f, void* H,
                                      void* ws, void* scratch, void* stream);

}  // namespace hy
