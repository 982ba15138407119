// plan.cpp -- argument validation, path choice and byte layouts.  Pure host
// code: no HIP runtime call is made here, so plans can be created and
// inspected on a machine without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>

#include "plan.h"

namespace hy {

namespace {
thread_local std::string g_last_error;

bool is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }
int64_t next_pow2(int64_t n)
{
    int64_t m = 1;
    while (m < n) m <<= 1;
    return m;
}
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

void add_segment(Plan& p, int64_t& off, int64_t ns, int64_t radix)
{
    TwSegment& s = p.seg[p.nseg++];
    s.off = off;
    s.ns = (int32_t)ns;
    s.radix = (int32_t)radix;
    off += (radix - 1) * ns;
}
// The four tables of one transform length: forward middle pass, forward last
// pass, inverse middle pass, inverse last pass.
void add_transform_segments(Plan& p, int64_t& off, int64_t L)
{
    const int l = (int)L;
    add_segment(p, off, lds1d_r0(l), lds1d_r1(l));
    add_segment(p, off, L / lds1d_rl(l), lds1d_rl(l));
    add_segment(p, off, lds1d_rl(l), lds1d_r1(l));
    add_segment(p, off, L / lds1d_r0(l), lds1d_r0(l));
}
}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }
hyena_status fail(hyena_status s, const std::string& msg)
{
    g_last_error = msg;
    log_msg("error %d: %s", (int)s, msg.c_str());
    return s;
}
const char* last_error_text() { return g_last_error.c_str(); }

bool log_on()
{
    static const bool on = [] {
        const char* v = getenv("HYENA_LOG");
        return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
    }();
    return on;
}

void log_msg(const char* fmt, ...)
{
    if (!log_on()) return;
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    fprintf(stderr, "[hyena] %s\n", buf);
    fflush(stderr);
}

// ---------------------------------------------------------------------------
// workspace record
// ---------------------------------------------------------------------------
namespace {
struct WsEntry {
    size_t bytes;
    uint64_t token;
};
std::mutex g_ws_mu;
std::map<uintptr_t, WsEntry> g_ws;  // first byte -> entry
std::atomic<uint64_t> g_next_token{1};

// Drop every entry overlapping [a, a + n) except the one at `keep` made by
// `keep_token` (keep = 0: none kept).  Caller holds g_ws_mu.
void drop_overlapping(uintptr_t a, size_t n, uintptr_t keep, uint64_t keep_token)
{
    if (n == 0) n = 1;
    // entries start below a + n; walk back from there while they may reach a
    auto it = g_ws.lower_bound(a + n);
    while (it != g_ws.begin()) {
        --it;
        const uintptr_t s = it->first;
        const size_t m = it->second.bytes ? it->second.bytes : 1;
        if (s + m <= a) {
            // entries further down start lower; one of them could still be
            // long enough to reach a, so keep walking (records are few)
            continue;
        }
        if (s == keep && it->second.token == keep_token) continue;
        log_msg("workspace record %p (plan %llu) dropped: overlapped by [%p, +%zu)", (void*)s,
                (unsigned long long)it->second.token, (void*)a, n);
        it = g_ws.erase(it);
    }
}
}  // namespace

void ws_record_init(const void* ws, size_t bytes, uint64_t token)
{
    std::lock_guard<std::mutex> lock(g_ws_mu);
    const uintptr_t a = (uintptr_t)ws;
    drop_overlapping(a, bytes, 0, 0);
    g_ws[a] = WsEntry{bytes, token};
    log_msg("workspace %p (+%zu bytes) holds the tables of plan %llu", ws, bytes,
            (unsigned long long)token);
}

bool ws_record_use(const void* ws, size_t bytes, uint64_t token)
{
    std::lock_guard<std::mutex> lock(g_ws_mu);
    const uintptr_t a = (uintptr_t)ws;
    auto it = g_ws.find(a);
    if (it == g_ws.end() || it->second.token != token) return false;
    drop_overlapping(a, bytes, a, token);
    return true;
}

bool ws_record_release(const void* ws, uint64_t token)
{
    std::lock_guard<std::mutex> lock(g_ws_mu);
    auto it = g_ws.find((uintptr_t)ws);
    if (it == g_ws.end() || it->second.token != token) return false;
    g_ws.erase(it);
    log_msg("workspace %p released by plan %llu", ws, (unsigned long long)token);
    return true;
}

void ws_record_drop(uint64_t token)
{
    std::lock_guard<std::mutex> lock(g_ws_mu);
    for (auto it = g_ws.begin(); it != g_ws.end();) {
        if (it->second.token == token) it = g_ws.erase(it);
        else ++it;
    }
}

size_t ws_record_count()
{
    std::lock_guard<std::mutex> lock(g_ws_mu);
    return g_ws.size();
}

// Four-step split of a 1D transform of length M into columns of length M1
// (sample t = M2 * n1 + n2) and rows of length M2.
static void fourstep_split(int64_t M, int64_t& M1, int64_t& M2)
{
    // columns carry the zero-padded half, rows are kept short enough for one
    // workgroup to hold a mirrored pair of them in LDS; columns at most 1024
    // (they move the activations), rows at most 4096
    M1 = 512;
    while (M1 > 32 && M / M1 < 32) M1 >>= 1;
    if (M / M1 > 1024) M1 = M / 1024 < 1024 ? M / 1024 : 1024;
    M2 = M / M1;
}

hyena_status plan_build(Plan& p, int64_t B, int64_t N, int64_t d, int32_t order,
                        const int64_t* dims, int32_t ndims, int32_t io_dtype,
                        int32_t spec_dtype, int32_t path, int32_t flags)
{
    if (flags & ~HYENA_FLAG_CIRCULAR) return fail(HYENA_ERR_UNSUPPORTED, "unknown flags");
    p.circular = (flags & HYENA_FLAG_CIRCULAR) ? 1 : 0;
    if (B < 1) return fail(HYENA_ERR_INVALID_ARGUMENT, "B must be >= 1");
    if (d < 1) return fail(HYENA_ERR_INVALID_ARGUMENT, "d must be >= 1");
    if (N < 1) return fail(HYENA_ERR_INVALID_ARGUMENT, "N must be >= 1");
    if (dims == nullptr) return fail(HYENA_ERR_INVALID_ARGUMENT, "dims is NULL");
    if (order < 1 || order > kMaxOrder)
        return fail(HYENA_ERR_UNSUPPORTED, "order must be in 1..8");
    if (io_dtype != HYENA_F32 && io_dtype != HYENA_BF16 && io_dtype != HYENA_F16)
        return fail(HYENA_ERR_UNSUPPORTED, "unknown io_dtype");
    if (spec_dtype != HYENA_F32 && spec_dtype != HYENA_BF16)
        return fail(HYENA_ERR_UNSUPPORTED, "unknown spectrum_dtype");
    if (io_dtype != HYENA_BF16 && spec_dtype == HYENA_BF16)
        return fail(HYENA_ERR_UNSUPPORTED, "a bfloat16 spectrum needs bfloat16 io");
    if (path < HYENA_PATH_AUTO || path > HYENA_PATH_ROWCOL3D)
        return fail(HYENA_ERR_UNSUPPORTED, "unknown path");
    if (ndims < 1 || ndims > 3) return fail(HYENA_ERR_UNSUPPORTED, "ndims must be 1, 2 or 3");
    // per-row element offsets are 32-bit inside the kernels
    if ((double)N * (double)d * 4.0 >= 2147483648.0)
        return fail(HYENA_ERR_UNSUPPORTED, "N * d * 4 must stay below 2^31 bytes");

    p.token = g_next_token.fetch_add(1);
    p.B = B;
    p.N = N;
    p.d = d;
    p.order = order;
    p.ndims = ndims;
    p.io_dtype = io_dtype;
    p.spec_dtype = spec_dtype;
    p.npairs = (d + 1) / 2;
    p.spec_entry_bytes = spec_dtype == HYENA_F32 ? 16 : 8;
    p.nseg = 0;
    int64_t off = 0;

    if (ndims == 1) {
        if (dims[0] != N) return fail(HYENA_ERR_INVALID_ARGUMENT, "dims[0] must equal N");
        if (N < 4 || N > kFourStepMaxM / 2)
            return fail(HYENA_ERR_UNSUPPORTED, "1D sequence length must be in 4..2097152");
        p.M = next_pow2(2 * N);
        if (p.circular) {
            // periodic boundary: the transform is the sequence itself (a power
            // of two), on the single-channel path up to 16384 and on the
            // four-step path (columns of 512 or 1024) from 32768 on
            if (!is_pow2(N) || N < 16)
                return fail(HYENA_ERR_UNSUPPORTED,
                            "periodic boundary needs N a power of two in 16..2097152");
            const int32_t want = N <= kLdsMaxM ? HYENA_PATH_LDS1D : HYENA_PATH_FOURSTEP1D;
            if (path != HYENA_PATH_AUTO && path != want)
                return fail(HYENA_ERR_UNSUPPORTED,
                            "periodic boundary: N up to 16384 runs on the LDS1D path, longer "
                            "sequences on the FOURSTEP1D path");
            p.M = N;
            path = want;
        }
        if (path == HYENA_PATH_AUTO) path = p.M <= kLdsMaxM ? HYENA_PATH_LDS1D : HYENA_PATH_FOURSTEP1D;
        if (path == HYENA_PATH_ROWCOL2D || path == HYENA_PATH_ROWCOL3D)
            return fail(HYENA_ERR_UNSUPPORTED, "the row-column paths need ndims = 2 or 3");
        if (path == HYENA_PATH_LDS1D && p.M > kLdsMaxM)
            return fail(HYENA_ERR_UNSUPPORTED, "LDS1D path holds transforms up to 16384 points");
        if (path == HYENA_PATH_FOURSTEP1D && p.M < 1024)
            return fail(HYENA_ERR_UNSUPPORTED, "FOURSTEP1D needs a transform of >= 1024 points");
        p.path = path;
        p.spec_entries_per_pair = p.M / 2;
        if (path == HYENA_PATH_LDS1D) {
            // N = M/2 (a power of two): single-channel kernels, one real
            // channel per length-M/2 complex transform, on activations staged
            // channel-major in the workspace (half the LDS of a channel pair,
            // so twice the workgroups per CU; measured faster at 2K and 8K).
            // Other N: channel-pair kernels reading channels-last rows per lane.
            const bool real = (2 * N == p.M || p.circular) && p.M >= 16;
            p.lds_io = real ? 3 : 0;
            const int64_t L = real ? p.M / 2 : p.M;
            p.R0 = lds1d_r0((int)L);
            p.R1 = lds1d_r1((int)L);
            p.RL = lds1d_rl((int)L);
            add_transform_segments(p, off, L);
            // exp(-2 pi i k / M), k < M/2: the bin twiddles of the
            // single-channel product
            add_segment(p, off, p.M / 2, 2);
        } else {
            fourstep_split(p.M, p.M1, p.M2);
            // outer (column, length M1) and inner (row, length M2) transforms use
            // the single-workgroup radix plan of their own length; then the
            // inter-step twiddle W_M^{n2 k1}, stored [n2 - 1][k1]
            add_transform_segments(p, off, p.M1);
            add_transform_segments(p, off, p.M2);
            add_segment(p, off, p.M1, p.M2);
        }
    } else if (ndims == 2) {
        if (p.circular) return fail(HYENA_ERR_UNSUPPORTED, "periodic boundary: ndims = 1 only");
        const int64_t X = dims[0], Y = dims[1];
        if (!is_pow2(X) || !is_pow2(Y) || X < 4 || Y < 4 || X > 1024 || Y > 1024)
            return fail(HYENA_ERR_UNSUPPORTED, "2D grid sides must be powers of two in 4..1024");
        if (X * Y != N) return fail(HYENA_ERR_INVALID_ARGUMENT, "N must equal X * Y");
        if (path == HYENA_PATH_AUTO) path = HYENA_PATH_ROWCOL2D;
        if (path != HYENA_PATH_ROWCOL2D)
            return fail(HYENA_ERR_UNSUPPORTED, "2D grids use the ROWCOL2D path");
        p.path = path;
        p.X = X;
        p.Y = Y;
        p.P1 = 2 * X;
        p.P2 = 2 * Y;
        p.spec_entries_per_pair = p.P1 * p.P2 / 2;
        // outer transforms run along q (length P2), inner along p (length P1)
        add_transform_segments(p, off, p.P2);
        add_transform_segments(p, off, p.P1);
    } else {
        if (p.circular) return fail(HYENA_ERR_UNSUPPORTED, "periodic boundary: ndims = 1 only");
        const int64_t X = dims[0], Y = dims[1], Z = dims[2];
        if (!is_pow2(X) || !is_pow2(Y) || !is_pow2(Z) || X < 4 || Y < 4 || Z < 4 || X > 256 ||
            Y > 256 || Z > 256)
            return fail(HYENA_ERR_UNSUPPORTED, "3D grid sides must be powers of two in 4..256");
        if (X * Y * Z > (1 << 20))
            return fail(HYENA_ERR_UNSUPPORTED, "3D grids hold at most 2^20 points");
        if (X * Y * Z != N) return fail(HYENA_ERR_INVALID_ARGUMENT, "N must equal X * Y * Z");
        if (path == HYENA_PATH_AUTO) path = HYENA_PATH_ROWCOL3D;
        if (path != HYENA_PATH_ROWCOL3D)
            return fail(HYENA_ERR_UNSUPPORTED, "3D grids use the ROWCOL3D path");
        p.path = path;
        p.X = X;
        p.Y = Y;
        p.Z = Z;
        p.P1 = 2 * X;
        p.P2 = 2 * Y;
        p.P3 = 2 * Z;
        p.spec_entries_per_pair = p.P1 * p.P2 * p.P3 / 2;
        // outer transforms along z (length P3, on the activations), inner
        // along x (length P1, with the product), and the middle pass along y
        add_transform_segments(p, off, p.P3);
        add_transform_segments(p, off, p.P1);
        add_transform_segments(p, off, p.P2);
    }

    p.tw_elems = off;
    p.tw_bytes = align_up((size_t)off * 8, 256);
    p.spectrum_bytes = (size_t)p.order * (size_t)p.npairs * (size_t)p.spec_entries_per_pair *
                       p.spec_entry_bytes;
    if (p.path == HYENA_PATH_LDS1D && p.lds_io == 3)  // M/4 entries per channel
        p.spectrum_bytes = (size_t)p.order * (size_t)d * (size_t)(p.M / 4) * p.spec_entry_bytes;

    // intermediate spectra of the multi-pass paths: one complex64 value per
    // transform point of the zero-padded half that is kept, for a chunk of
    // channel pairs that is walked through all passes before the next chunk
    p.inter_offset = p.tw_bytes;
    p.inter_bytes = 0;
    p.chunk_pairs = 0;
    if (p.path == HYENA_PATH_FOURSTEP1D || p.path == HYENA_PATH_ROWCOL2D) {
        // per channel pair: the forward chain keeps F[o][a] for the live inner
        // positions; the filter spectrum needs every inner position
        const int64_t fwd_pair = p.path == HYENA_PATH_FOURSTEP1D ? p.M * 8 : p.X * p.P2 * 8;
        const int64_t spec_pair = p.path == HYENA_PATH_FOURSTEP1D ? p.M * 8 : p.P1 * p.P2 * 8;
        // the chunk's intermediate near kChunkBytes (a measured size: smaller
        // chunks, which the last-level cache could hold, were no faster);
        // whole groups of 16 pairs
        int64_t chunk = kChunkBytes / fwd_pair;
        chunk = chunk / 16 * 16;
        if (chunk < 16) chunk = 16;
        const int64_t total_slots = p.B * ((p.npairs + 15) / 16) * 16;
        if (chunk > total_slots) chunk = total_slots;
        p.chunk_pairs = chunk;
        p.fwd_pair_bytes = fwd_pair;
        p.spec_pair_bytes = spec_pair;
        const int64_t need = chunk * (fwd_pair > spec_pair ? fwd_pair : spec_pair);
        p.inter_bytes = align_up((size_t)need, 256);
    }
    if (p.path == HYENA_PATH_ROWCOL3D) {
        // per channel pair: F1 after the z transforms ([x][y][kz]; the chain
        // keeps x < X, y < Y, the spectrum every x, y) and F2 after the y
        // transforms ([x][ky][kz])
        const int64_t fwd1 = p.X * p.Y * p.P3 * 8, fwd2 = p.X * p.P2 * p.P3 * 8;
        const int64_t spec1 = p.P1 * p.P2 * p.P3 * 8, spec2 = spec1;
        int64_t chunk = kChunkBytes / (fwd1 + fwd2);
        chunk = chunk / 16 * 16;
        if (chunk < 16) chunk = 16;
        const int64_t total_slots = p.B * ((p.npairs + 15) / 16) * 16;
        if (chunk > total_slots) chunk = total_slots;
        p.chunk_pairs = chunk;
        p.fwd_pair_bytes = fwd1;
        p.fwd_pair_bytes2 = fwd2;
        p.spec_pair_bytes = spec1;
        p.spec_pair_bytes2 = spec2;
        const size_t r1 = align_up((size_t)(chunk * (fwd1 > spec1 ? fwd1 : spec1)), 256);
        const size_t r2 = align_up((size_t)(chunk * (fwd2 > spec2 ? fwd2 : spec2)), 256);
        p.inter2_offset = p.inter_offset + r1;
        p.inter_bytes = r1 + r2;
    }
    if (p.path == HYENA_PATH_LDS1D && p.lds_io == 3) {
        // u, every gate and y, staged channel-major
        p.stage_offset = p.inter_offset + p.inter_bytes;
        p.stage_bytes = align_up((size_t)(p.order + 2) * (size_t)B * (size_t)N * (size_t)d *
                                     (io_dtype == HYENA_F32 ? 4u : 2u), 256);
    }
    size_t inter_end = p.inter_offset + p.inter_bytes;
    p.fwd_offset[0] = p.inter_offset;
    p.fwd2_offset[0] = p.inter2_offset;
    if (p.chunk_pairs > 0) {
        const int64_t total_slots = p.B * ((p.npairs + 15) / 16) * 16;
        if (total_slots > p.chunk_pairs) {
            // the second copy holds the chain's intermediates only
            p.inter_copies = 2;
            p.fwd_offset[1] = inter_end;
            const size_t f1 = align_up((size_t)(p.chunk_pairs * p.fwd_pair_bytes), 256);
            p.fwd2_offset[1] = p.fwd_offset[1] + f1;
            inter_end = p.fwd2_offset[1] +
                        align_up((size_t)(p.chunk_pairs * p.fwd_pair_bytes2), 256);
        }
    }
    p.workspace_bytes = inter_end + p.stage_bytes;
    static const char* kPathName[] = {"AUTO", "LDS1D", "FOURSTEP1D", "ROWCOL2D", "ROWCOL3D"};
    log_msg("plan %llu: B=%lld N=%lld d=%lld order=%d ndims=%d io=%d spectrum=%d circular=%d -> "
            "path %s, M=%lld (M1=%lld M2=%lld P=%lldx%lldx%lld), spectrum %zu B, workspace %zu B, "
            "chunk %lld pair slots, %d intermediate cop%s",
            (unsigned long long)p.token, (long long)B, (long long)N, (long long)d, order, ndims,
            io_dtype, spec_dtype, p.circular, kPathName[p.path], (long long)p.M, (long long)p.M1,
            (long long)p.M2, (long long)p.P1, (long long)p.P2, (long long)p.P3, p.spectrum_bytes,
            p.workspace_bytes, (long long)p.chunk_pairs, p.inter_copies,
            p.inter_copies == 1 ? "y" : "ies");
    return HYENA_OK;
}

}  // namespace hy
