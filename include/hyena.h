/*
 * hyena.h -- C ABI of the MI355X (gfx950) Hyena long-convolution library.
 *
 * What it computes.  The order-N Hyena chain of "Week 11: Hyena, Long
 * Convolution, and Linear Attention", section "The Hyena operator", in the
 * order-2 form of "Hyena -- Long Convolutions Math", section "The Toeplitz
 * picture" (y = x2 . (h2 * (x1 . (h1 * v)))), with the per-channel
 * feedthrough of the FFTConv equation ([P1] section "FFTConv"):
 *
 *   z_0 = u
 *   z_n[b,t,c] = gate_n[b,t,c] * ( sum_{s=0}^{t} h_n[c,s] z_{n-1}[b,t-s,c]
 *                                  + D_n[c] z_{n-1}[b,t,c] ),   n = 1..order
 *   y = z_order
 *
 * Each convolution is evaluated through the convolution theorem on a length
 * M = (power of two >= 2N) zero-padded transform, keeping the first N
 * outputs ("Hyena -- Long Convolutions Math", sections "The convolution
 * theorem" and "Linear vs circular").  With ndims = 2 the convolution is the
 * non-causal linear 2D convolution of "How HyenaND works" (section "The
 * convolution theorem (FFT)"; worked trace with zero padding and
 * is_causal=False): taps at every signed offset (i, j), |i| <= X-1,
 * |j| <= Y-1, output kept on the input grid.  ndims = 3 is the same on an
 * X x Y x Z grid (the page's native ND transform, here on 3D grids).
 *
 * Layouts (row-major, channels last; d is the fastest axis):
 *   u, gates[n], y : [B][N][d] (ndims = 1), [B][X][Y][d] (ndims = 2) or
 *                    [B][X][Y][Z][d] (ndims = 3)
 *   h              : [order][d][N] (ndims = 1);
 *                    [order][d][2X-1][2Y-1] (ndims = 2), the tap at offset
 *                    (i, j) stored at index (i + X - 1, j + Y - 1);
 *                    [order][d][2X-1][2Y-1][2Z-1] (ndims = 3), offset
 *                    (i, j, l) at (i + X - 1, j + Y - 1, l + Z - 1)
 *   D              : float32 [order][d]
 *   H (spectrum)   : opaque, spectrum_bytes long, laid out in the order the
 *                    forward kernels consume it (see hyena_spectrum_export)
 * io_dtype applies to u, gates, y and h; spectrum_dtype to H.  All arithmetic
 * is float32; bfloat16 values are widened exactly and stored with
 * round-to-nearest-even.
 *
 * Ownership and streams.  Every device buffer is owned by the caller and must
 * stay alive until the work enqueued on the stream has finished.  The library
 * never allocates device memory; it owns only host memory inside the plan.
 * All device work is enqueued on the given hipStream_t (passed as void*; NULL
 * is the null stream) with no host synchronisation.  The workspace holds
 * twiddle tables (written by hyena_workspace_init) and, on the multi-pass
 * paths, the intermediate spectra; it must not be shared by calls that run
 * concurrently.  A multi-pass forward whose channel pairs take two or more
 * chunks of the intermediate buffer runs every other chunk on a second
 * stream of the library's, with its own copy of that buffer in the
 * workspace: the second stream waits for an event recorded on the given
 * stream when the call starts, and the given stream waits for one recorded
 * on the second when the call's work is enqueued, so everything the call
 * does stays ordered on the given stream (graph capture included).  That
 * stream and its two events are created on first use, one set per host
 * thread and device, at default priority, and held until the process ends;
 * a thread that has none yet while its stream is being captured runs all
 * chunks on the given stream.
 *
 * Errors.  Argument problems are reported before anything is enqueued and
 * leave every output untouched; hyena_last_error() then returns a
 * thread-local description.  HYENA_ERR_DEVICE reports a failed launch;
 * faults inside a kernel surface at the caller's next synchronisation.
 *
 * Thread safety.  A plan is immutable after creation; the record of
 * initialised workspaces is process-wide and internally locked; plans may be
 * shared by host threads.  The forward pass uses no atomics, so the same plan
 * and inputs give bitwise-identical y.
 *
 * Diagnostics.  With the environment variable HYENA_LOG set (to anything but
 * "" or "0") the host side reports plan decisions, workspace records, errors
 * and every kernel launch (name, grid, block, stream) on stderr.
 */
#ifndef HYENA_MI355X_H
#define HYENA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hyena_plan_s* hyena_plan_t;

typedef enum hyena_status {
    HYENA_OK = 0,
    HYENA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned/overlapping pointer, bad size */
    HYENA_ERR_UNSUPPORTED = 2,      /* shape, order, dtype or path not supported */
    HYENA_ERR_WORKSPACE = 3,        /* workspace not initialised for this plan */
    HYENA_ERR_DEVICE = 4            /* a HIP launch or query failed */
} hyena_status;

/* Storage types.  HYENA_F16 (IEEE binary16, round to nearest even on store;
 * magnitudes above 65504 become infinite) is an io_dtype only and takes a
 * float32 spectrum. */
typedef enum hyena_dtype {
    HYENA_F32 = 0,
    HYENA_BF16 = 1,
    HYENA_F16 = 2
} hyena_dtype;

/* Which kernel family runs the transform.  AUTO picks: LDS1D when ndims = 1
 * and M <= 16384, FOURSTEP1D when ndims = 1 and M > 16384, ROWCOL2D when
 * ndims = 2, ROWCOL3D when ndims = 3.  FOURSTEP1D may be forced for any
 * M >= 1024 (tests use this to check it against the single-pass kernels at
 * small N). */
typedef enum hyena_path {
    HYENA_PATH_AUTO = 0,
    HYENA_PATH_LDS1D = 1,
    HYENA_PATH_FOURSTEP1D = 2,
    HYENA_PATH_ROWCOL2D = 3,
    HYENA_PATH_ROWCOL3D = 4
} hyena_path;

/*
 * Create a plan ("Hyena -- Long Convolutions Math", sections "The
 * primitive" and "Linear vs circular": zero-padded causal convolutions;
 * "How HyenaND works", section "2. The convolution theorem (FFT)": 2D and 3D
 * grids).  B >= 1 batch rows, d >= 1 channels, 1 <= order <= 8.
 * ndims = 1: dims = {N}, 4 <= N <= 2097152 (any N; M is the power of two
 *            >= 2N; N == the N argument).  M <= 16384 runs in one workgroup
 *            per channel (pair); longer transforms take the four-step path.
 * ndims = 2: dims = {X, Y}, X and Y powers of two in [4, 1024]; N must equal
 *            X * Y (and N * d * 4 below 2^31).
 * ndims = 3: dims = {X, Y, Z}, powers of two in [4, 256], X * Y * Z <= 2^20;
 *            N must equal X * Y * Z.
 * io_dtype, spectrum_dtype: hyena_dtype values.  The path is chosen
 * automatically (HYENA_PATH_AUTO); hyena_plan_create_ex below takes a path
 * and flags.  On success *plan receives a new plan (release with
 * hyena_plan_destroy).  This call touches no GPU state.
 */
hyena_status hyena_plan_create(hyena_plan_t* plan, int64_t B, int64_t N, int64_t d,
                               int32_t order, const int64_t* dims, int32_t ndims,
                               int32_t io_dtype, int32_t spectrum_dtype);

/*
 * hyena_plan_create with a path (hyena_path value; HYENA_PATH_AUTO as
 * above) and flags.  HYENA_FLAG_CIRCULAR: periodic boundary,
 * the unpadded length-N circular convolution of "Hyena -- Long Convolutions
 * Math", section "Linear vs circular" as the operator:
 *   z_n[b,t,c] = gate_n[b,t,c] * ( sum_{s=0}^{N-1} h_n[c,s] z_{n-1}[b,(t-s) mod N,c]
 *                                  + D_n[c] z_{n-1}[b,t,c] ),
 * for ndims = 1 and N a power of two in 16..2097152 (the transform is the
 * sequence itself: LDS1D path up to 16384, FOURSTEP1D path from 32768).
 * hyena_spectrum_export then gives bins k = 0..N/2 of the unpadded length-N
 * transform.
 */
#define HYENA_FLAG_CIRCULAR 1
hyena_status hyena_plan_create_ex(hyena_plan_t* plan, int64_t B, int64_t N, int64_t d,
                                  int32_t order, const int64_t* dims, int32_t ndims,
                                  int32_t io_dtype, int32_t spectrum_dtype, int32_t path,
                                  int32_t flags);

/* Sizes in bytes of the spectrum buffer H and of the workspace (either
 * output pointer may be NULL). */
hyena_status hyena_plan_query(hyena_plan_t plan, size_t* spectrum_bytes,
                              size_t* workspace_bytes);

/* The path (hyena_path value) the plan resolved to. */
hyena_status hyena_plan_path(hyena_plan_t plan, int32_t* path);

/* Write the plan's twiddle tables into a caller-allocated workspace of at
 * least workspace_bytes (16-byte aligned).  Required once per (plan,
 * workspace) before hyena_filter_spectrum or hyena_forward use it.
 *
 * The library keeps a process-wide record of which plan's tables each
 * workspace holds, keyed by its first byte.  A call with a workspace that is
 * not recorded for its plan returns HYENA_ERR_WORKSPACE before anything is
 * enqueued.  A record is dropped by hyena_workspace_release, by
 * hyena_plan_destroy, and when another plan initialises, or runs a call on,
 * a workspace whose bytes overlap it (its tables may then be overwritten).
 * The library cannot see the caller's allocator: before a workspace is freed
 * (and its memory possibly handed out again at the same address), release it
 * or destroy the plan; using an address whose record outlived its memory is
 * undefined and may give wrong results. */
hyena_status hyena_workspace_init(hyena_plan_t plan, void* workspace, void* stream);

/* Drop the record that `workspace` holds this plan's tables (no GPU work;
 * HYENA_OK also when there was none).  Call before freeing a workspace that
 * the plan will not use again. */
hyena_status hyena_workspace_release(hyena_plan_t plan, void* workspace);

/*
 * Filter spectrum ("Hyena -- Long Convolutions Math", section "The
 * convolution theorem": the transform of h is the filter's transfer
 * function).  Reads h (io_dtype, layout above) and writes H
 * (spectrum_bytes, spectrum_dtype) in the forward kernels' native order with
 * the 1/M inverse scale folded in.  D is not part of H; it is applied by
 * hyena_forward.  H stays valid for any call with a plan of the same shape
 * and dtypes.
 */
hyena_status hyena_filter_spectrum(hyena_plan_t plan, const void* h, void* H,
                                   void* workspace, void* stream);

/*
 * Forward chain.  u: input (io_dtype).  gates: host array of `order` device
 * pointers (io_dtype), gate n applied after convolution n.  H: spectrum from
 * hyena_filter_spectrum.  D: float32 [order][d] feedthrough.  y: output
 * (io_dtype); y must not overlap u, any gate, H, D or the workspace.  All
 * device pointers 16-byte aligned.
 */
hyena_status hyena_forward(hyena_plan_t plan, const void* u, const void* const* gates,
                           const void* H, const float* D, void* y, void* workspace,
                           void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * hyena_forward with the workspace taken from a fixed device array inside the
 * library (HYENA_NOALLOC_SCRATCH_BYTES per GPU, held from its first use on
 * that GPU until the process ends) instead of a caller buffer.  The call
 * allocates nothing: the caller still passes u, the gates, H, D and y, as for
 * hyena_forward.  It writes the plan's twiddle tables into the array itself
 * when they are not already there, so no hyena_workspace_init is needed.
 * Plans whose workspace_bytes exceed HYENA_NOALLOC_SCRATCH_BYTES are refused
 * with HYENA_ERR_UNSUPPORTED (the single-workgroup paths of the 2K and 8K
 * width-768 workloads fit; the multi-pass paths' chunked intermediates
 * usually do not).  The array is shared by every call on a GPU and keeps the
 * last call's contents, so calls that overlap on one GPU (different streams,
 * or different host threads) race and must be serialised by the caller.
 * The kernels and results are those of hyena_forward.
 */
#define HYENA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
hyena_status hyena_forward_noalloc(hyena_plan_t plan, const void* u, const void* const* gates,
                                   const void* H, const float* D, void* y, void* stream);

/*
 * HyenaND mixer ("How HyenaND works", section "Putting it together: the
 * HyenaND operator"), for ndims = 2 or 3 plans of order 1: the depthwise
 * short convolution (zero padding; 3x3 taps short_w [3][d][3][3] on 2D
 * grids, 3x3x3 taps short_w [3][d][3][3][3] on 3D grids, for q, k, v; biases
 * short_b [3][d] or NULL; float32), the inner gate, the long convolution and
 * the outer gate, in the passes of the grid transform:
 *   qs, ks, vs = shortconv(q), shortconv(k), shortconv(v)
 *   z = qs . SiLU(ks),   y = SiLU(vs) . (K * z + D z),   SiLU(x) = x / (1 + e^-x)
 * q, k, v, y: [B][X][Y][d] or [B][X][Y][Z][d] in the plan's io dtype; y must
 * not overlap q, k, v, H, D or the workspace.  The projections producing
 * q, k, v and the norms around the mixer are the caller's.
 */
typedef struct hyena_nd_mixer {
    const void* q;
    const void* k;
    const void* v;
    const float* short_w;
    const float* short_b;
} hyena_nd_mixer;

hyena_status hyena_nd_mixer_forward(hyena_plan_t plan, const hyena_nd_mixer* m, const void* H,
                                    const float* D, void* y, void* workspace, void* stream);

/*
 * Implicit filters ("Hyena -- Long Convolutions Math", sections "Implicit
 * filters: an MLP over positions" and "The decay window"): instead of taps,
 * the caller passes a small sine MLP shared over positions, and
 *   h_n[c, t] = exp(-alpha[n][c] t) * FFN(gamma(t))[n d + c],  t = 0..N-1,
 *   gamma(t)  = [t/N, cos(2 pi t/N), sin(2 pi t/N), ..., cos(2 pi K t/N),
 *                sin(2 pi K t/N)]                    (m = 2K + 1 features)
 *   z1 = sin(omega (W1 gamma + b1)),  z2 = sin(omega (W2 z1 + b2)),
 *   FFN(gamma) = W3 z2 + b3.
 * All weights are float32 device arrays, row-major: W1 [H][m], b1 [H],
 * W2 [H][H], b2 [H], W3 [order d][H], b3 [order d], alpha [order][d].
 * 0 <= K <= 64, 1 <= H <= 256.  Only ndims = 1 plans.
 */
typedef struct hyena_implicit_filter {
    int32_t n_freqs; /* K */
    int32_t hidden;  /* H */
    float omega;
    const float* W1;
    const float* b1;
    const float* W2;
    const float* b2;
    const float* W3;
    const float* b3;
    const float* alpha;
} hyena_implicit_filter;

/* Bytes of the caller-owned scratch buffer hyena_filter_spectrum_implicit
 * needs for this plan and hidden width: the hidden features of every
 * position (float32, width rounded up to 16).  The taps themselves are never
 * stored. */
hyena_status hyena_implicit_scratch_bytes(hyena_plan_t plan, int32_t hidden, size_t* bytes);

/*
 * hyena_filter_spectrum with the taps generated from `f` on the device: the
 * hidden features z2 of every position go to `scratch`; the spectrum kernels
 * then evaluate each tap, window . (W3 z2 + b3), in registers where their
 * forward transform needs it, so the taps exist neither in the caller's
 * memory nor in the library's.
 * scratch: device buffer of hyena_implicit_scratch_bytes, 16-byte aligned,
 * not shared with concurrently running calls.  `f` is read on the host
 * during the call; the arrays it points to must stay alive until the stream
 * work completes.
 */
hyena_status hyena_filter_spectrum_implicit(hyena_plan_t plan, const hyena_implicit_filter* f,
                                            void* H, void* workspace, void* scratch,
                                            void* stream);

/*
 * Test/inspection helper: expand H into natural-order transfer functions,
 * complex64 (re, im) pairs, unscaled (the plain DFT of the zero-padded
 * filter).  ndims = 1: [order][d][M/2 + 1] bins k = 0..M/2.
 * ndims = 2: [order][d][P1][P2/2 + 1] with P1 = 2X, P2 = 2Y.
 * ndims = 3: [order][d][P1][P2][P3/2 + 1] with P3 = 2Z.
 */
hyena_status hyena_spectrum_export(hyena_plan_t plan, const void* H, void* natural,
                                   void* stream);

/*
 * Launch timing, a profiling aid that computes nothing.  After
 * hyena_timing_begin(max_launches), every kernel that a hyena_* call made on
 * this host thread enqueues is bracketed by two HIP timing events recorded on
 * that call's stream, for the first max_launches launches (later launches run
 * unrecorded and are counted as dropped).  The events are created by begin on
 * the device current at that time; use the same device until the end.
 *
 * hyena_timing_end(&n_kernels, &dropped) stops recording, waits for the
 * recorded events and groups the launch durations by kernel;
 * hyena_timing_kernel(i, ...) reads group i (0 <= i < n_kernels): the kernel's
 * name as the runtime's kernel trace prints it, without the leading return
 * type and argument list (for example "hy::hyena_lds1d_forward<16384,
 * unsigned short, unsigned short, 2>"), its launches, and the total, shortest
 * and longest durations in milliseconds.  The name stays valid until the next
 * begin or release.  hyena_timing_release() frees the events.  State is
 * thread-local; the recorded events add one marker to the stream before and
 * after each launch.
 */
hyena_status hyena_timing_begin(int32_t max_launches);
hyena_status hyena_timing_end(int32_t* n_kernels, int64_t* dropped);
hyena_status hyena_timing_kernel(int32_t i, const char** name, int64_t* launches,
                                 double* total_ms, double* min_ms, double* max_ms);
hyena_status hyena_timing_release(void);

/* Release a plan (NULL is accepted). */
hyena_status hyena_plan_destroy(hyena_plan_t plan);

/* Static text for a status code. */
const char* hyena_status_string(hyena_status status);

/* Thread-local text describing the last error raised on this thread. */
const char* hyena_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HYENA_MI355X_H */
