"""The C-ABI library: it loads, exports every symbol include/hyena.h
declares, and its host-side validation returns the documented status codes
(no GPU work is started by any of these calls)."""
import ctypes
import os
import re

import pytest

from long_convolution_sequence_rfft_amd import hyena

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "hyena.h")).read()
    return sorted(set(re.findall(r"\b(hyena_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = hyena.load()
    names = _header_functions()
    assert set(names) == set(hyena.EXPORTED_SYMBOLS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    assert hyena.hyena_status_string(0) == "HYENA_OK"
    assert hyena.hyena_status_string(3) == "HYENA_ERR_WORKSPACE"
    assert hyena.hyena_status_string(99) == "HYENA_ERR_UNKNOWN"


@pytest.mark.parametrize("args,code", [
    (dict(B=0, N=8, d=2, order=1, dims=[8]), hyena.HYENA_ERR_INVALID_ARGUMENT),
    (dict(B=1, N=8, d=0, order=1, dims=[8]), hyena.HYENA_ERR_INVALID_ARGUMENT),
    (dict(B=1, N=8, d=2, order=0, dims=[8]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=8, d=2, order=9, dims=[8]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=8, d=2, order=1, dims=[4]), hyena.HYENA_ERR_INVALID_ARGUMENT),
    (dict(B=1, N=2, d=2, order=1, dims=[2]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=2097153, d=2, order=1, dims=[2097153]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=64, d=2, order=1, dims=[8, 8], path=hyena.HYENA_PATH_LDS1D),
     hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=60, d=2, order=1, dims=[6, 10]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=64, d=2, order=1, dims=[8, 4]), hyena.HYENA_ERR_INVALID_ARGUMENT),
    # 2D sides: powers of two in 4..1024, and N * d * 4 below 2^31
    (dict(B=1, N=2048 * 8, d=2, order=1, dims=[2048, 8]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=8 * 2048, d=2, order=1, dims=[8, 2048]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=1024 * 1024, d=512, order=1, dims=[1024, 1024]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=16384, d=2, order=1, dims=[16384], path=hyena.HYENA_PATH_LDS1D),
     hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=256, d=2, order=1, dims=[256], path=hyena.HYENA_PATH_FOURSTEP1D),
     hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=64, d=2, order=1, dims=[64], io_dtype=hyena.HYENA_F32,
          spectrum_dtype=hyena.HYENA_BF16), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=64, d=2, order=1, dims=[64], io_dtype=7), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=64, d=2, order=1, dims=[64], io_dtype=hyena.HYENA_F16,
          spectrum_dtype=hyena.HYENA_BF16), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=64, d=2, order=1, dims=[64], io_dtype=hyena.HYENA_F16,
          spectrum_dtype=hyena.HYENA_F16), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=64, d=2, order=1, dims=[64], path=9), hyena.HYENA_ERR_UNSUPPORTED),
    # 3D grids: power-of-two sides in 4..256, at most 2^20 points, N = X Y Z
    (dict(B=1, N=6 * 8 * 8, d=2, order=1, dims=[6, 8, 8]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=2 * 8 * 8, d=2, order=1, dims=[2, 8, 8]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=512 * 8 * 8, d=2, order=1, dims=[512, 8, 8]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=256 * 256 * 32, d=2, order=1, dims=[256, 256, 32]), hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=512, d=2, order=1, dims=[8, 8, 4]), hyena.HYENA_ERR_INVALID_ARGUMENT),
    (dict(B=1, N=512, d=2, order=1, dims=[8, 8, 8], path=hyena.HYENA_PATH_ROWCOL2D),
     hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=512, d=2, order=1, dims=[8, 8, 8], flags=hyena.HYENA_FLAG_CIRCULAR),
     hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=64, d=2, order=1, dims=[64], path=hyena.HYENA_PATH_ROWCOL3D),
     hyena.HYENA_ERR_UNSUPPORTED),
    (dict(B=1, N=64, d=2, order=1, dims=[4, 4, 2, 2]), hyena.HYENA_ERR_UNSUPPORTED),
])
def test_plan_create_rejects(args, code):
    st, plan = hyena.hyena_plan_create(check=False, **args)
    assert st == code, hyena.hyena_last_error()
    assert plan is None
    assert hyena.hyena_last_error()


def test_plan_create_null_output_pointer():
    lib = hyena.load()
    dims = (ctypes.c_int64 * 1)(8)
    assert lib.hyena_plan_create(None, 1, 8, 2, 1, dims, 1, 0, 0) == \
        hyena.HYENA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("N,path,M", [(4, 1, 8), (256, 1, 512), (2048, 1, 4096),
                                      (5000, 1, 16384), (8192, 1, 16384), (65536, 2, 131072),
                                      (16385, 2, 65536), (65537, 2, 262144),
                                      (524288, 2, 1 << 20), (1000000, 2, 1 << 21),
                                      (2097152, 2, 1 << 22)])
def test_path_choice_and_sizes(N, path, M):
    _, plan = hyena.hyena_plan_create(2, N, 6, 2, [N])
    spec, ws, p = hyena.hyena_plan_query(plan)
    assert p == path
    assert spec == 2 * 3 * (M // 2) * 16  # order * pairs * M/2 entries * 16 bytes
    assert ws >= 256
    hyena.hyena_plan_destroy(plan)


def test_2d_plan_sizes():
    _, plan = hyena.hyena_plan_create(1, 256 * 256, 256, 2, [256, 256])
    spec, ws, p = hyena.hyena_plan_query(plan)
    assert p == hyena.HYENA_PATH_ROWCOL2D
    assert spec == 2 * 128 * (512 * 512 // 2) * 16
    hyena.hyena_plan_destroy(plan)


@pytest.mark.parametrize("B,d,slots,copies", [(1, 768, 64, 2), (1, 32, 16, 1), (2, 64, 64, 1),
                                               (3, 64, 64, 2), (8, 768, 64, 2)])
def test_fourstep_workspace_holds_one_chunk_per_stream(B, d, slots, copies):
    # the 64K-token chain walks its channel pairs in chunks of about 64 MiB
    # of intermediate (1 MiB per pair slot of a 131072-point transform), in
    # whole groups of 16 pairs; with two or more chunks they alternate
    # between two streams, each with its own copy: the workspace holds one
    # or two chunks, never the whole intermediate of a wide plan
    _, plan = hyena.hyena_plan_create(B, 65536, d, 2, [65536])
    _, ws, p = hyena.hyena_plan_query(plan)
    assert p == hyena.HYENA_PATH_FOURSTEP1D
    inter = copies * slots * 131072 * 8
    assert inter <= ws < inter + (8 << 20)  # plus the twiddle tables
    hyena.hyena_plan_destroy(plan)


@pytest.mark.parametrize("X,Y,Z,d", [(64, 64, 64, 32), (4, 8, 16, 3), (256, 64, 64, 1)])
def test_3d_plan_sizes(X, Y, Z, d):
    _, plan = hyena.hyena_plan_create(2, X * Y * Z, d, 2, [X, Y, Z])
    spec, ws, p = hyena.hyena_plan_query(plan)
    assert p == hyena.HYENA_PATH_ROWCOL3D
    # the Hermitian half of a 2X x 2Y x 2Z grid: 8XYZ reals per channel and filter
    assert spec == 2 * ((d + 1) // 2) * (8 * X * Y * Z // 2) * 16
    # two intermediates per pair slot (after z: X Y 2Z, after y: X 2Y 2Z
    # complex64 in the chain; 8 X Y Z each for spectra), at least one slot
    assert ws >= 2 * 8 * X * Y * Z * 8
    hyena.hyena_plan_destroy(plan)
    # the mixer and implicit filters are not defined for 3D plans
    _, plan = hyena.hyena_plan_create(1, X * Y * Z, d, 1, [X, Y, Z])
    assert hyena.hyena_implicit_scratch_bytes(plan, 64)[0] == hyena.HYENA_ERR_UNSUPPORTED
    hyena.hyena_plan_destroy(plan)


def test_bf16_spectrum_halves_bytes():
    _, p32 = hyena.hyena_plan_create(2, 8192, 768, 2, [8192], hyena.HYENA_BF16, hyena.HYENA_F32)
    _, p16 = hyena.hyena_plan_create(2, 8192, 768, 2, [8192], hyena.HYENA_BF16, hyena.HYENA_BF16)
    assert hyena.hyena_plan_query(p32)[0] == 2 * hyena.hyena_plan_query(p16)[0]
    # the headline accounting: 2N reals per channel and filter at 2 bytes
    assert hyena.hyena_plan_query(p16)[0] == 2 * 768 * 2 * 8192 * 2
    hyena.hyena_plan_destroy(p32)
    hyena.hyena_plan_destroy(p16)


class _Fake:
    """Aligned, distinct, never-dereferenced addresses: validation fails first."""
    base = 1 << 40

    @classmethod
    def ptr(cls, i):
        return cls.base + i * (1 << 32)


def _plan(N=64, d=4, order=2):
    _, plan = hyena.hyena_plan_create(1, N, d, order, [N])
    return plan


def test_forward_validation_codes():
    plan = _plan()
    f = _Fake.ptr
    u, g0, g1, H, D, y, ws = (f(i) for i in range(7))
    # null pointers
    assert hyena.hyena_forward(plan, None, [g0, g1], H, D, y, ws) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_forward(plan, u, [g0, None], H, D, y, ws) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_forward(plan, u, [g0, g1], H, D, y, None) == hyena.HYENA_ERR_INVALID_ARGUMENT
    # misaligned
    assert hyena.hyena_forward(plan, u + 4, [g0, g1], H, D, y, ws) == hyena.HYENA_ERR_INVALID_ARGUMENT
    # y overlapping u, a gate, H
    assert hyena.hyena_forward(plan, u, [g0, g1], H, D, u + 16, ws) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_forward(plan, u, [g0, g1], H, D, g1, ws) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_forward(plan, u, [g0, g1], H, D, H + 32, ws) == hyena.HYENA_ERR_INVALID_ARGUMENT
    # valid pointers but the workspace was never initialised for this plan
    assert hyena.hyena_forward(plan, u, [g0, g1], H, D, y, ws) == hyena.HYENA_ERR_WORKSPACE
    assert "hyena_workspace_init" in hyena.hyena_last_error()
    assert hyena.hyena_filter_spectrum(plan, u, H, ws) == hyena.HYENA_ERR_WORKSPACE
    assert hyena.hyena_filter_spectrum(plan, None, H, ws) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_workspace_init(plan, None) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_workspace_init(plan, ws + 8) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_spectrum_export(plan, None, y) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_forward(None, u, [g0, g1], H, D, y, ws) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_plan_destroy(plan) == hyena.HYENA_OK
    assert hyena.hyena_plan_destroy(None) == hyena.HYENA_OK


def test_last_error_is_thread_local():
    import threading
    st, _ = hyena.hyena_plan_create(0, 8, 2, 1, [8], check=False)
    main_msg = hyena.hyena_last_error()
    seen = {}

    def other():
        hyena.hyena_plan_create(1, 8, 2, 99, [8], check=False)
        seen["msg"] = hyena.hyena_last_error()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert "order" in seen["msg"]
    assert hyena.hyena_last_error() == main_msg


def test_plans_can_be_created_from_many_threads():
    import threading
    errs = []

    def work():
        try:
            for N in (64, 1000, 8192, 65536):
                _, p = hyena.hyena_plan_create(2, N, 10, 2, [N])
                hyena.hyena_plan_query(p)
                hyena.hyena_plan_destroy(p)
        except Exception as e:  # pragma: no cover
            errs.append(e)

    ts = [threading.Thread(target=work) for _ in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errs


def test_timing_argument_errors():
    lib = hyena.load()
    assert lib.hyena_timing_begin(0) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert lib.hyena_timing_begin((1 << 20) + 1) == hyena.HYENA_ERR_INVALID_ARGUMENT
    # nothing recorded: end reports no kernels, reading one is out of range
    recs, dropped = hyena.hyena_timing_end()
    assert recs == {} and dropped == 0
    assert lib.hyena_timing_kernel(0, None, None, None, None, None) == hyena.HYENA_ERR_INVALID_ARGUMENT
    assert "out of range" in hyena.hyena_last_error()
    hyena.hyena_timing_release()


def test_implicit_scratch_sizes_and_validation():
    # the hidden features only (N x hidden rounded up to 16, float32, 256-byte
    # aligned): the taps are evaluated inside the spectrum kernels and never stored
    _, plan = hyena.hyena_plan_create(2, 2048, 6, 2, [2048])
    st, n = hyena.hyena_implicit_scratch_bytes(plan, 62)
    assert st == hyena.HYENA_OK and n == 2048 * 64 * 4
    assert hyena.hyena_implicit_scratch_bytes(plan, 0)[0] == hyena.HYENA_ERR_UNSUPPORTED
    assert hyena.hyena_implicit_scratch_bytes(plan, 257)[0] == hyena.HYENA_ERR_UNSUPPORTED
    f = hyena.ImplicitFilter(8, 64, 8.0, 16, 16, 16, 16, 16, 16, 16)
    # NULL H, NULL weights, out-of-range sizes: rejected before any GPU work
    assert hyena.hyena_filter_spectrum_implicit(plan, f, None, 16, 16) == \
        hyena.HYENA_ERR_INVALID_ARGUMENT
    assert hyena.hyena_filter_spectrum_implicit(plan, None, 16, 16, 16) == \
        hyena.HYENA_ERR_INVALID_ARGUMENT
    bad = hyena.ImplicitFilter(65, 64, 8.0, 16, 16, 16, 16, 16, 16, 16)
    assert hyena.hyena_filter_spectrum_implicit(plan, bad, 16, 16, 16) == \
        hyena.HYENA_ERR_UNSUPPORTED
    nul = hyena.ImplicitFilter(8, 64, 8.0, 16, 16, None, 16, 16, 16, 16)
    assert hyena.hyena_filter_spectrum_implicit(plan, nul, 16, 16, 16) == \
        hyena.HYENA_ERR_INVALID_ARGUMENT
    hyena.hyena_plan_destroy(plan)
    _, plan = hyena.hyena_plan_create(1, 20000, 3, 2, [20000])
    st, n = hyena.hyena_implicit_scratch_bytes(plan, 50)
    assert n == 20000 * 64 * 4
    hyena.hyena_plan_destroy(plan)
    _, plan = hyena.hyena_plan_create(1, 4096, 4, 2, [4096], hyena.HYENA_BF16, hyena.HYENA_BF16)
    st, n = hyena.hyena_implicit_scratch_bytes(plan, 64)
    assert n == 4096 * 64 * 4
    hyena.hyena_plan_destroy(plan)
    # grids have no implicit filters here
    _, plan = hyena.hyena_plan_create(1, 64, 2, 1, [8, 8])
    assert hyena.hyena_implicit_scratch_bytes(plan, 64)[0] == hyena.HYENA_ERR_UNSUPPORTED
    hyena.hyena_plan_destroy(plan)


@pytest.mark.parametrize("N,dims,path,flags,code", [
    (1024, [1024], 0, 1, hyena.HYENA_OK),
    (16384, [16384], 1, 1, hyena.HYENA_OK),
    (1000, [1000], 0, 1, hyena.HYENA_ERR_UNSUPPORTED),       # not a power of two
    (8, [8], 0, 1, hyena.HYENA_ERR_UNSUPPORTED),             # below 16
    (32768, [32768], 0, 1, hyena.HYENA_OK),                  # four-step path from 32768
    (2097152, [2097152], 2, 1, hyena.HYENA_OK),
    (32768, [32768], 1, 1, hyena.HYENA_ERR_UNSUPPORTED),     # beyond one workgroup
    (4096, [4096], 2, 1, hyena.HYENA_ERR_UNSUPPORTED),       # four-step below 32768
    (1 << 22, [1 << 22], 0, 1, hyena.HYENA_ERR_UNSUPPORTED),  # longest sequence 2097152
    (64, [8, 8], 0, 1, hyena.HYENA_ERR_UNSUPPORTED),         # grids
    (64, [64], 0, 2, hyena.HYENA_ERR_UNSUPPORTED),           # unknown flag
])
def test_periodic_boundary_plans(N, dims, path, flags, code):
    st, plan = hyena.hyena_plan_create(1, N, 4, 2, dims, path=path, flags=flags, check=False)
    assert st == code, hyena.hyena_last_error()
    if st == hyena.HYENA_OK:
        spec, _, p = hyena.hyena_plan_query(plan)
        if N <= 16384:
            assert p == 1
            assert spec == 2 * 4 * (N // 4) * 16  # order * d * (N/4 entries) * 16 bytes
        else:
            # four-step: order * channel pairs * (N/2 entries) * 16 bytes
            assert p == 2
            assert spec == 2 * 2 * (N // 2) * 16
        hyena.hyena_plan_destroy(plan)


def test_nd_mixer_validation():
    m = hyena.NdMixer(16, 16, 16, 16, None)
    _, p1 = hyena.hyena_plan_create(1, 64, 4, 1, [64])
    assert hyena.hyena_nd_mixer_forward(p1, m, 16, 16, 16, 16) == hyena.HYENA_ERR_UNSUPPORTED
    hyena.hyena_plan_destroy(p1)
    _, p2 = hyena.hyena_plan_create(1, 64, 4, 2, [8, 8])
    assert hyena.hyena_nd_mixer_forward(p2, m, 16, 16, 16, 16) == hyena.HYENA_ERR_UNSUPPORTED
    hyena.hyena_plan_destroy(p2)
    _, p4 = hyena.hyena_plan_create(1, 512, 4, 2, [8, 8, 8])
    assert hyena.hyena_nd_mixer_forward(p4, m, 16, 16, 16, 16) == hyena.HYENA_ERR_UNSUPPORTED
    hyena.hyena_plan_destroy(p4)
    _, p3 = hyena.hyena_plan_create(1, 64, 4, 1, [8, 8])
    assert hyena.hyena_nd_mixer_forward(p3, None, 16, 16, 16, 16) == \
        hyena.HYENA_ERR_INVALID_ARGUMENT
    bad = hyena.NdMixer(16, None, 16, 16, None)
    assert hyena.hyena_nd_mixer_forward(p3, bad, 16, 16, 16, 16) == \
        hyena.HYENA_ERR_INVALID_ARGUMENT
    # y on top of q
    same = hyena.NdMixer(4096, 16, 16, 16, None)
    assert hyena.hyena_nd_mixer_forward(p3, same, 16, 16, 4096, 16) == \
        hyena.HYENA_ERR_INVALID_ARGUMENT
    hyena.hyena_plan_destroy(p3)


def test_noalloc_refuses_before_touching_the_gpu():
    # the size check comes first, so these need no GPU
    assert hyena.hyena_forward_noalloc(None, 16, [16], 16, 16, 16) == \
        hyena.HYENA_ERR_INVALID_ARGUMENT
    st, big = hyena.hyena_plan_create(1, 65536, 768, 2, [65536])
    try:
        _, ws, _ = hyena.hyena_plan_query(big)
        assert ws > hyena.HYENA_NOALLOC_SCRATCH_BYTES
        assert hyena.hyena_forward_noalloc(big, 16, [16, 16], 16, 16, 16) == \
            hyena.HYENA_ERR_UNSUPPORTED
        assert "static scratch" in hyena.hyena_last_error()
    finally:
        hyena.hyena_plan_destroy(big)
    # the 2K and 8K width-768 workloads fit the array
    for B, N, io in ((4, 2048, hyena.HYENA_F32), (2, 8192, hyena.HYENA_BF16)):
        st, p = hyena.hyena_plan_create(B, N, 768, 2, [N], io)
        try:
            assert hyena.hyena_plan_query(p)[1] <= hyena.HYENA_NOALLOC_SCRATCH_BYTES
        finally:
            hyena.hyena_plan_destroy(p)


def test_2d_plans_up_to_1024_sides():
    for X, Y, d in ((1024, 1024, 511), (1024, 4, 3), (4, 1024, 3)):
        st, p = hyena.hyena_plan_create(1, X * Y, d, 2, [X, Y])
        try:
            spec, ws, path = hyena.hyena_plan_query(p)
            assert path == hyena.HYENA_PATH_ROWCOL2D
            assert spec == 2 * ((d + 1) // 2) * (2 * X * 2 * Y // 2) * 16
        finally:
            hyena.hyena_plan_destroy(p)


def test_plan_create_has_the_boundary_signature_and_path_is_queried_apart():
    # hyena_plan_create(plan, B, N, d, order, dims, ndims, io_dtype, spectrum_dtype) picks the
    # path itself; hyena_plan_path reports it, and rejects a NULL output
    lib = hyena.load()
    dims = (ctypes.c_int64 * 1)(65536)
    h = ctypes.c_void_p()
    assert lib.hyena_plan_create(ctypes.byref(h), 1, 65536, 4, 2, dims, 1, 0, 0) == hyena.HYENA_OK
    try:
        spec, ws = ctypes.c_size_t(), ctypes.c_size_t()
        assert lib.hyena_plan_query(h, ctypes.byref(spec), ctypes.byref(ws)) == hyena.HYENA_OK
        assert spec.value > 0 and ws.value > 0
        path = ctypes.c_int32(-1)
        assert lib.hyena_plan_path(h, ctypes.byref(path)) == hyena.HYENA_OK
        assert path.value == hyena.HYENA_PATH_FOURSTEP1D
        assert lib.hyena_plan_path(h, None) == hyena.HYENA_ERR_INVALID_ARGUMENT
        assert lib.hyena_plan_path(None, ctypes.byref(path)) == hyena.HYENA_ERR_INVALID_ARGUMENT
    finally:
        lib.hyena_plan_destroy(h)
