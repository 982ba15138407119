"""ctypes binding to ``libhyena_mi355x.so`` (the C ABI of include/hyena.h).

The functions below carry the C names and only marshal arguments: every step
of the computation runs in the library's HIP kernels.  ``Plan`` is a small
convenience wrapper that takes torch tensors (torch provides device memory
and the current HIP stream) and calls the same entry points.

There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhyena_mi355x.so")

HYENA_OK = 0
HYENA_ERR_INVALID_ARGUMENT = 1
HYENA_ERR_UNSUPPORTED = 2
HYENA_ERR_WORKSPACE = 3
HYENA_ERR_DEVICE = 4

HYENA_F32 = 0
HYENA_BF16 = 1
HYENA_F16 = 2

HYENA_PATH_AUTO = 0
HYENA_PATH_LDS1D = 1
HYENA_PATH_FOURSTEP1D = 2
HYENA_PATH_ROWCOL2D = 3
HYENA_PATH_ROWCOL3D = 4

EXPORTED_SYMBOLS = (
    "hyena_plan_create", "hyena_plan_query", "hyena_workspace_init", "hyena_filter_spectrum",
    "hyena_forward", "hyena_spectrum_export", "hyena_plan_destroy", "hyena_status_string",
    "hyena_last_error", "hyena_timing_begin", "hyena_timing_end", "hyena_timing_kernel",
    "hyena_timing_release", "hyena_implicit_scratch_bytes", "hyena_filter_spectrum_implicit",
    "hyena_plan_create_ex", "hyena_nd_mixer_forward", "hyena_workspace_release",
    "hyena_plan_path",
    "hyena_forward_noalloc",
)

HYENA_NOALLOC_SCRATCH_BYTES = 128 << 20


class NdMixer(ctypes.Structure):
    """hyena_nd_mixer: q, k, v and the short-convolution taps (device pointers)."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("short_w", ctypes.c_void_p), ("short_b", ctypes.c_void_p)]

HYENA_FLAG_CIRCULAR = 1


class ImplicitFilter(ctypes.Structure):
    """hyena_implicit_filter: weights of the sine MLP that generates the taps
    (device pointers as ints; see include/hyena.h)."""
    _fields_ = [("n_freqs", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("omega", ctypes.c_float), ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("b2", ctypes.c_void_p), ("W3", ctypes.c_void_p),
                ("b3", ctypes.c_void_p), ("alpha", ctypes.c_void_p)]

_lock = threading.Lock()
_lib = None


class HyenaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_name(status)}: {detail}")
        self.status = status


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "long_convolution_sequence_rfft_amd.build.build()")
            lib = ctypes.CDLL(LIB_PATH)
            i64, i32, p, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
            lib.hyena_plan_create.argtypes = [ctypes.POINTER(p), i64, i64, i64, i32,
                                              ctypes.POINTER(i64), i32, i32, i32]
            lib.hyena_plan_create_ex.argtypes = [ctypes.POINTER(p), i64, i64, i64, i32,
                                                 ctypes.POINTER(i64), i32, i32, i32, i32, i32]
            lib.hyena_plan_query.argtypes = [p, ctypes.POINTER(sz), ctypes.POINTER(sz)]
            lib.hyena_plan_path.argtypes = [p, ctypes.POINTER(i32)]
            lib.hyena_workspace_init.argtypes = [p, p, p]
            lib.hyena_workspace_release.argtypes = [p, p]
            lib.hyena_filter_spectrum.argtypes = [p, p, p, p, p]
            lib.hyena_forward.argtypes = [p, p, ctypes.POINTER(p), p, p, p, p, p]
            lib.hyena_forward_noalloc.argtypes = [p, p, ctypes.POINTER(p), p, p, p, p]
            lib.hyena_spectrum_export.argtypes = [p, p, p, p]
            lib.hyena_plan_destroy.argtypes = [p]
            lib.hyena_status_string.argtypes = [ctypes.c_int]
            lib.hyena_status_string.restype = ctypes.c_char_p
            lib.hyena_last_error.argtypes = []
            lib.hyena_last_error.restype = ctypes.c_char_p
            lib.hyena_timing_begin.argtypes = [i32]
            lib.hyena_timing_end.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i64)]
            lib.hyena_timing_kernel.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p),
                                                ctypes.POINTER(i64)] + \
                [ctypes.POINTER(ctypes.c_double)] * 3
            lib.hyena_timing_release.argtypes = []
            lib.hyena_implicit_scratch_bytes.argtypes = [p, i32, ctypes.POINTER(sz)]
            lib.hyena_nd_mixer_forward.argtypes = [p, ctypes.POINTER(NdMixer), p, p, p, p, p]
            lib.hyena_filter_spectrum_implicit.argtypes = [p, ctypes.POINTER(ImplicitFilter), p, p,
                                                           p, p]
            for name in ("hyena_plan_create", "hyena_plan_create_ex", "hyena_plan_query",
                         "hyena_plan_path",
                         "hyena_workspace_init", "hyena_workspace_release",
                         "hyena_filter_spectrum", "hyena_forward", "hyena_forward_noalloc",
                         "hyena_spectrum_export",
                         "hyena_plan_destroy", "hyena_timing_begin", "hyena_timing_end",
                         "hyena_timing_kernel", "hyena_timing_release",
                         "hyena_implicit_scratch_bytes", "hyena_filter_spectrum_implicit",
                         "hyena_nd_mixer_forward"):
                getattr(lib, name).restype = ctypes.c_int
            _lib = lib
    return _lib


def status_name(status: int) -> str:
    return load().hyena_status_string(int(status)).decode()


def hyena_last_error() -> str:
    return load().hyena_last_error().decode()


def hyena_status_string(status: int) -> str:
    return status_name(status)


def _check(status: int, where: str):
    if status != HYENA_OK:
        raise HyenaError(status, where, hyena_last_error())


# --------------------------------------------------------------------------
# C entry points (raw pointers as Python ints)
# --------------------------------------------------------------------------

def hyena_plan_create(B, N, d, order, dims, io_dtype=HYENA_F32, spectrum_dtype=None,
                      path=HYENA_PATH_AUTO, check=True, flags=0):
    """Returns (status, plan handle or None); a path other than AUTO, or flags,
    go through hyena_plan_create_ex."""
    lib = load()
    if spectrum_dtype is None:
        spectrum_dtype = HYENA_F32 if io_dtype == HYENA_F16 else io_dtype
    dims_arr = (ctypes.c_int64 * max(1, len(dims)))(*[int(x) for x in dims])
    h = ctypes.c_void_p()
    if flags or path != HYENA_PATH_AUTO:
        st = lib.hyena_plan_create_ex(ctypes.byref(h), int(B), int(N), int(d), int(order),
                                      dims_arr, len(dims), int(io_dtype), int(spectrum_dtype),
                                      int(path), int(flags))
    else:
        st = lib.hyena_plan_create(ctypes.byref(h), int(B), int(N), int(d), int(order), dims_arr,
                                   len(dims), int(io_dtype), int(spectrum_dtype))
    if check:
        _check(st, "hyena_plan_create")
    return st, (h.value if st == HYENA_OK else None)


def hyena_plan_query(plan):
    spec = ctypes.c_size_t()
    ws = ctypes.c_size_t()
    path = ctypes.c_int32()
    _check(load().hyena_plan_query(plan, ctypes.byref(spec), ctypes.byref(ws)), "hyena_plan_query")
    _check(load().hyena_plan_path(plan, ctypes.byref(path)), "hyena_plan_path")
    return spec.value, ws.value, path.value


def hyena_workspace_init(plan, workspace, stream=0):
    return load().hyena_workspace_init(plan, workspace, stream)


def hyena_workspace_release(plan, workspace):
    return load().hyena_workspace_release(plan, workspace)


def hyena_filter_spectrum(plan, h, H, workspace, stream=0):
    return load().hyena_filter_spectrum(plan, h, H, workspace, stream)


def hyena_forward(plan, u, gates, H, D, y, workspace, stream=0):
    arr = (ctypes.c_void_p * max(1, len(gates)))(*gates)
    return load().hyena_forward(plan, u, arr, H, D, y, workspace, stream)


def hyena_forward_noalloc(plan, u, gates, H, D, y, stream=0):
    arr = (ctypes.c_void_p * max(1, len(gates)))(*gates)
    return load().hyena_forward_noalloc(plan, u, arr, H, D, y, stream)


def hyena_implicit_scratch_bytes(plan, hidden):
    """Returns (status, bytes)."""
    n = ctypes.c_size_t()
    st = load().hyena_implicit_scratch_bytes(plan, int(hidden), ctypes.byref(n))
    return st, n.value


def hyena_filter_spectrum_implicit(plan, f, H, workspace, scratch, stream=0):
    return load().hyena_filter_spectrum_implicit(plan, ctypes.byref(f) if f is not None else None,
                                                 H, workspace, scratch, stream)


def hyena_nd_mixer_forward(plan, mixer, H, D, y, workspace, stream=0):
    return load().hyena_nd_mixer_forward(plan, ctypes.byref(mixer) if mixer is not None else None,
                                         H, D, y, workspace, stream)


def hyena_spectrum_export(plan, H, natural, stream=0):
    return load().hyena_spectrum_export(plan, H, natural, stream)


def hyena_plan_destroy(plan):
    return load().hyena_plan_destroy(plan)


def hyena_timing_begin(max_launches):
    _check(load().hyena_timing_begin(int(max_launches)), "hyena_timing_begin")


def hyena_timing_end():
    """Stop recording; returns ({kernel name: {launches, total_ms, min_ms,
    max_ms}}, dropped launches)."""
    lib = load()
    n = ctypes.c_int32()
    dropped = ctypes.c_int64()
    _check(lib.hyena_timing_end(ctypes.byref(n), ctypes.byref(dropped)), "hyena_timing_end")
    out = {}
    for i in range(n.value):
        name = ctypes.c_char_p()
        launches = ctypes.c_int64()
        tot, mn, mx = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        _check(lib.hyena_timing_kernel(i, ctypes.byref(name), ctypes.byref(launches),
                                       ctypes.byref(tot), ctypes.byref(mn), ctypes.byref(mx)),
               "hyena_timing_kernel")
        out[name.value.decode()] = {"launches": launches.value, "total_ms": tot.value,
                                    "min_ms": mn.value, "max_ms": mx.value}
    return out, dropped.value


def hyena_timing_release():
    _check(load().hyena_timing_release(), "hyena_timing_release")


# --------------------------------------------------------------------------
# torch convenience wrapper (device memory and stream plumbing only)
# --------------------------------------------------------------------------

class Plan:
    """One plan plus its workspace on a torch device.

    ``dims`` is ``(N,)`` for sequences, ``(X, Y)`` or ``(X, Y, Z)`` for grids.  Tensors are
    float32 or bfloat16 (io), channels last; see include/hyena.h for layouts.
    """

    def __init__(self, B, d, order, dims, io_dtype=HYENA_F32, spectrum_dtype=None,
                 path=HYENA_PATH_AUTO, device="cuda", circular=False):
        import torch
        self.torch = torch
        N = 1
        for v in dims:
            N *= int(v)
        self.B, self.N, self.d, self.order, self.dims = int(B), N, int(d), int(order), tuple(dims)
        self.io_dtype = io_dtype
        if spectrum_dtype is None:  # binary16 io takes a float32 spectrum
            spectrum_dtype = HYENA_F32 if io_dtype == HYENA_F16 else io_dtype
        self.spectrum_dtype = spectrum_dtype
        self.circular = bool(circular)
        _, self.handle = hyena_plan_create(B, N, d, order, dims, io_dtype, self.spectrum_dtype,
                                           path, flags=HYENA_FLAG_CIRCULAR if circular else 0)
        self.spectrum_bytes, self.workspace_bytes, self.path = hyena_plan_query(self.handle)
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.workspace = torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8,
                                     device=self.device)
        _check(hyena_workspace_init(self.handle, self.workspace.data_ptr(), self.stream()),
               "hyena_workspace_init")

    def stream(self):
        return self.torch.cuda.current_stream(self.device).cuda_stream

    @property
    def torch_io_dtype(self):
        return {HYENA_F32: self.torch.float32, HYENA_BF16: self.torch.bfloat16,
                HYENA_F16: self.torch.float16}[self.io_dtype]

    # ------------------------------------------------------------------
    # argument checks: every tensor is checked (dtype, contiguity, device,
    # shape or byte count) before anything is enqueued, so an undersized or
    # misplaced buffer raises ValueError instead of reaching a kernel
    # ------------------------------------------------------------------
    @property
    def act_shape(self):
        """Shape of u, the gates and y: [B, *dims, d]."""
        return (self.B,) + self.dims + (self.d,)

    @property
    def filter_shape(self):
        """Shape of the taps h: [order, d, N] or [order, d, 2X-1, 2Y-1(, 2Z-1)]."""
        if len(self.dims) == 1:
            return (self.order, self.d, self.N)
        return (self.order, self.d) + tuple(2 * int(s) - 1 for s in self.dims)

    def _tensor(self, t, name, dtype, shape=None, min_bytes=None):
        torch = self.torch
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != self.device:
            raise ValueError(f"{name} must be on {self.device}, got {t.device}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
        if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
            raise ValueError(f"{name} must hold at least {min_bytes} bytes, got "
                             f"{t.numel() * t.element_size()}")
        return t

    def _io(self, t, name, shape=None):
        return self._tensor(t, name, self.torch_io_dtype,
                            self.act_shape if shape is None else shape)

    def _spec(self, H, name="H"):
        return self._tensor(H, name, self.torch.uint8, min_bytes=self.spectrum_bytes)

    def _f32(self, t, name, shape):
        return self._tensor(t, name, self.torch.float32, shape)

    def _feedthrough(self, D):
        """D: float32 [order, d] ([d] is accepted for order 1)."""
        shape = (self.order, self.d)
        if self.order == 1 and isinstance(D, self.torch.Tensor) and D.dim() == 1:
            shape = (self.d,)
        return self._f32(D, "D", shape)

    def spectrum(self, h, H=None):
        h = self._io(h, "h", self.filter_shape)
        if H is None:
            H = self.torch.empty(self.spectrum_bytes, dtype=self.torch.uint8, device=self.device)
        self._spec(H)
        _check(hyena_filter_spectrum(self.handle, h.data_ptr(), H.data_ptr(),
                                     self.workspace.data_ptr(), self.stream()),
               "hyena_filter_spectrum")
        return H

    def spectrum_implicit(self, W1, b1, W2, b2, W3, b3, alpha, omega, H=None):
        """Spectrum from an implicit filter; weights are float32 device tensors
        W1 [hidden, 2K+1], b1 [hidden], W2 [hidden, hidden], b2 [hidden],
        W3 [order*d, hidden], b3 [order*d], alpha [order, d]."""
        ws = [W1, b1, W2, b2, W3, b3, alpha]
        if not isinstance(W1, self.torch.Tensor) or W1.dim() != 2:
            raise ValueError("W1 must be a 2-D tensor [hidden, 2K+1]")
        hidden, m = (int(x) for x in W1.shape)
        if m % 2 != 1:
            raise ValueError(f"W1 must have an odd width 2K+1, got {m}")
        nd = self.order * self.d
        for t, name, shape in ((W1, "W1", (hidden, m)), (b1, "b1", (hidden,)),
                               (W2, "W2", (hidden, hidden)), (b2, "b2", (hidden,)),
                               (W3, "W3", (nd, hidden)), (b3, "b3", (nd,)),
                               (alpha, "alpha", (self.order, self.d))):
            self._f32(t, name, shape)
        f = ImplicitFilter((m - 1) // 2, hidden, float(omega), *[t.data_ptr() for t in ws])
        st, nbytes = hyena_implicit_scratch_bytes(self.handle, hidden)
        _check(st, "hyena_implicit_scratch_bytes")
        # kept with the plan and reused, like the workspace (calls of one plan
        # must not run concurrently on different streams)
        scratch = getattr(self, "_implicit_scratch", None)
        if scratch is None or scratch.numel() < nbytes:
            scratch = self._implicit_scratch = None
            scratch = self.torch.empty(max(nbytes, 256), dtype=self.torch.uint8, device=self.device)
        if H is None:
            H = self.torch.empty(self.spectrum_bytes, dtype=self.torch.uint8, device=self.device)
        self._spec(H)
        _check(hyena_filter_spectrum_implicit(self.handle, f, H.data_ptr(),
                                              self.workspace.data_ptr(), scratch.data_ptr(),
                                              self.stream()),
               "hyena_filter_spectrum_implicit")
        self._implicit_scratch = scratch
        return H

    def forward(self, u, gates, H, D, y=None):
        u = self._io(u, "u")
        gates = list(gates)
        if len(gates) != self.order:
            raise ValueError(f"need one gate per filter ({self.order}), got {len(gates)}")
        gates = [self._io(g, f"gate {n}") for n, g in enumerate(gates)]
        self._spec(H)
        self._feedthrough(D)
        if y is None:
            y = self.torch.empty_like(u)
        self._io(y, "y")
        _check(hyena_forward(self.handle, u.data_ptr(), [g.data_ptr() for g in gates],
                             H.data_ptr(), D.data_ptr(), y.data_ptr(), self.workspace.data_ptr(),
                             self.stream()),
               "hyena_forward")
        return y

    def nd_mixer(self, q, k, v, short_w, short_b, H, D, y=None):
        """HyenaND mixer (ndims = 2 or 3, order 1): y = SiLU(sc(v)) . (K * z + D z),
        z = sc(q) . SiLU(sc(k)); short_w float32 [3, d, 3, 3] (2D) or [3, d, 3, 3, 3]
        (3D), short_b [3, d] or None."""
        q, k, v = self._io(q, "q"), self._io(k, "k"), self._io(v, "v")
        taps = (3,) * len(self.dims)
        self._f32(short_w, "short_w", (3, self.d) + taps)
        if short_b is not None:
            self._f32(short_b, "short_b", (3, self.d))
        self._feedthrough(D)
        self._spec(H)
        if y is None:
            y = self.torch.empty_like(q)
        self._io(y, "y")
        m = NdMixer(q.data_ptr(), k.data_ptr(), v.data_ptr(), short_w.data_ptr(),
                    short_b.data_ptr() if short_b is not None else None)
        _check(hyena_nd_mixer_forward(self.handle, m, H.data_ptr(), D.data_ptr(), y.data_ptr(),
                                      self.workspace.data_ptr(), self.stream()),
               "hyena_nd_mixer_forward")
        return y

    def export_spectrum(self, H):
        self._spec(H)
        if len(self.dims) == 1:
            M = 1
            while M < (self.N if self.circular else 2 * self.N):
                M *= 2
            shape = (self.order, self.d, M // 2 + 1, 2)
        elif len(self.dims) == 2:
            X, Y = self.dims
            shape = (self.order, self.d, 2 * X, Y + 1, 2)
        else:
            X, Y, Z = self.dims
            shape = (self.order, self.d, 2 * X, 2 * Y, Z + 1, 2)
        out = self.torch.zeros(shape, dtype=self.torch.float32, device=self.device)
        _check(hyena_spectrum_export(self.handle, H.data_ptr(), out.data_ptr(), self.stream()),
               "hyena_spectrum_export")
        return out

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                hyena_plan_destroy(self.handle)
                self.handle = None
        except Exception:
            pass
