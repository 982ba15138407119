"""Float64 CPU oracle for the Hyena long-convolution chain.

TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only code allowed to import this module.
The GPU library never imports, links or calls it, and it imports nothing from
the GPU package.  The arithmetic lives in ``oracle.c`` (plain C, OpenMP over
independent (batch, channel) units); this module only builds it with gcc and
marshals numpy float64 arrays through ctypes.

Functions follow the pages cited in ``oracle.c``:
  * ``causal_conv(z, h, D, method)``  -- [P2] "The primitive" / [P1] "FFTConv"
  * ``hyena1d(u, gates, h, D, method)`` -- [P1] "The Hyena operator", [P2]
    "The Toeplitz picture" (gate after each convolution)
  * ``conv2d`` / ``hyena2d`` -- [P3] "How HyenaND works", non-causal zero-padded
    2D convolution on the native grid
  * ``conv3d`` / ``hyena3d`` -- the same on a 3D grid
  * ``dwconv3x3x3`` / ``hyena3d_block`` -- the mixer on a 3D grid (3x3x3 short
    convolutions)
  * ``fft`` -- [P2] "Counting the cost" radix-2 FFT
  * ``circular_conv`` -- [P2] "Linear vs circular" (the unpadded contrast)
  * ``circular_conv_direct`` / ``hyena1d_circular`` -- the chain with periodic
    (unpadded, length-N circular) convolutions
  * ``dwconv3x3`` / ``hyena2d_block`` -- [P3] "Putting it together": short
    conv, inner gate q . SiLU(k), 2D long conv, outer gate SiLU(v)
  * ``implicit_filter`` -- [P2] "Implicit filters" and "The decay window":
    taps window(t) * FFN(gamma(t)) from a sine MLP over positions

Every function has at least one pin in ``tests/test_oracle_pins.py`` that does
not go through this code (printed worked example, numpy routines, closed
forms, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DIRECT = 0
FFT = 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_fft.argtypes = [i64, p, p, ctypes.c_int]
            lib.oracle_fft.restype = ctypes.c_int
            lib.oracle_causal_conv_direct.argtypes = [i64, i64, i64, p, p, p, p]
            lib.oracle_causal_conv_direct.restype = None
            lib.oracle_causal_conv_fft.argtypes = [i64, i64, i64, p, p, p, p]
            lib.oracle_causal_conv_fft.restype = ctypes.c_int
            lib.oracle_circular_conv_fft.argtypes = [i64, i64, i64, p, p, p]
            lib.oracle_circular_conv_fft.restype = ctypes.c_int
            lib.oracle_hyena1d.argtypes = [i64, i64, i64, i32, p, p, p, p, p, i32]
            lib.oracle_hyena1d.restype = ctypes.c_int
            lib.oracle_conv2d_direct.argtypes = [i64, i64, i64, i64, p, p, p, p]
            lib.oracle_conv2d_direct.restype = None
            lib.oracle_conv2d_fft.argtypes = [i64, i64, i64, i64, p, p, p, p]
            lib.oracle_conv2d_fft.restype = ctypes.c_int
            lib.oracle_hyena2d.argtypes = [i64, i64, i64, i64, i32, p, p, p, p, p, i32]
            lib.oracle_hyena2d.restype = ctypes.c_int
            lib.oracle_conv3d_direct.argtypes = [i64, i64, i64, i64, i64, p, p, p, p]
            lib.oracle_conv3d_direct.restype = None
            lib.oracle_conv3d_fft.argtypes = [i64, i64, i64, i64, i64, p, p, p, p]
            lib.oracle_conv3d_fft.restype = ctypes.c_int
            lib.oracle_hyena3d.argtypes = [i64, i64, i64, i64, i64, i32, p, p, p, p, p, i32]
            lib.oracle_hyena3d.restype = ctypes.c_int
            lib.oracle_dwconv3x3x3.argtypes = [i64, i64, i64, i64, i64, p, p, p, p]
            lib.oracle_dwconv3x3x3.restype = None
            lib.oracle_hyena3d_block.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, p, p, p,
                                                 i32]
            lib.oracle_hyena3d_block.restype = ctypes.c_int
            lib.oracle_circular_conv_direct.argtypes = [i64, i64, i64, p, p, p, p]
            lib.oracle_circular_conv_direct.restype = None
            lib.oracle_hyena1d_circular.argtypes = [i64, i64, i64, i32, p, p, p, p, p, i32]
            lib.oracle_hyena1d_circular.restype = ctypes.c_int
            lib.oracle_dwconv3x3.argtypes = [i64, i64, i64, i64, p, p, p, p]
            lib.oracle_dwconv3x3.restype = None
            lib.oracle_hyena2d_block.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p, i32]
            lib.oracle_hyena2d_block.restype = ctypes.c_int
            lib.oracle_implicit_filter.argtypes = [i64, i64, i32, i32, i32, ctypes.c_double,
                                                   p, p, p, p, p, p, p, p]
            lib.oracle_implicit_filter.restype = None
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def fft(x, inverse: bool = False) -> np.ndarray:
    """Unscaled radix-2 DFT of a complex vector (sign -1 forward, +1 inverse)."""
    x = np.asarray(x, dtype=np.complex128)
    re = np.ascontiguousarray(x.real.copy())
    im = np.ascontiguousarray(x.imag.copy())
    rc = _load().oracle_fft(re.size, _ptr(re), _ptr(im), +1 if inverse else -1)
    if rc != 0:
        raise ValueError("length must be a power of two")
    return re + 1j * im


def causal_conv(z, h, D, method: int = DIRECT) -> np.ndarray:
    """w[b,t,c] = sum_{s<=t} h[c,s] z[b,t-s,c] + D[c] z[b,t,c]; z [B,N,d], h [d,N]."""
    z, h, D = _f64(z), _f64(h), _f64(D)
    B, N, d = z.shape
    assert h.shape == (d, N) and D.shape == (d,)
    w = np.empty_like(z)
    lib = _load()
    if method == DIRECT:
        lib.oracle_causal_conv_direct(B, N, d, _ptr(z), _ptr(h), _ptr(D), _ptr(w))
    else:
        if lib.oracle_causal_conv_fft(B, N, d, _ptr(z), _ptr(h), _ptr(D), _ptr(w)) != 0:
            raise MemoryError("oracle_causal_conv_fft failed")
    return w


def circular_conv(z, h) -> np.ndarray:
    """Unpadded length-N circular convolution (the wrap-around contrast)."""
    z, h = _f64(z), _f64(h)
    B, N, d = z.shape
    w = np.empty_like(z)
    if _load().oracle_circular_conv_fft(B, N, d, _ptr(z), _ptr(h), _ptr(w)) != 0:
        raise ValueError("N must be a power of two")
    return w


def hyena1d(u, gates, h, D, method: int = DIRECT) -> np.ndarray:
    """Order-N chain: u [B,N,d], gates [order,B,N,d], h [order,d,N], D [order,d]."""
    u, gates, h, D = _f64(u), _f64(gates), _f64(h), _f64(D)
    B, N, d = u.shape
    order = gates.shape[0]
    assert gates.shape == (order, B, N, d)
    assert h.shape == (order, d, N) and D.shape == (order, d)
    y = np.empty_like(u)
    rc = _load().oracle_hyena1d(B, N, d, order, _ptr(u), _ptr(gates), _ptr(h), _ptr(D),
                                _ptr(y), method)
    if rc != 0:
        raise MemoryError("oracle_hyena1d failed")
    return y


def conv2d(z, K, D, method: int = DIRECT) -> np.ndarray:
    """Non-causal 2D conv: z [B,X,Y,d], K [d,2X-1,2Y-1] (offset (i,j) at (i+X-1,j+Y-1))."""
    z, K, D = _f64(z), _f64(K), _f64(D)
    B, X, Y, d = z.shape
    assert K.shape == (d, 2 * X - 1, 2 * Y - 1) and D.shape == (d,)
    w = np.empty_like(z)
    lib = _load()
    if method == DIRECT:
        lib.oracle_conv2d_direct(B, X, Y, d, _ptr(z), _ptr(K), _ptr(D), _ptr(w))
    else:
        if lib.oracle_conv2d_fft(B, X, Y, d, _ptr(z), _ptr(K), _ptr(D), _ptr(w)) != 0:
            raise MemoryError("oracle_conv2d_fft failed")
    return w


def hyena2d(u, gates, K, D, method: int = DIRECT) -> np.ndarray:
    """2D chain: u [B,X,Y,d], gates [order,B,X,Y,d], K [order,d,2X-1,2Y-1], D [order,d]."""
    u, gates, K, D = _f64(u), _f64(gates), _f64(K), _f64(D)
    B, X, Y, d = u.shape
    order = gates.shape[0]
    assert gates.shape == (order, B, X, Y, d)
    assert K.shape == (order, d, 2 * X - 1, 2 * Y - 1) and D.shape == (order, d)
    y = np.empty_like(u)
    rc = _load().oracle_hyena2d(B, X, Y, d, order, _ptr(u), _ptr(gates), _ptr(K), _ptr(D),
                                _ptr(y), method)
    if rc != 0:
        raise MemoryError("oracle_hyena2d failed")
    return y


IMPLICIT_MAX_FREQS = 64
IMPLICIT_MAX_HIDDEN = 256


def implicit_filter(N, d, order, omega, W1, b1, W2, b2, W3, b3, alpha) -> np.ndarray:
    """Taps h [order, d, N] = exp(-alpha t) * FFN(gamma(t)); W1 [H, 2K+1],
    W2 [H, H], W3 [order*d, H], alpha [order, d] (see oracle.c)."""
    W1, b1, W2, b2 = _f64(W1), _f64(b1), _f64(W2), _f64(b2)
    W3, b3, alpha = _f64(W3), _f64(b3), _f64(alpha)
    H, m = W1.shape
    K = (m - 1) // 2
    assert m == 2 * K + 1 and K <= IMPLICIT_MAX_FREQS and H <= IMPLICIT_MAX_HIDDEN
    assert b1.shape == (H,) and W2.shape == (H, H) and b2.shape == (H,)
    assert W3.shape == (order * d, H) and b3.shape == (order * d,)
    assert alpha.shape == (order, d)
    h = np.empty((order, d, N))
    _load().oracle_implicit_filter(N, d, order, K, H, float(omega), _ptr(W1), _ptr(b1),
                                   _ptr(W2), _ptr(b2), _ptr(W3), _ptr(b3), _ptr(alpha), _ptr(h))
    return h


def circular_conv_direct(z, h, D) -> np.ndarray:
    """w[b,t,c] = sum_s h[c,s] z[b,(t-s) mod N,c] + D[c] z[b,t,c] (written out)."""
    z, h, D = _f64(z), _f64(h), _f64(D)
    B, N, d = z.shape
    assert h.shape == (d, N) and D.shape == (d,)
    w = np.empty_like(z)
    _load().oracle_circular_conv_direct(B, N, d, _ptr(z), _ptr(h), _ptr(D), _ptr(w))
    return w


def hyena1d_circular(u, gates, h, D, method: int = DIRECT) -> np.ndarray:
    """Order-N chain with periodic convolutions (shapes as hyena1d)."""
    u, gates, h, D = _f64(u), _f64(gates), _f64(h), _f64(D)
    B, N, d = u.shape
    order = gates.shape[0]
    assert gates.shape == (order, B, N, d)
    assert h.shape == (order, d, N) and D.shape == (order, d)
    y = np.empty_like(u)
    rc = _load().oracle_hyena1d_circular(B, N, d, order, _ptr(u), _ptr(gates), _ptr(h), _ptr(D),
                                         _ptr(y), method)
    if rc != 0:
        raise ValueError("oracle_hyena1d_circular failed (FFT route needs N a power of two)")
    return y


def dwconv3x3(x, w, bias=None) -> np.ndarray:
    """Depthwise 3x3 cross-correlation, zero padding 1: x [B,X,Y,d], w [d,3,3]."""
    x, w = _f64(x), _f64(w)
    B, X, Y, d = x.shape
    assert w.shape == (d, 3, 3)
    b = _f64(bias) if bias is not None else None
    o = np.empty_like(x)
    _load().oracle_dwconv3x3(B, X, Y, d, _ptr(x), _ptr(w), _ptr(b) if b is not None else None,
                             _ptr(o))
    return o


def conv3d(z, K, D, method: int = DIRECT) -> np.ndarray:
    """Non-causal 3D conv: z [B,X,Y,Z,d], K [d,2X-1,2Y-1,2Z-1] (offset (i,j,l) at
    (i+X-1, j+Y-1, l+Z-1))."""
    z, K, D = _f64(z), _f64(K), _f64(D)
    B, X, Y, Z, d = z.shape
    assert K.shape == (d, 2 * X - 1, 2 * Y - 1, 2 * Z - 1) and D.shape == (d,)
    w = np.empty_like(z)
    lib = _load()
    if method == DIRECT:
        lib.oracle_conv3d_direct(B, X, Y, Z, d, _ptr(z), _ptr(K), _ptr(D), _ptr(w))
    else:
        if lib.oracle_conv3d_fft(B, X, Y, Z, d, _ptr(z), _ptr(K), _ptr(D), _ptr(w)) != 0:
            raise MemoryError("oracle_conv3d_fft failed")
    return w


def hyena3d(u, gates, K, D, method: int = DIRECT) -> np.ndarray:
    """3D chain: u [B,X,Y,Z,d], gates [order,B,X,Y,Z,d], K [order,d,2X-1,2Y-1,2Z-1],
    D [order,d]."""
    u, gates, K, D = _f64(u), _f64(gates), _f64(K), _f64(D)
    B, X, Y, Z, d = u.shape
    order = gates.shape[0]
    assert gates.shape == (order, B, X, Y, Z, d)
    assert K.shape == (order, d, 2 * X - 1, 2 * Y - 1, 2 * Z - 1) and D.shape == (order, d)
    y = np.empty_like(u)
    rc = _load().oracle_hyena3d(B, X, Y, Z, d, order, _ptr(u), _ptr(gates), _ptr(K), _ptr(D),
                                _ptr(y), method)
    if rc != 0:
        raise MemoryError("oracle_hyena3d failed")
    return y


def hyena2d_block(q, k, v, sw, sb, K, D, method: int = DIRECT) -> np.ndarray:
    """HyenaND mixer: q, k, v [B,X,Y,d]; sw [3,d,3,3]; sb [3,d] or None;
    K [d,2X-1,2Y-1]; D [d]."""
    q, k, v, sw, K, D = _f64(q), _f64(k), _f64(v), _f64(sw), _f64(K), _f64(D)
    B, X, Y, d = q.shape
    assert sw.shape == (3, d, 3, 3) and K.shape == (d, 2 * X - 1, 2 * Y - 1) and D.shape == (d,)
    b = _f64(sb) if sb is not None else None
    y = np.empty_like(q)
    rc = _load().oracle_hyena2d_block(B, X, Y, d, _ptr(q), _ptr(k), _ptr(v), _ptr(sw),
                                      _ptr(b) if b is not None else None, _ptr(K), _ptr(D),
                                      _ptr(y), method)
    if rc != 0:
        raise MemoryError("oracle_hyena2d_block failed")
    return y


def dwconv3x3x3(x, w, bias=None) -> np.ndarray:
    """Depthwise 3x3x3 cross-correlation, zero padding 1: x [B,X,Y,Z,d], w [d,3,3,3]."""
    x, w = _f64(x), _f64(w)
    B, X, Y, Z, d = x.shape
    assert w.shape == (d, 3, 3, 3)
    b = _f64(bias) if bias is not None else None
    o = np.empty_like(x)
    _load().oracle_dwconv3x3x3(B, X, Y, Z, d, _ptr(x), _ptr(w),
                               _ptr(b) if b is not None else None, _ptr(o))
    return o


def hyena3d_block(q, k, v, sw, sb, K, D, method: int = DIRECT) -> np.ndarray:
    """HyenaND mixer on a 3D grid: q, k, v [B,X,Y,Z,d]; sw [3,d,3,3,3]; sb [3,d] or None;
    K [d,2X-1,2Y-1,2Z-1]; D [d]."""
    q, k, v, sw, K, D = _f64(q), _f64(k), _f64(v), _f64(sw), _f64(K), _f64(D)
    B, X, Y, Z, d = q.shape
    assert sw.shape == (3, d, 3, 3, 3) and D.shape == (d,)
    assert K.shape == (d, 2 * X - 1, 2 * Y - 1, 2 * Z - 1)
    b = _f64(sb) if sb is not None else None
    y = np.empty_like(q)
    rc = _load().oracle_hyena3d_block(B, X, Y, Z, d, _ptr(q), _ptr(k), _ptr(v), _ptr(sw),
                                      _ptr(b) if b is not None else None, _ptr(K), _ptr(D),
                                      _ptr(y), method)
    if rc != 0:
        raise MemoryError("oracle_hyena3d_block failed")
    return y
