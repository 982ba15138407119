"""Seeded synthetic inputs for the Hyena long-convolution chain.

This module only draws numbers: it holds none of the convolution, transform or
gating arithmetic, and both the GPU path (tests, bench) and the float64 oracle
are fed from it.  Values are drawn in float64 with ``numpy.random.default_rng``
(PCG64) in a fixed order, then rounded to the storage dtype; the oracle is fed
the rounded values, upcast, so the two sides see identical inputs.

Filter laws (the pages' implicit-filter sections motivate both envelopes):
  * 1D: h[c,t] = sin(w_c t + phi_c) * exp(-alpha_c t), t = 0..N-1, the
    exponentially decaying window of "Hyena -- Long Convolutions Math",
    section "The decay window", on a damped sinusoid.
  * 2D: K[c,i,j] = sin(w_c . (i,j) + phi_c) * exp(-(i^2+j^2) / (2 sigma_c^2))
    at every signed offset |i| <= X-1, |j| <= Y-1, the Gaussian window of
    "How HyenaND works", section "An implicit filter".
Draw order: for each filter n: w^n, phi^n, alpha^n (2D: w^n [d,2], phi^n,
sigma^n); then D^n for every n; then u; then gate^n for every n.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"
F16 = "f16"   # IEEE binary16 storage (numpy float16, round to nearest even)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == F16:
        return x32.astype(np.float16)
    return f32_to_bf16_bits(x32) if dtype == BF16 else x32


def _np_storage(dtype: str):
    return {F32: np.float32, BF16: np.uint16, F16: np.float16}[dtype]


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == F16:
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


@dataclass
class Inputs:
    """Host arrays in storage dtype; ``f64()`` gives the upcast copies for the oracle.

    1D: u [B,N,d], gates [order,B,N,d], h [order,d,N]
    2D: u [B,X,Y,d], gates [order,B,X,Y,d], h [order,d,2X-1,2Y-1]
    3D: u [B,X,Y,Z,d], gates [order,B,X,Y,Z,d], h [order,d,2X-1,2Y-1,2Z-1]
    D is always float32 [order,d].
    """
    u: np.ndarray
    gates: np.ndarray
    h: np.ndarray
    D: np.ndarray
    dtype: str
    dims: tuple
    B: int
    d: int
    order: int
    meta: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        n = 1
        for v in self.dims:
            n *= v
        return n

    def f64(self):
        return (stored_to_f64(self.u, self.dtype), stored_to_f64(self.gates, self.dtype),
                stored_to_f64(self.h, self.dtype), self.D.astype(np.float64))


def make_1d(B: int, N: int, d: int, order: int, alpha_range=(1e-3, 5e-2),
            dtype: str = F32, seed: int = 0) -> Inputs:
    """Inputs for the 1D causal chain: u, gates ~ N(0,1); damped-sinusoid filters."""
    rng = np.random.default_rng(seed)
    t = np.arange(N, dtype=np.float64)
    h = np.empty((order, d, N), dtype=_np_storage(dtype))
    for n in range(order):
        w = rng.uniform(0.0, np.pi, size=d)
        phi = rng.uniform(0.0, 2.0 * np.pi, size=d)
        alpha = rng.uniform(alpha_range[0], alpha_range[1], size=d)
        hn = np.sin(w[:, None] * t[None, :] + phi[:, None]) * np.exp(-alpha[:, None] * t[None, :])
        h[n] = _store(hn, dtype)
        del hn
    D = np.stack([rng.standard_normal(d) for _ in range(order)]).astype(np.float32)
    u = _store(rng.standard_normal((B, N, d)), dtype)
    gates = np.empty((order, B, N, d), dtype=u.dtype)
    for n in range(order):
        gates[n] = _store(rng.standard_normal((B, N, d)), dtype)
    return Inputs(u=u, gates=gates, h=h, D=D, dtype=dtype, dims=(N,), B=B, d=d, order=order,
                  meta={"alpha_range": tuple(alpha_range), "seed": seed})


def make_2d(B: int, X: int, Y: int, d: int, order: int, sigma_range=(16.0, 128.0),
            dtype: str = F32, seed: int = 0) -> Inputs:
    """Inputs for the 2D non-causal chain: taps at every offset in [-(X-1), X-1] x [-(Y-1), Y-1]."""
    rng = np.random.default_rng(seed)
    i = np.arange(-(X - 1), X, dtype=np.float64)
    j = np.arange(-(Y - 1), Y, dtype=np.float64)
    r2 = i[:, None] ** 2 + j[None, :] ** 2
    K = np.empty((order, d, 2 * X - 1, 2 * Y - 1),
                 dtype=_np_storage(dtype))
    for n in range(order):
        w = rng.uniform(0.0, np.pi, size=(d, 2))
        phi = rng.uniform(0.0, 2.0 * np.pi, size=d)
        sigma = rng.uniform(sigma_range[0], sigma_range[1], size=d)
        for c in range(d):
            kc = np.sin(w[c, 0] * i[:, None] + w[c, 1] * j[None, :] + phi[c]) * \
                np.exp(-r2 / (2.0 * sigma[c] ** 2))
            K[n, c] = _store(kc, dtype)
    D = np.stack([rng.standard_normal(d) for _ in range(order)]).astype(np.float32)
    u = _store(rng.standard_normal((B, X, Y, d)), dtype)
    gates = np.empty((order, B, X, Y, d), dtype=u.dtype)
    for n in range(order):
        gates[n] = _store(rng.standard_normal((B, X, Y, d)), dtype)
    return Inputs(u=u, gates=gates, h=K, D=D, dtype=dtype, dims=(X, Y), B=B, d=d, order=order,
                  meta={"sigma_range": tuple(sigma_range), "seed": seed})


def make_3d(B: int, X: int, Y: int, Z: int, d: int, order: int, sigma_range=(4.0, 32.0),
            dtype: str = F32, seed: int = 0) -> Inputs:
    """Inputs for the 3D non-causal chain: taps at every offset in
    [-(X-1), X-1] x [-(Y-1), Y-1] x [-(Z-1), Z-1], the 2D law with a third axis:
    sin(w . (i, j, l) + phi) exp(-(i^2 + j^2 + l^2) / (2 sigma^2))."""
    rng = np.random.default_rng(seed)
    i = np.arange(-(X - 1), X, dtype=np.float64)[:, None, None]
    j = np.arange(-(Y - 1), Y, dtype=np.float64)[None, :, None]
    l = np.arange(-(Z - 1), Z, dtype=np.float64)[None, None, :]
    r2 = i ** 2 + j ** 2 + l ** 2
    K = np.empty((order, d, 2 * X - 1, 2 * Y - 1, 2 * Z - 1), dtype=_np_storage(dtype))
    for n in range(order):
        w = rng.uniform(0.0, np.pi, size=(d, 3))
        phi = rng.uniform(0.0, 2.0 * np.pi, size=d)
        sigma = rng.uniform(sigma_range[0], sigma_range[1], size=d)
        for c in range(d):
            kc = np.sin(w[c, 0] * i + w[c, 1] * j + w[c, 2] * l + phi[c]) * \
                np.exp(-r2 / (2.0 * sigma[c] ** 2))
            K[n, c] = _store(kc, dtype)
    D = np.stack([rng.standard_normal(d) for _ in range(order)]).astype(np.float32)
    u = _store(rng.standard_normal((B, X, Y, Z, d)), dtype)
    gates = np.empty((order, B, X, Y, Z, d), dtype=u.dtype)
    for n in range(order):
        gates[n] = _store(rng.standard_normal((B, X, Y, Z, d)), dtype)
    return Inputs(u=u, gates=gates, h=K, D=D, dtype=dtype, dims=(X, Y, Z), B=B, d=d, order=order,
                  meta={"sigma_range": tuple(sigma_range), "seed": seed})


# The workloads: an order-1 smoke shape, the 2K / 8K / 64K language-model
# lengths at width 768, a 256x256 image grid at width 256, and a 64^3 volume
# at width 64.
WORKLOADS = {
    0: dict(kind="1d", B=1, N=256, d=4, order=1, alpha_range=(1e-3, 5e-2), dtype=F32),
    1: dict(kind="1d", B=4, N=2048, d=768, order=2, alpha_range=(1e-4, 1e-2), dtype=F32),
    2: dict(kind="1d", B=2, N=8192, d=768, order=2, alpha_range=(1e-5, 1e-3), dtype=BF16),
    3: dict(kind="1d", B=1, N=65536, d=768, order=2, alpha_range=(1e-6, 1e-4), dtype=F32),
    4: dict(kind="2d", B=1, X=256, Y=256, d=256, order=2, sigma_range=(16.0, 128.0), dtype=F32),
    5: dict(kind="3d", B=1, X=64, Y=64, Z=64, d=64, order=2, sigma_range=(4.0, 32.0), dtype=F32),
}

WORKLOAD_NAMES = {
    0: "order1_B1_N256_d4_f32",
    1: "order2_B4_N2048_d768_f32",
    2: "order2_B2_N8192_d768_bf16",
    3: "order2_B1_N65536_d768_f32",
    4: "order2_2d_B1_256x256_d256_f32",
    5: "order2_3d_B1_64x64x64_d64_f32",
}


def make_workload(idx: int, seed: int | None = None, **override) -> Inputs:
    cfg = dict(WORKLOADS[idx])
    cfg.update(override)
    seed = idx if seed is None else seed
    kind = cfg.pop("kind")
    if kind == "1d":
        return make_1d(cfg["B"], cfg["N"], cfg["d"], cfg["order"], cfg["alpha_range"],
                       cfg["dtype"], seed)
    if kind == "3d":
        return make_3d(cfg["B"], cfg["X"], cfg["Y"], cfg["Z"], cfg["d"], cfg["order"],
                       cfg["sigma_range"], cfg["dtype"], seed)
    return make_2d(cfg["B"], cfg["X"], cfg["Y"], cfg["d"], cfg["order"], cfg["sigma_range"],
                   cfg["dtype"], seed)


@dataclass
class ImplicitWeights:
    """Weights of the implicit filter's sine MLP, stored float32 (the oracle
    gets the same values upcast)."""
    K: int
    H: int
    omega: float
    W1: np.ndarray
    b1: np.ndarray
    W2: np.ndarray
    b2: np.ndarray
    W3: np.ndarray
    b3: np.ndarray
    alpha: np.ndarray

    def arrays(self):
        return dict(W1=self.W1, b1=self.b1, W2=self.W2, b2=self.b2, W3=self.W3, b3=self.b3,
                    alpha=self.alpha)


def make_implicit(d: int, order: int, K: int = 8, H: int = 64, omega: float = 8.0,
                  alpha_range=(1e-4, 1e-2), seed: int = 0) -> ImplicitWeights:
    """Random (untrained) sine-MLP weights: uniform first layer in
    [-1/m, 1/m], hidden and output layers uniform in +-sqrt(6/H)/omega and
    +-sqrt(6/H), biases uniform in [-0.5, 0.5] (first two) and N(0, 0.1)
    (output), decay rates uniform in alpha_range.  Draw order: W1, b1, W2, b2,
    W3, b3, alpha."""
    rng = np.random.default_rng(seed)
    m = 2 * K + 1
    W1 = rng.uniform(-1.0 / m, 1.0 / m, size=(H, m))
    b1 = rng.uniform(-0.5, 0.5, size=H)
    lim = np.sqrt(6.0 / H)
    W2 = rng.uniform(-lim / omega, lim / omega, size=(H, H))
    b2 = rng.uniform(-0.5, 0.5, size=H)
    W3 = rng.uniform(-lim, lim, size=(order * d, H))
    b3 = rng.normal(0.0, 0.1, size=order * d)
    alpha = rng.uniform(*alpha_range, size=(order, d))
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return ImplicitWeights(K, H, float(np.float32(omega)), f32(W1), f32(b1), f32(W2), f32(b2),
                           f32(W3), f32(b3), f32(alpha))
