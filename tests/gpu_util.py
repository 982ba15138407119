"""Shared helpers for the GPU tests: run the HIP path through the C ABI on
seeded inputs, and compute the oracle on the same stored values."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from long_convolution_sequence_rfft_amd import synth


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == synth.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == synth.F16:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_torch(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == synth.BF16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu(inp: synth.Inputs, path=0, spectrum_dtype=None, plan=None, reps=1):
    """Spectrum + forward through the C ABI.  Returns (y float64, plan, H)."""
    import torch
    from long_convolution_sequence_rfft_amd import hyena
    io = {synth.F32: hyena.HYENA_F32, synth.BF16: hyena.HYENA_BF16,
          synth.F16: hyena.HYENA_F16}[inp.dtype]
    say(f"[gpu] B={inp.B} dims={inp.dims} d={inp.d} order={inp.order} dtype={inp.dtype} "
        f"path={path} spec={spectrum_dtype}")
    if plan is None:
        plan = hyena.Plan(inp.B, inp.d, inp.order, inp.dims, io_dtype=io,
                          spectrum_dtype=spectrum_dtype, path=path)
    u = to_torch(inp.u, inp.dtype)
    gates = [to_torch(inp.gates[n], inp.dtype) for n in range(inp.order)]
    h = to_torch(inp.h, inp.dtype)
    D = torch.from_numpy(inp.D).cuda()
    H = plan.spectrum(h)
    y = None
    for _ in range(reps):
        y = plan.forward(u, gates, H, D)
    torch.cuda.synchronize()
    return from_torch(y, inp.dtype), plan, H


def oracle_ref(inp: synth.Inputs, channels=None, method=oracle.FFT) -> np.ndarray:
    """Oracle on the stored values (float64), optionally on a channel subset."""
    u, g, h, D = inp.f64()
    if channels is not None:
        ch = np.asarray(channels)
        u, g, D = u[..., ch], g[..., ch], D[:, ch]
        h = h[:, ch]
    if len(inp.dims) == 1:
        return oracle.hyena1d(u, g, h, D, method)
    if len(inp.dims) == 2:
        return oracle.hyena2d(u, g, h, D, method)
    return oracle.hyena3d(u, g, h, D, method)


def rel_err(y, ref) -> float:
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-300))
