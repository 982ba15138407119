"""GPU parity of filter spectra generated from an implicit filter (a sine MLP
over positions, "Hyena -- Long Convolutions Math", section "Implicit filters:
an MLP over positions") against the float64 oracle's taps."""
import numpy as np
import pytest

import oracle
from long_convolution_sequence_rfft_amd import synth
from gpu_util import from_torch, rel_err, say, to_torch

pytestmark = pytest.mark.gpu


def _oracle_taps(w: synth.ImplicitWeights, N, d, order):
    a = {k: v.astype(np.float64) for k, v in w.arrays().items()}
    return oracle.implicit_filter(N, d, order, w.omega, **a)


def _run(N, d, B, dtype, seed, K=8, H=64):
    import torch
    from long_convolution_sequence_rfft_amd import hyena
    inp = synth.make_1d(B=B, N=N, d=d, order=2, dtype=dtype, seed=seed)
    w = synth.make_implicit(d, 2, K=K, H=H, seed=seed + 1)
    io = hyena.HYENA_F32 if dtype == synth.F32 else hyena.HYENA_BF16
    say(f"[gpu] implicit N={N} d={d} B={B} {dtype} K={K} H={H}")
    plan = hyena.Plan(B, d, 2, (N,), io_dtype=io)
    dev = {k: torch.from_numpy(v).cuda() for k, v in w.arrays().items()}
    Hs = plan.spectrum_implicit(omega=w.omega, **dev)
    u = to_torch(inp.u, dtype)
    gates = [to_torch(g, dtype) for g in inp.gates]
    D = torch.from_numpy(inp.D).cuda()
    y = plan.forward(u, gates, Hs, D)
    torch.cuda.synchronize()
    u64, g64, _, D64 = inp.f64()
    h = _oracle_taps(w, N, d, 2)
    ref = oracle.hyena1d(u64, g64, h, D64, oracle.FFT)
    return from_torch(y, dtype), ref, plan, Hs, h


@pytest.mark.parametrize("N,d,B", [(2048, 6, 2), (256, 3, 1), (8192, 2, 1)])
def test_implicit_single_channel_path(N, d, B):
    y, ref, plan, _, _ = _run(N, d, B, synth.F32, seed=50)
    assert plan.path == 1
    assert rel_err(y, ref) < 1e-5


@pytest.mark.parametrize("N,d,B", [(1000, 5, 2), (20000, 3, 1)])
def test_implicit_other_paths(N, d, B):
    # ragged N (channel-pair kernels) and the four-step path
    y, ref, _, _, _ = _run(N, d, B, synth.F32, seed=51)
    assert rel_err(y, ref) < 1e-5


@pytest.mark.parametrize("N,d,H", [(1001, 37, 50), (4096, 40, 16), (2048, 3, 1)])
def test_implicit_ragged_tiles(N, d, H):
    # taps tiles of 64 rows x 64 positions: order d not a multiple of 64, N
    # not a multiple of 4 (scalar stores), hidden widths off the 16-chunk
    y, ref, _, _, _ = _run(N, d, 1, synth.F32, seed=54, K=5, H=H)
    assert rel_err(y, ref) < 1e-5


@pytest.mark.parametrize("N,d,H", [(65536, 3, 64), (32768, 5, 256), (20000, 33, 16)])
def test_implicit_four_step(N, d, H):
    # the taps evaluated in the four-step spectrum's first pass; d = 33 walks
    # several pair groups with a ragged last one, H = 256 the widest layer
    y, ref, plan, _, _ = _run(N, d, 1, synth.F32, seed=55, H=H)
    assert plan.path == 2
    e = rel_err(y, ref)
    say(f"[gpu] implicit four-step N={N} d={d} H={H}: rel err {e:.3e}")
    assert e < (5e-5 if N >= 65536 else 1e-5)


@pytest.mark.parametrize("N,d", [(4096, 5), (256, 2)])
def test_implicit_periodic(N, d):
    # periodic plan: every one of the N taps is live
    import torch
    from long_convolution_sequence_rfft_amd import hyena
    inp = synth.make_1d(B=1, N=N, d=d, order=2, seed=56)
    w = synth.make_implicit(d, 2, K=8, H=64, seed=57)
    say(f"[gpu] implicit periodic N={N} d={d}")
    plan = hyena.Plan(1, d, 2, (N,), circular=True)
    dev = {k: torch.from_numpy(v).cuda() for k, v in w.arrays().items()}
    Hs = plan.spectrum_implicit(omega=w.omega, **dev)
    y = plan.forward(to_torch(inp.u, synth.F32), [to_torch(g, synth.F32) for g in inp.gates], Hs,
                     torch.from_numpy(inp.D).cuda())
    torch.cuda.synchronize()
    u64, g64, _, D64 = inp.f64()
    h = _oracle_taps(w, N, d, 2)
    ref = oracle.hyena1d_circular(u64, g64, h, D64, oracle.FFT)
    assert rel_err(from_torch(y, synth.F32), ref) < 1e-5


def test_implicit_bf16_storage():
    y, ref, _, _, _ = _run(4096, 4, 2, synth.BF16, seed=52)
    assert rel_err(y, ref) < 1e-2


def test_implicit_spectrum_matches_transform_of_oracle_taps():
    _, _, plan, Hs, h = _run(2048, 3, 1, synth.F32, seed=53, K=16, H=32)
    nat = plan.export_spectrum(Hs).cpu().numpy().astype(np.float64)
    nat = nat[..., 0] + 1j * nat[..., 1]
    M = 4096
    for n in range(2):
        for c in range(3):
            ref = oracle.fft(np.concatenate([h[n, c], np.zeros(M - 2048)]))[:M // 2 + 1]
            assert rel_err(nat[n, c], ref) < 1e-5
