"""The torch wrapper checks every tensor it hands to the C ABI (dtype,
contiguity, device, shape, byte count) and raises ValueError before anything
is enqueued.  These run on the CPU: the plan's device is the host, so a call
whose arguments pass every check reaches the library, which rejects it with
HYENA_ERR_WORKSPACE (the workspace was never initialised) -- again before any
GPU work."""
import pytest
import torch

from long_convolution_sequence_rfft_amd import hyena


def host_plan(B, d, order, dims, io=hyena.HYENA_F32, circular=False):
    """A Plan bound to host memory, built without the GPU workspace set-up."""
    p = object.__new__(hyena.Plan)
    p.torch = torch
    N = 1
    for v in dims:
        N *= int(v)
    p.B, p.N, p.d, p.order, p.dims = B, N, d, order, tuple(dims)
    p.io_dtype = io
    p.spectrum_dtype = hyena.HYENA_F32 if io == hyena.HYENA_F16 else io
    p.circular = circular
    _, p.handle = hyena.hyena_plan_create(B, N, d, order, dims, io, p.spectrum_dtype)
    p.spectrum_bytes, p.workspace_bytes, p.path = hyena.hyena_plan_query(p.handle)
    p.device = torch.device("cpu")
    p.workspace = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8)
    p.stream = lambda: 0
    return p


def good_forward_args(p):
    dt = p.torch_io_dtype
    u = torch.zeros(p.act_shape, dtype=dt)
    gates = [torch.zeros(p.act_shape, dtype=dt) for _ in range(p.order)]
    H = torch.zeros(p.spectrum_bytes, dtype=torch.uint8)
    D = torch.zeros((p.order, p.d), dtype=torch.float32)
    y = torch.empty(p.act_shape, dtype=dt)
    return u, gates, H, D, y


def expect_workspace_error(fn):
    with pytest.raises(hyena.HyenaError) as e:
        fn()
    assert e.value.status == hyena.HYENA_ERR_WORKSPACE


@pytest.mark.parametrize("dims", [(64,), (8, 16), (4, 8, 8)])
def test_forward_arguments_that_pass_reach_the_library(dims):
    p = host_plan(2, 6, 2, dims)
    expect_workspace_error(lambda: p.forward(*good_forward_args(p)))


@pytest.mark.parametrize("what", ["u_shape", "u_dtype", "u_noncontig", "gate_count",
                                  "gate_shape", "H_small", "H_dtype", "D_shape", "D_dtype",
                                  "y_shape", "y_dtype", "u_numpy"])
def test_forward_rejects_bad_tensors(what):
    p = host_plan(2, 6, 2, (64,))
    u, gates, H, D, y = good_forward_args(p)
    if what == "u_shape":
        u = torch.zeros((2, 32, 6))
    elif what == "u_dtype":
        u = u.to(torch.float64)
    elif what == "u_noncontig":
        u = torch.zeros((2, 6, 64)).transpose(1, 2)
    elif what == "gate_count":
        gates = gates[:1]
    elif what == "gate_shape":
        gates[1] = torch.zeros((2, 64, 5))
    elif what == "H_small":
        H = H[:-16]
    elif what == "H_dtype":
        H = torch.zeros(p.spectrum_bytes // 4, dtype=torch.float32)
    elif what == "D_shape":
        D = torch.zeros((p.order * p.d,), dtype=torch.float32)
    elif what == "D_dtype":
        D = D.to(torch.float64)
    elif what == "y_shape":
        y = torch.empty((2, 63, 6))
    elif what == "y_dtype":
        y = torch.empty(p.act_shape, dtype=torch.bfloat16)
    elif what == "u_numpy":
        u = u.numpy()
    with pytest.raises(ValueError):
        p.forward(u, gates, H, D, y)


def test_spectrum_checks_filter_shape_and_output_size():
    p = host_plan(1, 4, 2, (32,))
    h = torch.zeros((2, 4, 32))
    expect_workspace_error(lambda: p.spectrum(h, torch.zeros(p.spectrum_bytes, dtype=torch.uint8)))
    with pytest.raises(ValueError):
        p.spectrum(torch.zeros((2, 4, 31)))
    with pytest.raises(ValueError):
        p.spectrum(h, torch.zeros(p.spectrum_bytes - 1, dtype=torch.uint8))
    g = host_plan(1, 3, 1, (8, 4))
    expect_workspace_error(lambda: g.spectrum(torch.zeros((1, 3, 15, 7)),
                                              torch.zeros(g.spectrum_bytes, dtype=torch.uint8)))
    with pytest.raises(ValueError):
        g.spectrum(torch.zeros((1, 3, 16, 8)))


def implicit_weights(p, hidden=8, K=3):
    m = 2 * K + 1
    f = lambda *s: torch.zeros(s, dtype=torch.float32)
    return dict(W1=f(hidden, m), b1=f(hidden), W2=f(hidden, hidden), b2=f(hidden),
                W3=f(p.order * p.d, hidden), b3=f(p.order * p.d), alpha=f(p.order, p.d))


@pytest.mark.parametrize("bad", [None, "W1_even", "W1_1d", "b1", "W2", "b2", "W3", "b3",
                                 "alpha", "H_small"])
def test_implicit_filter_weights_are_checked(bad):
    p = host_plan(1, 4, 2, (256,))
    w = implicit_weights(p)
    H = torch.zeros(p.spectrum_bytes, dtype=torch.uint8)
    if bad is None:
        # passes every check; the library then refuses the uninitialised workspace
        # (the scratch buffer is host memory here and is never touched)
        expect_workspace_error(lambda: p.spectrum_implicit(omega=8.0, H=H, **w))
        return
    if bad == "W1_even":
        w["W1"] = torch.zeros((8, 6))
    elif bad == "W1_1d":
        w["W1"] = torch.zeros(56)
    elif bad == "H_small":
        H = H[:-1]
    else:
        w[bad] = torch.zeros(w[bad].numel() + 1)
    with pytest.raises(ValueError):
        p.spectrum_implicit(omega=8.0, H=H, **w)


def test_nd_mixer_checks_taps_and_biases():
    p = host_plan(1, 4, 1, (8, 8))
    dt = torch.float32
    q, k, v = (torch.zeros(p.act_shape, dtype=dt) for _ in range(3))
    H = torch.zeros(p.spectrum_bytes, dtype=torch.uint8)
    D = torch.zeros((1, 4), dtype=dt)
    sw, sb = torch.zeros((3, 4, 3, 3)), torch.zeros((3, 4))
    expect_workspace_error(lambda: p.nd_mixer(q, k, v, sw, sb, H, D))
    expect_workspace_error(lambda: p.nd_mixer(q, k, v, sw, None, H, D))
    with pytest.raises(ValueError):
        p.nd_mixer(q, k, v, torch.zeros((3, 4, 3, 3, 3)), sb, H, D)
    with pytest.raises(ValueError):
        p.nd_mixer(q, k, v, sw, torch.zeros((3, 5)), H, D)
    with pytest.raises(ValueError):
        p.nd_mixer(q, k, torch.zeros((1, 8, 7, 4)), sw, sb, H, D)
    p3 = host_plan(1, 2, 1, (4, 4, 8))
    q3 = torch.zeros(p3.act_shape)
    H3 = torch.zeros(p3.spectrum_bytes, dtype=torch.uint8)
    expect_workspace_error(lambda: p3.nd_mixer(q3, q3.clone(), q3.clone(),
                                               torch.zeros((3, 2, 3, 3, 3)), None, H3,
                                               torch.zeros((1, 2))))
    with pytest.raises(ValueError):
        p3.nd_mixer(q3, q3.clone(), q3.clone(), torch.zeros((3, 2, 3, 3)), None, H3,
                    torch.zeros((1, 2)))


def test_export_checks_spectrum_size():
    p = host_plan(1, 2, 1, (64,))
    with pytest.raises(ValueError):
        p.export_spectrum(torch.zeros(p.spectrum_bytes - 4, dtype=torch.uint8))
