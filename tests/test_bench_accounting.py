"""Host-side checks of the benchmark's accounting (no GPU): the algorithmic
bytes of each workload, the split of the flop model over the kernels that
carry it, the roofline record, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_convolution_sequence_rfft_amd.synth import WORKLOADS  # noqa: E402


@pytest.mark.parametrize("idx,mb", [(1, 125.8), (2, 151.0), (3, 1610.6), (4, 805.3), (5, 1342.2)])
def test_algorithmic_bytes(idx, mb):
    # (2 + order) activations + order Hermitian half-spectra + feedthrough
    cfg = WORKLOADS[idx]
    spec = "bf16" if cfg["dtype"] == "bf16" else "f32"
    assert abs(bench.algorithmic_bytes(cfg, spec) / 1e6 - mb) < 0.1


def _split(cfg, kernels):
    return [bench.kernel_share(cfg, k) for k in kernels]


@pytest.mark.parametrize("idx,kernels", [
    (1, ["hy::hyena_lds1d_real_forward<2048, float, float, false>",
         "hy::hyena_stage<float, true, false>", "hy::hyena_stage<float, false, true>"]),
    (2, ["hy::hyena_lds1d_real_forward<8192, unsigned short, unsigned short, false>",
         "hy::hyena_stage16_full<true>", "hy::hyena_stage16_full<false>"]),
    (3, ["hy::hyena_mp_outer<512, float, 0, true, true>", "hy::hyena_mp_outer<512, float, 1, true, true>",
         "hy::hyena_mp_outer<512, float, 2, true, true>", "hy::hyena_mp_inner<256, float, 0, false>"]),
    (4, ["hy::hyena_mp_outer<512, float, 0, true, true>", "hy::hyena_mp_outer<512, float, 1, true, true>",
         "hy::hyena_mp_outer<512, float, 2, true, true>", "hy::hyena_mp_inner<512, float, 0, true>"]),
    (5, ["hy::hyena_mp_outer<128, float, 0, true, false>", "hy::hyena_mp_outer<128, float, 1, true, false>",
         "hy::hyena_mp_outer<128, float, 2, true, false>", "hy::hyena_mp_mid<128, 0, true>",
         "hy::hyena_mp_mid<128, 1, true>", "hy::hyena_mp_inner<128, float, 0, true>"]),
])
def test_kernel_shares_cover_the_forward(idx, kernels):
    # the flops of the model and the algorithmic bytes are each attributed
    # once across the kernels of one forward (flops up to the 8-vs-9 per-tc
    # rounding of the product term in the multi-pass split)
    cfg = WORKLOADS[idx]
    parts = _split(cfg, kernels)
    flops = sum(p[0] for p in parts)
    nbytes = sum(p[1] for p in parts)
    total_f = bench.algorithmic_flops(cfg)
    assert abs(flops - total_f) / total_f < 0.01
    assert nbytes == bench.algorithmic_bytes(cfg, cfg["dtype"])


def test_roofline_record_fields():
    cfg = WORKLOADS[2]
    name = "hy::hyena_lds1d_real_forward<8192, unsigned short, unsigned short, false>"
    res = {"cfg": cfg, "workload": "no-such-workload",
           "kernels": {name: {"launches_per_forward": 1.0, "avg_launch_ms": 0.1,
                              "ms_per_forward": 0.1}}}
    r = bench.roofline_of(res)
    assert r["bound"] == "alu" and r["unit"] == "TFLOP/s"
    assert abs(r["achieved"] - bench.algorithmic_flops(cfg) / 1e-4 / 1e12) < 1e-2
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None  # no counters for this workload name


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    msg = json.loads(out.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_roofline_reports_the_hbm_fraction_beside_the_alu_one():
    cfg = WORKLOADS[2]
    name = "hy::hyena_lds1d_real_forward<8192, unsigned short, unsigned short, false>"
    res = {"cfg": cfg, "workload": "no-such-workload",
           "kernels": {name: {"launches_per_forward": 1.0, "avg_launch_ms": 0.1,
                              "ms_per_forward": 0.1}}}
    r = bench.roofline_of(res)
    gbps = bench.algorithmic_bytes(cfg, "bf16") / 1e-4 / 1e9
    assert abs(r["hbm"]["achieved"] - gbps) < 0.1
    assert abs(r["hbm"]["frac"] - gbps / 8000.0) < 1e-4
    assert r["alu"]["frac"] == r["frac"]
    assert "packed" in r["peak_kind"]
    assert abs(r["frac_of_published_fp32"] - r["achieved"] / 157.3) < 1e-3


def test_host_info_fields():
    info = bench.host_info()
    assert info["host_cpus_available"] >= 1
    assert set(info) == {"host_cpus_available", "cpu_model", "omp_num_threads_env"}


def test_roofline_reports_kernel_overlap():
    # two launches of 0.6 ms each per 1.0 ms forward: the kernels overlap
    cfg = WORKLOADS[3]
    a = "hy::hyena_mp_inner<256, float, 0, false>"
    b = "hy::hyena_mp_outer<512, float, 1, true, true>"
    res = {"cfg": cfg, "workload": "no-such-workload", "traced_ms_per_step": 1.0,
           "kernels": {a: {"launches_per_forward": 1.0, "avg_launch_ms": 0.6, "ms_per_forward": 0.6},
                       b: {"launches_per_forward": 1.0, "avg_launch_ms": 0.6, "ms_per_forward": 0.6}}}
    assert bench.roofline_of(res)["kernel_time_over_step_time"] == 1.2
    del res["traced_ms_per_step"]
    assert "kernel_time_over_step_time" not in bench.roofline_of(res)
