"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The plan logic and workspace record (csrc/plan.cpp, pure host code) and the
float64 oracle (oracle/oracle.c) are compiled for the CPU with
-fsanitize=address,undefined and driven by small native programs in
tests/native/.  Any sanitizer report makes the program exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "long_convolution_sequence_rfft_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")


def _build_and_run(tmp_path, compiler, sources, extra, name):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    exe = str(tmp_path / name)
    cmd = [compiler] + SAN + extra + sources + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed: {' '.join(cmd)}\n{r.stderr}"
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    return out


def test_plan_and_workspace_record_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "g++", [os.path.join(NATIVE, "host_checks.cpp"),
                                           os.path.join(CSRC, "plan.cpp")],
                         ["-std=c++17", "-pthread", "-I", CSRC, "-I",
                          os.path.join(ROOT, "include")], "host_checks")
    assert "host checks passed" in out


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "gcc", [os.path.join(NATIVE, "oracle_checks.c"),
                                           os.path.join(ROOT, "oracle", "oracle.c")],
                         ["-std=c99", "-fopenmp", "-lm"], "oracle_checks")
    assert "oracle checks passed" in out


def test_hyena_log_reports_plans_and_errors():
    code = ("from long_convolution_sequence_rfft_amd import hyena\n"
            "st, p = hyena.hyena_plan_create(2, 8192, 16, 2, [8192], check=False)\n"
            "hyena.hyena_plan_destroy(p)\n"
            "hyena.hyena_plan_create(1, 3, 2, 1, [3], check=False)\n")
    env = dict(os.environ, HYENA_LOG="1", PYTHONPATH=ROOT)
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert "[hyena] plan" in r.stderr and "path LDS1D" in r.stderr
    assert "[hyena] error 2" in r.stderr
    env["HYENA_LOG"] = "0"
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env,
                       timeout=120)
    assert "[hyena]" not in r.stderr
