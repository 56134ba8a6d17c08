"""The host-side library code (codebooks, seeded matrices, status strings,
argument checks) built with AddressSanitizer and UndefinedBehaviorSanitizer
and run on the CPU; its results must equal the shipped library's up to the
last bits (the two builds use different compilers, which contract and order
fp64 operations differently).  The device code is not built here (GPU
sanitizers are not available)."""

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_run(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = tmp_path_factory.mktemp("asan") / "host_sanitize"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_sanitize.cpp"),
           os.path.join(ROOT, "online_vector_quantization_amd", "csrc", "host_math.cpp"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(out)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    rows = {}
    for line in r.stdout.splitlines():
        parts = line.split()
        if parts[0] in ("codebook", "rotation"):
            rows[(parts[0], int(parts[1]), int(parts[2]))] = np.array([float(x) for x in parts[3:]])
        elif parts[0] == "polar":
            rows[("polar", int(parts[1]))] = np.array([float(x) for x in parts[2:]])
        elif parts[0] == "status":
            rows[("status", int(parts[1]))] = " ".join(parts[2:])
        elif parts[0] == "bad":
            rows["bad"] = int(parts[1])
    return rows


def test_sanitized_host_code_is_clean(sanitized_run):
    assert sanitized_run["bad"] == 0


def test_sanitized_results_equal_the_library(sanitized_run):
    import online_vector_quantization_amd as tq
    for (kind, d, b), v in [(k, r) for k, r in sanitized_run.items() if isinstance(k, tuple) and k[0] == "codebook"]:
        c, t, mse = tq.make_codebook(d, b)
        np.testing.assert_allclose(v, np.concatenate([c, t, [mse]]), rtol=1e-12, atol=1e-14, err_msg=str((d, b)))
    for (kind, d, k), v in [(k, r) for k, r in sanitized_run.items() if isinstance(k, tuple) and k[0] == "rotation"]:
        m = tq.make_rotation(d, 7, k).reshape(-1)
        np.testing.assert_allclose(v, m[:len(v)], rtol=1e-12, atol=1e-14, err_msg=str((d, k)))
    for d in (64, 256):
        c, t = tq.make_polar_codebook(d)
        np.testing.assert_allclose(sanitized_run[("polar", d)], np.concatenate([c.reshape(-1), t.reshape(-1)]),
                                   rtol=1e-12, atol=1e-14, err_msg=str(d))
    for s in range(-5, 1):
        assert sanitized_run[("status", s)] == tq.status_string(s)
