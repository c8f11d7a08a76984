"""The indexer-logits kernel source, built for the CPU (tests/cpu_build: one
host thread per lane, cross-lane operations and barriers emulated, every
wait time-limited) under AddressSanitizer, and run through the library's own
launcher on the inputs of the GPU tests -- the causal-range case whose GPU
run did not finish among them.

It checks what the source itself does on those inputs: that every workgroup
finishes (no barrier some lanes miss, no collective some lanes skip, no
endless loop), that no global or LDS access leaves its buffer, that nothing
outside the rows' ranges or in the padding columns is written, and that the
values agree with the oracle within the GPU tests' bound.  The compiled GPU
code and the hardware are not modelled; a pass here clears the source, not
the machine code.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SENTINEL = np.float32(-1234.5)


@pytest.fixture(scope="module")
def host_kernel(tmp_path_factory):
    if not os.path.exists(CLANG) and not shutil.which("clang++"):
        pytest.skip("clang++ not available")
    clang = CLANG if os.path.exists(CLANG) else shutil.which("clang++")
    exe = tmp_path_factory.mktemp("cpu_build") / "mqa_logits_host"
    cmd = [clang, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
           "-pthread", "-Wno-psabi",
           "-I", os.path.join(ROOT, "tests", "cpu_build", "shim"),
           "-I", os.path.join(ROOT, "paged_quantized_kv_amd", "csrc"),
           "-I", os.path.join(ROOT, "include"),
           "-x", "c++", os.path.join(ROOT, "tests", "cpu_build", "mqa_logits_host.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def run_host(exe, tmp_path, q, k, k_scale, w, ks, ke, cols, pad=0):
    M, H, _ = q.shape
    N = k.shape[0]
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([M, H, N, cols, cols + pad], np.int64).tobytes())
        for a, t in ((q, np.uint8), (k, np.uint8), (k_scale, np.float32), (w, np.float32),
                     (ks, np.int32), (ke, np.int32)):
            f.write(np.ascontiguousarray(a, dtype=t).tobytes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([str(exe), str(inp), str(out)], capture_output=True, text=True,
                       timeout=900, env=env)
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    return np.fromfile(out, np.float32).reshape(M, cols + pad)


def check(exe, tmp_path, q, k, k_scale, w, ks, ke, cols, pad=0):
    from test_gpu_logits import bound   # the GPU tests' derived bound
    got = run_host(exe, tmp_path, q, k, k_scale, w, ks, ke, cols, pad)
    M = q.shape[0]
    ref = np.full((M, cols), np.nan)
    oracle.fp8_mqa_logits(q, k, k_scale, w, ks, ke, ref)
    assert np.all(got[:, cols:] == SENTINEL), "padding columns written"
    body = got[:, :cols].astype(np.float64)
    valid = ~np.isnan(ref)
    assert np.all(body[~valid] == SENTINEL), "elements outside the ranges written"
    b = bound(q, k, k_scale, w, ks, ke, cols, ref)
    err = np.abs(body[valid] - ref[valid])
    assert np.all(err <= b[valid]), f"max err/bound = {np.max(err / b[valid]):.3g}"


def test_cpu_build_on_the_causal_request_case(host_kernel, tmp_path):
    g = workloads.mqa_logits_case(7, num_q=0, num_heads=64, num_k=0, causal_lens=[1, 70, 129, 5])
    check(host_kernel, tmp_path, g.q, g.k, g.k_scale, g.weights, g.ks, g.ke,
          int(max(g.ke - g.ks)), pad=12)


@pytest.mark.parametrize("H", [16, 48])
def test_cpu_build_on_random_ranges(host_kernel, tmp_path, H):
    g = workloads.mqa_logits_case(100 + H, num_q=37, num_heads=H, num_k=300)
    ks, ke = g.ks.copy(), g.ke.copy()
    ks[:4] = [-5, 0, 290, 100]
    ke[:4] = [20, 300, 350, 100]
    check(host_kernel, tmp_path, g.q, g.k, g.k_scale, g.weights, ks, ke, 200)


@pytest.mark.parametrize("case,needle", [("oob", "AddressSanitizer"), ("skip", "DEADLOCK")])
def test_cpu_build_reports_planted_mistakes(tmp_path, case, needle):
    """The CPU build is not blind: a lane reading past its buffer stops the
    run under AddressSanitizer, and half a wave in a cross-lane exchange while
    the other half waits at the workgroup barrier is reported as a deadlock
    (tests/cpu_build/selfcheck.cpp)."""
    clang = CLANG if os.path.exists(CLANG) else shutil.which("clang++")
    if not clang:
        pytest.skip("clang++ not available")
    exe = tmp_path / "selfcheck"
    r = subprocess.run([clang, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-pthread",
                        "-Wno-psabi", "-I", os.path.join(ROOT, "tests", "cpu_build", "shim"),
                        "-x", "c++", os.path.join(ROOT, "tests", "cpu_build", "selfcheck.cpp"),
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe), case], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, EMU_WAIT_S="2", ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode != 0 and needle in r.stderr, (r.returncode, r.stderr[-2000:])
