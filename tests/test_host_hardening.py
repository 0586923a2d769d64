"""The C ABI's host code (argument checks, size arithmetic, error
propagation) built with the address and undefined-behaviour sanitizers and
run without a GPU: tests/host/host_checks.cpp calls every entry point with
every argument the header rejects, with token counts whose sizes would
overflow, and with HIP runtime calls and kernel launches that fail (a faked
runtime, tests/host/fake_hip.cpp, injects the errors), and checks the status
codes and sparse_ffn_last_error()."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.fixture(scope="module")
def host_checks(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang++ not available")
    out = tmp_path_factory.mktemp("host_checks")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "activation_sparse_ffn_amd", "csrc")]
    srcs = [os.path.join(ROOT, "activation_sparse_ffn_amd", "csrc", "capi.cpp"),
            os.path.join(ROOT, "tests", "host", "fake_hip.cpp"),
            os.path.join(ROOT, "tests", "host", "host_checks.cpp")]
    objs = []
    for src in srcs:
        obj = str(out / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-w", *SAN, *inc, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    # the host objects name a device code object that is not built here
    undef = subprocess.run(["nm", "-u", objs[0]], capture_output=True, text=True, check=True).stdout
    fatbins = sorted(set(re.findall(r"\b(__hip_fatbin\w*)", undef)))
    exe = str(out / "host_checks")
    cmd = [CLANG, "-fsanitize=address,undefined", "-g", *objs, "-o", exe, "-lpthread",
           *[f"-Wl,--defsym,{f}=fake_fatbin" for f in fatbins]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_every_rejection_and_hip_error_under_sanitizers(host_checks):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([host_checks], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
