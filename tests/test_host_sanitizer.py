"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

attn_api.cpp (the C ABI: validation, workspace and scratch handling) and
attn_host.cpp (the tile planner) are compiled with g++ -fsanitize=address,
undefined against the stub HIP runtime of tests/sanitizer, without any GPU
code. A child pytest then runs the ABI suite (no device: every valid call
ends in a device error) and the simulated-device cases (host buffers of the
documented sizes; the stub launchers touch every byte the kernels would) with
the binding pointed at that build. Any sanitizer report aborts the child."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "efficient_exact_attention_amd", "csrc")
STUB = os.path.join(ROOT, "tests", "sanitizer")


def _libasan():
    if not shutil.which("g++"):
        return None
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitizer_lib(tmp_path_factory):
    if _libasan() is None:
        pytest.skip("g++ with libasan is not available")
    out = str(tmp_path_factory.mktemp("asan") / "libattn_host_asan.so")
    cmd = ["g++", "-std=c++17", "-fPIC", "-shared", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
           f"-I{STUB}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "attn_api.cpp"), os.path.join(CSRC, "attn_host.cpp"),
           os.path.join(STUB, "hip_stub.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def test_host_code_is_clean_under_asan_and_ubsan(sanitizer_lib, tmp_path):
    env = dict(os.environ)
    env.update(EEA_SANITIZER_LIB=sanitizer_lib, LD_PRELOAD=_libasan(),
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={tmp_path}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan",
               PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(STUB, "simulated_device_cases.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = ""
    for name in sorted(os.listdir(tmp_path)):
        if name.startswith(("asan", "ubsan")):
            with open(os.path.join(tmp_path, name)) as f:
                reports += f.read()
    assert r.returncode == 0 and not reports, (r.stdout[-4000:] + r.stderr[-2000:] + reports[:6000])
    # both files ran, nothing was skipped for want of the sanitizer build
    assert " passed" in r.stdout and "skipped" not in r.stdout, r.stdout[-2000:]
