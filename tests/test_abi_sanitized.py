"""The library's host ABI (pkv_abi.cpp) built with the address and undefined-behaviour sanitizers
against a host-only fake of the HIP runtime and stub kernel launchers (tests/native/), then run:
every entry point's argument errors and status codes, nothing enqueued by a call that fails
validation, PKV_E_NOMEM with nothing left allocated when any allocation of paged_kv_alloc fails
(pool capacity beyond the device, each allocation in turn, the PKV_FAIL_HOST_ALLOC injection of a
failed pinned-host allocation), and the page free list. CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_checks")
    srcs = [os.path.join(ROOT, "paged_kv_cache_fwd_amd", "csrc", "pkv_abi.cpp"),
            os.path.join(NATIVE, "fake_hip.cpp"), os.path.join(NATIVE, "stub_launch.cpp"),
            os.path.join(NATIVE, "abi_checks.cpp")]
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"), *srcs,
           "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("PKV_FAIL_HOST_ALLOC", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert " 0 failed" in r.stdout
