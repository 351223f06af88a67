"""The host control plane under AddressSanitizer and UndefinedBehaviorSanitizer.

host.cpp is compiled with g++ (host code only; the kernel launchers are
replaced by stubs that do nothing) and driven through the C ABI by random
Reserve / Trim / plan / train queries, including invalid slots and
capacities.  Runs on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")


def _rocm_include():
    for d in ("/opt/rocm/include",):
        if os.path.exists(os.path.join(d, "hip", "hip_runtime.h")):
            return d
    return None


@pytest.mark.skipif(shutil.which("g++") is None or _rocm_include() is None,
                    reason="needs g++ and the HIP headers")
def test_host_plane_is_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "pager_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", _rocm_include(),
           os.path.join(ROOT, "non_uniform_paged_amd", "csrc", "host.cpp"),
           os.path.join(NATIVE, "launch_stubs.cpp"), os.path.join(NATIVE, "pager_fuzz.cpp"),
           "-o", exe, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    for seed in (1, 2, 3):
        r = subprocess.run([exe, str(seed)], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.startswith("ok"), r.stdout
