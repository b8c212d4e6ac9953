"""The split planner (api.cpp) built for the host with the address and undefined-behaviour
sanitizers, driven by randomised valid and malformed arguments (tests/sanitize/
planner_fuzz.cpp): every call must return a status without an out-of-bounds access or
undefined arithmetic, and every accepted plan must cover each request's visible tokens
exactly once per KV head and query-block group.  Host compiler only; no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_split_kv_stage1_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP runtime headers")
def test_planner_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "planner_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(ROOT, "tests", "sanitize", "planner_fuzz.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "device_stubs.cpp"), os.path.join(CSRC, "api.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    for seed in ("1", "20240611"):
        r = subprocess.run([exe, "1500", seed], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0 and "0 failures" in r.stdout, (r.stdout[-2000:], r.stderr[-3000:])
