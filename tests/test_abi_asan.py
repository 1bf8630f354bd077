"""The C ABI's argument checks and host planning under AddressSanitizer (CPU).

Builds api.hip and plan.hip with the host side sanitized and every kernel
launcher replaced by a recording stub (tests/asan/launch_stubs.hip), links a
driver (tests/asan/abi_main.cpp) that makes rejected and accepted calls, and
runs it.  Nothing reaches a device."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_gated_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_checks_under_address_sanitizer(tmp_path):
    exe = str(tmp_path / "abi_asan")
    srcs = [os.path.join(CSRC, "api.hip"), os.path.join(CSRC, "plan.hip"),
            os.path.join(ROOT, "tests", "asan", "launch_stubs.hip"),
            os.path.join(ROOT, "tests", "asan", "abi_main.cpp")]
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *host_asan]
    objs = []
    for s in srcs:
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        lang = ["-x", "hip"] if s.endswith(".cpp") else []
        r = subprocess.run(cmd + lang + ["-c", s, "-o", o], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(o)
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *host_asan, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "abi checks ok" in r.stdout
