"""The C ABI layer's host code (argument validation, planning arithmetic,
workspace layout) built with AddressSanitizer and UndefinedBehaviorSanitizer
and run on the CPU: the kernel launchers are replaced by recording stand-ins
(tests/asan/launch_stubs.cpp), and the driver (tests/asan/driver.cpp) checks
statuses and that every workspace address a launch would use lies inside the
workspace it sized."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_layer_under_host_sanitizers(tmp_path):
    inc = ["-I" + os.path.join(ROOT, "include")]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + SAN + inc
    srcs = [os.path.join(ROOT, "sparse_attention_07_amd", "csrc", "api.hip"),
            os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"),
            os.path.join(ROOT, "tests", "asan", "driver.cpp")]
    objs = []
    for s in srcs:
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        lang = [] if s.endswith(".hip") else ["-x", "hip"]
        r = subprocess.run([HIPCC, *flags, *lang, "-c", s, "-o", o], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(o)
    exe = str(tmp_path / "driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all checks passed" in r.stdout
