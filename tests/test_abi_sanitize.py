"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled with the sanitizers on for their host code
(the device code is built as usual; nothing here launches a kernel), and tests/abi_sanitize_check.cpp
drives every workspace-size query and every host-side rejection path over valid,
edge and near-int32-limit shapes.  Any sanitizer report or failed check fails the
test.  Host code only: nothing here touches a GPU.
"""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_09_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# the sanitizers apply to host code only (-Xarch_host before each of them)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_host_code_clean_under_address_and_ub_sanitizers(tmp_path):
    common = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", *SAN,
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([*common, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(ROOT, "tests", "abi_sanitize_check.cpp")]
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_san")
    r = subprocess.run([*common, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]
    assert "abi host checks ran" in r.stdout
