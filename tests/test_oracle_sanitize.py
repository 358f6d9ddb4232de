"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sanitize_check.c calls every oracle entry point on the edge cases of the
path (queries before the start of the cache, empty sequences, lengths past the
cache capacity, fewer candidates than index_topk, skipped / repeated /
all-skipped index entries, codec special values; DeepSeek-V3.2 model
documentation, "DeepSeek Sparse Attention (DSA)", items 1 and 2).  It is built
here with gcc together with dsa_oracle.c; any sanitizer report or failed check
fails the test.  Host code only: nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ORC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_clean_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "orc_san")
    cmd = ["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-fopenmp", os.path.join(ORC, "dsa_oracle.c"),
           os.path.join(ORC, "sanitize_check.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]
    assert "all oracle entry points ran" in r.stdout
