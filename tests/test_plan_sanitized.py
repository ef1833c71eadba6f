"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

pic_plan.cpp is plain host C++ (integer index and schedule arithmetic), so it is built
on its own with g++ -fsanitize=address,undefined into a planner-only library, and
tests/plan_sanitized_driver.py runs the planner checks of test_abi_and_plan.py against
it (worked example, exhaustive small grids, error paths, the 32k and EPIC-scale
batches, paged plans, and hypothesis searches) in a child process with the sanitizer
runtimes preloaded.  Any report (out-of-bounds access, use after free, signed
overflow, bad shift, ...) ends the child with a non-zero status.
"""

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "position_independent_kv_rope_amd", "csrc")


def test_planner_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    lib = str(tmp_path / "libpic_plan_san.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared", "-fPIC",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "pic_plan.cpp"), "-o", lib]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    rt = [subprocess.check_output([gxx, "-print-file-name=lib%s.so" % n], text=True).strip()
          for n in ("asan", "ubsan")]
    env = dict(os.environ)
    env.update(LD_PRELOAD=":".join(rt),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24",
               PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, os.path.join(HERE, "plan_sanitized_driver.py"), lib],
                       env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.returncode, r.stdout[-4000:], r.stderr[-4000:])
    assert "sanitized planner: ok" in r.stdout
