"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
block manager of the C ABI (block_manager.cpp, plain C++) and the test
oracle (oracle/oracle.c) are compiled with g++ / gcc and the sanitizers and
driven by tests/native/sanitize_driver.cpp — seeded random operation
sequences on the allocator with its invariants checked after every step, bad
arguments, and the oracle's routines on random and edge-case inputs.  Any
sanitizer report fails the run.  CPU only."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "paged_kv_cache_gather_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not shutil.which("g++") or not shutil.which("gcc"):
        pytest.skip("needs g++ and gcc")
    out = tmp_path_factory.mktemp("san")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    objs = []
    for src, cc, extra in ((os.path.join(CSRC, "block_manager.cpp"), "g++", ["-std=c++17"]),
                           (os.path.join(ROOT, "oracle", "oracle.c"), "gcc", ["-std=c11", "-fopenmp"]),
                           (os.path.join(ROOT, "tests", "native", "sanitize_driver.cpp"), "g++", ["-std=c++17"])):
        obj = str(out / (os.path.basename(src) + ".o"))
        cmd = [cc, *san, *extra, "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(out / "sanitize_driver")
    r = subprocess.run(["g++", *san, "-fopenmp", *objs, "-o", exe, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_allocator_and_oracle_under_sanitizers(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([driver, "40"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert "passed" in r.stdout
