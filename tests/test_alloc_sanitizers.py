"""The host block manager under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/alloc_stress.cpp drives the block manager's C ABI through seeded random operation sequences
(admission with shared prefixes, appends, copy-on-write batches, forks, frees, metadata, error
paths, forced hash collisions) and checks the state the ABI exposes after every operation.  Here it
is built from the library's own allocator sources with the sanitizers and run; any memory error,
leak or undefined behaviour aborts it.
"""

import os
import shutil
import subprocess

import pytest

from paged_kv_cache_kvcache_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
gxx = shutil.which("g++")


@pytest.mark.skipif(gxx is None, reason="g++ not available")
def test_block_manager_under_sanitizers(tmp_path):
    exe = str(tmp_path / "alloc_stress")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{B.INCLUDE}", f"-I{B.CSRC}", os.path.join(B.CSRC, "alloc.cpp"),
           os.path.join(B.CSRC, "errors.cpp"), os.path.join(HERE, "alloc_stress.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "6", "1500"], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-1000:] + r.stderr[-3000:]
    assert "checks passed" in r.stdout
