"""Static checks on the gfx950 assembly of this repository's own kernels (CPU only, needs hipcc).

A DPP lane exchange executed while some lanes are switched off by the exec mask reads zeros (or
stale values) from the disabled lanes.  Every cross-lane reduction in the attention kernels must
therefore run with the whole wavefront active; this test fails if the compiler (or a careless
ternary around a reduction) places a DPP instruction inside an exec-masked region.
"""

import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_kvcache_amd import build as B

hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(hipcc), reason="hipcc not available")


def _asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [hipcc, *[f for f in B.FLAGS if f != "-fPIC"], "-S", "--cuda-device-only", src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _dpp_inside_exec_masked_regions(asm, kernel_pattern):
    found = {}
    name, depth = None, 0
    for ln in asm.split("\n"):
        m = re.match(r"^(_Z\w+):", ln)
        if m:
            name = m.group(1) if re.search(kernel_pattern, m.group(1)) else None
            depth = 0
            if name:
                found[name] = 0
            continue
        if name is None:
            continue
        if "s_and_saveexec" in ln:
            depth += 1
        if re.search(r"s_or_b64 exec, exec", ln):
            depth = max(0, depth - 1)
        if "_dpp" in ln and depth > 0:
            found[name] += 1
        if "s_endpgm" in ln:
            name = None
    return found


def test_decode_reductions_run_with_full_exec(tmp_path):
    asm = _asm(os.path.join(B.CSRC, "decode.hip"), tmp_path)
    found = _dpp_inside_exec_masked_regions(asm, "decode_split_kernel")
    assert len(found) == 24  # 3 dtypes x 2 head dims x 4 group sizes
    bad = {k: v for k, v in found.items() if v}
    assert not bad, f"DPP inside exec-masked code: {bad}"
