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
    """Per kernel, the DPP instructions that lie (in text order) inside a region opened by
    s_and_saveexec into some register pair and not yet closed by s_or_b64 exec, exec with that pair.
    Several branches may save into the same pair and rejoin at one restore, which closes them all;
    an if/else moves the saved mask to another pair (s_xor_b64 new, exec, old) before its restore."""
    found = {}
    name, open_pairs = None, []
    for ln in asm.split("\n"):
        m = re.match(r"^(_Z\w+):", ln)
        if m:
            name = m.group(1) if re.search(kernel_pattern, m.group(1)) else None
            open_pairs = []
            if name:
                found[name] = 0
            continue
        if name is None:
            continue
        m = re.search(r"s_and_saveexec_b64 (s\[\d+:\d+\])", ln)
        if m:
            open_pairs.append(m.group(1))
        m = re.search(r"s_xor_b64 (s\[\d+:\d+\]), exec, (s\[\d+:\d+\])", ln)  # if/else: the mask moves
        if m:
            open_pairs = [m.group(1) if p == m.group(2) else p for p in open_pairs]
        m = re.search(r"s_or_b64 exec, exec, (s\[\d+:\d+\])", ln)
        if m:
            open_pairs = [p for p in open_pairs if p != m.group(1)]
        if "_dpp" in ln and open_pairs:
            found[name] += 1
        if "s_endpgm" in ln:
            name = None
    return found


def test_decode_reductions_run_with_full_exec(tmp_path):
    asm = _asm(os.path.join(B.CSRC, "decode.hip"), tmp_path)
    found = _dpp_inside_exec_masked_regions(asm, "decode_split_kernel")
    # 3 dtypes x 2 head dims x 4 group sizes, each with and without device-data checks
    assert len(found) == 48
    bad = {k: v for k, v in found.items() if v}
    assert not bad, f"DPP inside exec-masked code: {bad}"


def test_exec_region_scan_on_hand_written_snippets():
    """The scan itself: a DPP between s_and_saveexec and its restore is flagged; branches that share
    one restore, and an if/else whose mask moves to another pair, close their regions."""
    masked = "_Za:\n s_and_saveexec_b64 s[4:5], vcc\n v_add_f32_dpp v1, v2, v3\n s_or_b64 exec, exec, s[4:5]\n s_endpgm\n"
    shared = ("_Zb:\n s_and_saveexec_b64 s[4:5], vcc\n s_cbranch_execnz .L1\n s_and_saveexec_b64 s[4:5], s[8:9]\n"
              ".L1:\n s_or_b64 exec, exec, s[4:5]\n v_add_f32_dpp v1, v2, v3\n s_endpgm\n")
    if_else = ("_Zc:\n s_and_saveexec_b64 s[60:61], s[8:9]\n s_xor_b64 s[8:9], exec, s[60:61]\n"
               " s_or_saveexec_b64 s[8:9], s[8:9]\n s_xor_b64 exec, exec, s[8:9]\n s_or_b64 exec, exec, s[8:9]\n"
               " v_add_f32_dpp v1, v2, v3\n s_endpgm\n")
    assert _dpp_inside_exec_masked_regions(masked, "_Za") == {"_Za": 1}
    assert _dpp_inside_exec_masked_regions(shared, "_Zb") == {"_Zb": 0}
    assert _dpp_inside_exec_masked_regions(if_else, "_Zc") == {"_Zc": 0}
