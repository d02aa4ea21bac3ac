"""Checks on the gfx950 assembly of the attention and gather kernels (CPU only).

The gathers replace a tile's padding entries by the slot of its first row,
read from lane 0 with readfirstlane.  That read must run with every lane of
the wave active: under a mask of only the padding lanes it returns a padding
entry (-1) and the gather addresses a row before the cache.  This compiles
the kernels to assembly and checks that no readfirstlane in them sits inside
an exec-mask region opened by s_and_saveexec.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "top_sparse_attention_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "qsa_attend.s"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, "qsa_attend.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    funcs, cur = {}, None
    for line in out.read_text().splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
        elif cur:
            funcs[cur].append(line.strip())
    return funcs


def test_lane0_reads_run_with_the_full_wave(kernel_asm):
    checked = 0
    for name, body in kernel_asm.items():
        if "attend_kernel" not in name and "gather_only_kernel" not in name:
            continue
        checked += 1
        depth = 0
        for ins in body:
            if ins.startswith("s_and_saveexec"):
                depth += 1
            elif ins.startswith("s_or_b64 exec") and depth:
                depth -= 1
            elif ins.startswith("v_readfirstlane"):
                assert depth == 0, f"{name}: readfirstlane under a partial exec mask"
    assert checked >= 8     # split and non-split, BF16 and FP8, both layouts, gather-only
