"""Checks on the generated gfx950 code of the attention kernels (CPU: compile only).

The wide sparse-MLA kernel issues its LDS-DMA copies as inline asm that sets M0 itself; M0 is a
reserved register the compiler does not let asm clobber, so the copies are correct only while
the compiler makes no other use of M0 in those kernels.  This compiles the source to gfx950
assembly and checks every instance of the kernel."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_06_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_wide_mla_kernels_use_m0_only_in_their_copy_asm(tmp_path):
    out = tmp_path / "sparse_mla.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "sparse_mla.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    lines = out.read_text().split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"_ZN3dsa12_GLOBAL__N_115mla_wide_kernel\S*:", l)]
    assert len(starts) >= 10, "every instance of the wide kernel is compiled"
    for i in starts:
        j = i
        while not lines[j].startswith(".Lfunc_end"):
            j += 1
        in_asm, copies = False, 0
        for l in lines[i:j]:
            t = l.strip()
            if t.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if t.startswith(";;#ASMEND"):
                in_asm = False
                continue
            code = t.split(";")[0]
            if in_asm:
                copies += "global_load_lds_dwordx4" in code
            else:
                assert not re.search(r"\bm0\b", code), f"{lines[i][:60]}: compiler uses M0: {t}"
        assert copies > 0
