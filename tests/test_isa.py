"""Static checks on the gfx950 code of the LDS-DMA ring kernels (CPU only).

The ring GEMM and ring attention kernels issue their global -> LDS copies from
inline assembly that writes M0 (the copy's LDS address).  M0 is a reserved
register the compiler does not save around an asm statement, so the kernels are
only correct while the compiler itself keeps nothing in M0: every M0 reference
in their code must be one of those writes, each followed by its wait state and
its copy.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _ring_bodies(tmp_path, source, kernel):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / (source + ".s")
    src = os.path.join(ROOT, "drafting_draft_expand_amd", "csrc", source)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S", "-o", str(out), src]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    bodies = {}
    # the whole function, up to its end label: the compiler may place blocks
    # (copies included) after an s_endpgm
    for m in re.finditer(r"^(_Z\S*" + kernel + r"\S*):.*?\n(.*?)^\.Lfunc_end", text, re.S | re.M):
        bodies[m.group(1)] = [ln.strip() for ln in m.group(2).split("\n")
                              if ln.strip() and not ln.strip().startswith(";")]
    return bodies


@pytest.mark.parametrize("source,kernel", [("gemm.hip", "gemm_ring_kernel"), ("attention.hip", "attn_ring_kernel")])
def test_ring_kernels_use_m0_only_for_their_copies(tmp_path, source, kernel):
    bodies = _ring_bodies(tmp_path, source, kernel)
    assert bodies, "no ring kernel instantiated"
    for name, lines in bodies.items():
        writes = copies = 0
        for i, ln in enumerate(lines):
            if re.search(r"\bm0\b", ln):
                assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), f"{name}: unexpected M0 use: {ln}"
                assert lines[i + 1] == "s_nop 0", f"{name}: no wait state after {ln}"
                assert lines[i + 2].startswith("global_load_lds_dwordx4"), f"{name}: M0 write not followed by a copy"
                writes += 1
            if ln.startswith("global_load_lds_dwordx4"):
                copies += 1
        assert writes == copies > 0, f"{name}: {writes} M0 writes for {copies} copies"
