"""The forward's gfx950 assembly is free of the spill-before-exec-restore
miscompile (a register spill stored under the partial exec of the divergent
region just left; see mamba_ssd_chunked_04_amd/asmcheck.py).  CPU only:
compiles the three forward translation units to assembly (about a minute).
"""
import shutil

import pytest

from mamba_ssd_chunked_04_amd import asmcheck


def test_detector_finds_the_pattern():
    asm = "\n".join([
        "_Zkernel:  ; @_Zkernel",
        "\ts_and_saveexec_b64 s[18:19], s[8:9]",
        "\tds_write_b32 v1, v2",
        ".LBB0_71:",
        "\tscratch_store_dwordx2 off, v[6:7], off",
        "\ts_or_b64 exec, exec, s[18:19]",
        "\tscratch_load_dwordx2 v[0:1], off, off",
        ".Lfunc_end0:",
        "_Zclean:  ; @_Zclean",
        ".LBB1_3:",
        "\ts_or_b64 exec, exec, s[4:5]",
        "\tscratch_store_dword off, v5, off offset:8",
        ".Lfunc_end1:",
    ])
    assert asmcheck.spills_before_exec_restore(asm) == [("_Zkernel", 1)]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_forward_assembly_is_clean():
    bad = asmcheck.check_forward()
    assert bad == [], f"spill stores before an exec restore: {bad}"
