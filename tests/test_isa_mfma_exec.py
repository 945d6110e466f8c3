"""The compiled gfx950 kernels never reach a matrix-core instruction with an
empty EXEC mask (MFMA ignores EXEC, so such an instruction would add garbage
to an accumulator), and none uses scratch memory (register spills).
Compiles every HIP source to assembly with hipcc."""
import shutil

import pytest

from ulysses_sequence_parallelism_head_amd import isa_check


def test_scanner_flags_unskipped_mfma():
    asm = "\n".join([
        "kern:",
        "\ts_and_saveexec_b64 s[0:1], s[8:9]",
        "; %bb.70:",
        "\tv_mfma_f32_32x32x16_bf16 v[66:81], v[18:21], v[56:59], v[66:81]",
        "\ts_or_b64 exec, exec, s[0:1]",
        "\ts_and_saveexec_b64 s[2:3], vcc",
        "\ts_cbranch_execz .LBB0_2",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
        ".LBB0_2:",
        "\ts_endpgm",
    ])
    bad = isa_check.scan(asm)
    assert len(bad) == 1 and bad[0][1] == 4


def test_scanner_follows_fall_through_and_scalar_branches():
    """An MFMA reached through a labelled fall-through block, a branch on
    SCC, an unconditional branch, or the taken side of s_cbranch_execz is
    flagged; one behind s_cbranch_execz's fall-through or after the EXEC
    restore is not."""
    asm = "\n".join([
        "kern:",
        "\ts_and_saveexec_b64 s[0:1], vcc",               # 2
        "\ts_cmp_eq_u32 s4, 0",
        "\ts_cbranch_scc1 .LBB0_3",                        # 4: both ways
        ".LBB0_1:",                                        # fall-through into a label
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",   # 6: flagged
        "\ts_branch .LBB0_4",
        ".LBB0_3:",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",   # 9: flagged (SCC taken)
        ".LBB0_4:",
        "\ts_or_b64 exec, exec, s[0:1]",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",   # 12: EXEC restored
        "\ts_and_saveexec_b64 s[2:3], vcc",
        "\ts_cbranch_execz .LBB0_6",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",   # 15: EXEC non-empty here
        "\ts_or_b64 exec, exec, s[2:3]",
        "\ts_endpgm",
        ".LBB0_6:",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",   # 19: flagged (EXEC empty)
        "\ts_or_b64 exec, exec, s[2:3]",
        "\ts_endpgm",
    ])
    assert [b[1] for b in isa_check.scan(asm)] == [6, 9, 19]


def test_scratch_parser():
    asm = "\n".join([
        "\t.amdhsa_kernel kern_a",
        "\t\t.amdhsa_private_segment_fixed_size 0",
        "\t.end_amdhsa_kernel",
        "\t.amdhsa_kernel kern_b",
        "\t\t.amdhsa_private_segment_fixed_size 28",
        "\t.end_amdhsa_kernel",
    ])
    assert isa_check.scratch_kernels(asm) == [("kern_b", 28)]


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists(isa_check.HIPCC),
                    reason="hipcc not available")
def test_no_mfma_reachable_with_empty_exec():
    assert isa_check.check(verbose=False) == []
