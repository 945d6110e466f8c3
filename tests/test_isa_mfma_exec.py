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
