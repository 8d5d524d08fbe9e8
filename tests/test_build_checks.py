"""Checks on the compiled prefill kernels (CPU only).

The causal prefill waits for its direct global-to-LDS tile loads with
hand-counted s_waitcnt vmcnt(N), which is right only while those loads are
the only vector-memory operations in its loop; scratch traffic from a
register spill would break that silently.  build.check_no_scratch parses the
compiler's kernel-resource-usage remarks and raises for such a kernel.

Those loads are inline assembly, which the compiler's hazard checks do not
look into: build.check_dma_hazards finds a load whose scalar base registers a
vector instruction (a spill restore, say) wrote fewer than the five wait
states the hardware needs before a vector-memory read; the prefill source is
compiled to gfx950 assembly and checked.
"""
import os
import subprocess

import pytest

from gqa_paged_attention_amd import build as B

NAME = "_ZN4attn12_GLOBAL__N_112prefill_bf16ILi64ELb0ELb0ELi4EEEvNS0_11PrefillArgsE"


def _remarks(name, scratch):
    return (f"x.hip:1:1: remark: Function Name: {name} [-Rpass-analysis=kernel-resource-usage]\n"
            f"x.hip:1:1: remark:     VGPRs: 250 [-Rpass-analysis=kernel-resource-usage]\n"
            f"x.hip:1:1: remark:     ScratchSize [bytes/lane]: {scratch} "
            f"[-Rpass-analysis=kernel-resource-usage]\n")


def test_prefill_kernel_with_scratch_is_refused():
    with pytest.raises(RuntimeError, match="scratch"):
        B.check_no_scratch(_remarks(NAME, 16), "prefill.hip")


def test_prefill_kernel_without_scratch_passes():
    B.check_no_scratch(_remarks(NAME, 0), "prefill.hip")


def test_other_kernels_may_spill():
    # the decode kernels' loads are waited for by the compiler itself
    B.check_no_scratch(_remarks("_ZN4attn12_GLOBAL__N_117decode_split_bf16ILi64ELi4EEEvNS0_9SplitArgsE",
                                20), "decode.hip")


LOAD = "\ts_nop 4\n\tglobal_load_lds_dwordx4 v196, s[8:9]\n"


def test_dma_hazard_is_found():
    asm = "\tv_readlane_b32 s9, v230, 42\n\t;;#ASMSTART\n\ts_nop 0\n" \
          "\tglobal_load_lds_dwordx4 v196, s[8:9]\n"
    with pytest.raises(RuntimeError, match="s9"):
        B.check_dma_hazards(asm)


def test_dma_with_enough_wait_states_passes():
    asm = "\tv_readlane_b32 s8, v230, 41\n\tv_readlane_b32 s9, v230, 42\n" + LOAD
    assert B.check_dma_hazards(asm) == 1
    # other registers, or writes far enough back, are fine
    asm = "\tv_readlane_b32 s10, v230, 41\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v1, s[8:9]\n"
    assert B.check_dma_hazards(asm) == 1


@pytest.mark.skipif(not os.path.exists(B.hipcc()), reason="hipcc is not available")
def test_compiled_prefill_has_no_dma_hazard(tmp_path):
    out = tmp_path / "prefill.s"
    cmd = [B.hipcc(), *B.COMMON_FLAGS, "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(B.CSRC, "prefill.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    assert B.check_dma_hazards(out.read_text()) > 100
