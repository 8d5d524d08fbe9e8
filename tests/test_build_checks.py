"""The build refuses a prefill kernel that spills (CPU only).

The causal prefill waits for its direct global-to-LDS tile loads with
hand-counted s_waitcnt vmcnt(N), which is right only while those loads are
the only vector-memory operations in its loop; scratch traffic from a
register spill would break that silently.  build.check_no_scratch parses the
compiler's kernel-resource-usage remarks and raises for such a kernel.
"""
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
