"""The prefill's kernel variants give the same bits.

With a group size divisible by 4 a prefill workgroup takes the same rows
of four query heads (head_dim 64 and 128); the debug settings give each workgroup
one head instead (ATTN_DEBUG_PREFILL_ONE_HEAD) and make every tile wait
take all loads in flight (ATTN_DEBUG_PREFILL_WAIT_ALL).  The per-row
arithmetic is the same in all of them, so their outputs must be
bit-identical; the wait-all variant
also guards the hand-counted waits of the direct K/V tile loads (a load the
count missed would let a wave read a stage before it lands, which the
variant that waits for everything cannot do).  Each case is also checked
against the oracle.
"""
import pytest
import torch

import gqa_paged_attention_amd as ga
from gqa_paged_attention_amd import workloads as wl
from tests.gpu_helpers import (check_sampled, compare, note, oracle_full, require_gpu,
                               run_prefill, scale_keys)
from tests.test_gpu_ragged import run_ragged

pytestmark = pytest.mark.gpu

VARIANTS = {
    "four heads": (0, 0),
    "four heads, wait all": (0, 1),
    "one head": (1, 0),
    "one head, wait all": (1, 1),
}


def _each_variant(fn):
    require_gpu()
    outs = {}
    try:
        for name, (one_head, wait_all) in VARIANTS.items():
            ga.attn_sinks_set_debug(ga.ATTN_DEBUG_PREFILL_ONE_HEAD, one_head)
            ga.attn_sinks_set_debug(ga.ATTN_DEBUG_PREFILL_WAIT_ALL, wait_all)
            outs[name] = fn()
    finally:
        ga.attn_sinks_set_debug(ga.ATTN_DEBUG_PREFILL_ONE_HEAD, 0)
        ga.attn_sinks_set_debug(ga.ATTN_DEBUG_PREFILL_WAIT_ALL, 0)
    base = outs["four heads"]
    for name, o in outs.items():
        assert torch.equal(o.view(torch.int16), base.view(torch.int16)), \
            f"{name} differs from the default"
    note(f"  {len(outs)} variants bit-identical")
    return base


CASES = [
    # id, seq_lens, q_lens, Hq, Hkv
    ("causal_ragged", [1, 17, 130, 300, 600, 1000], [1, 17, 130, 300, 600, 1000], 16, 2),
    ("chunks_over_prefix", [500, 1000, 64, 3000], [100, 257, 1, 700], 16, 2),
    ("one_tile_many_heads", [256, 255, 257], [256, 255, 257], 64, 8),
    ("group_2_one_head_only", [900, 40], [900, 40], 4, 2),
    ("group_16", [700, 129], [300, 129], 32, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_variants_bit_identical(case):
    name, L, Lq, Hq, Hkv = case
    b = wl.small_batch(len(name) * 7 + 3, "bf16", L, Lq, Hq, Hkv, 64, sink_mode="normal")
    note(f"prefill variants {name}: L={L} Lq={Lq} Hq={Hq} Hkv={Hkv}")
    out = _each_variant(lambda: run_prefill(b))
    compare(out, oracle_full(b), "bf16", f"prefill {name}")


def test_prefill_variants_exact_recompute():
    # late keys far above early ones: rows go through the exact recompute
    b = wl.small_batch(77, "bf16", [700, 300], [190, 300], 16, 2, 64)
    b = scale_keys(b, 64, 100.0)
    note("prefill variants, large late logits")
    out = _each_variant(lambda: run_prefill(b))
    compare(out, oracle_full(b), "bf16", "prefill variants large late logits")


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "unmasked"])
def test_ragged_variants_bit_identical(causal):
    r = wl.ragged_batch(91 + int(causal), "bf16", [300, 1000, 17], [300, 1000, 17], 16, 2, 64)
    note(f"ragged variants causal={causal}")
    out = _each_variant(lambda: run_ragged(r, causal, with_lse=False)[0])
    compare(out, oracle_full(r.paged) if causal else
            __import__("oracle").attention(r.paged, threads=16, causal=False), "bf16",
            f"ragged variants causal={causal}")


def test_full_gptoss_prefill_variants():
    pre = wl.gptoss_prefill(0)
    note("full gpt-oss prefill, every variant")
    out = _each_variant(lambda: run_prefill(pre))
    check_sampled(out, pre, 256, seed=5, what="gpt-oss prefill, variants")


@pytest.mark.parametrize("hkv", [4, 2], ids=["group_4", "group_16"])
def test_prefill_d128_variants_bit_identical(hkv):
    # head_dim 128: 32 rows of four heads per workgroup or 128 rows of one,
    # 4 loads per tile and wave; chunks over prefixes and a ragged tail
    b = wl.small_batch(131 + hkv, "bf16", [700, 129, 1000, 45], [300, 129, 1000, 45], 32, hkv,
                       128, sink_mode="normal")
    note(f"prefill d=128 variants, Hq=32 Hkv={hkv}")
    out = _each_variant(lambda: run_prefill(b))
    compare(out, oracle_full(b), "bf16", f"prefill d=128 variants Hkv={hkv}")


def test_ragged_d128_variants_bit_identical():
    r = wl.ragged_batch(97, "bf16", [300, 1000, 17], [300, 1000, 17], 16, 4, 128)
    note("ragged d=128 variants, causal")
    out = _each_variant(lambda: run_ragged(r, True, with_lse=False)[0])
    compare(out, oracle_full(r.paged), "bf16", "ragged d=128 variants")
