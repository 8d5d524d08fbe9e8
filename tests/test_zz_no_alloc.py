"""attn_sinks_decode_noalloc: the decode with its partial results in the
library's fixed per-GPU scratch instead of a caller workspace.

Its output must be bit-identical to attn_sinks_decode_window's (the same
kernels on the same inputs) and within the bar of the fp64 oracle.  Two
calls in a row, the second with a smaller input, check that nothing of the
first call's scratch contents leaks into the second; a third call exercises
the windowed split path.
"""
import pytest
import torch

import gqa_paged_attention_amd as ga
from gqa_paged_attention_amd import workloads as wl

from .gpu_helpers import compare, note, oracle_full, require_gpu, run_decode

pytestmark = pytest.mark.gpu


def _noalloc(batch_cpu, window=0):
    require_gpu()
    g = batch_cpu.to("cuda")
    out = torch.full_like(g.q, float("nan"))
    ga.attn_sinks_decode_noalloc(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.sinks,
                                 g.scale, window, out, batch_cpu.max_seq_len)
    torch.cuda.synchronize()
    return out.cpu()


def _same_bits(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{what}: bits differ"
    note(f"  {what}: bit-identical")


def test_noalloc_two_calls_then_window():
    big = wl.gptoss_decode(0)
    note("noalloc: gpt-oss decode workload (64 seqs, 64/8 heads, d 64)")
    got = _noalloc(big)
    _same_bits(got, run_decode(big), "noalloc vs attn_sinks_decode, gpt-oss decode")
    compare(got, oracle_full(big), "bf16", "noalloc vs oracle, gpt-oss decode")

    small = wl.small_batch(7, "bf16", [600, 1, 1500, 33, 4097], [1] * 5, 16, 2, 128,
                           sink_mode="normal")
    note("noalloc: second, smaller call (5 seqs, 16/2 heads, d 128, one of length 1)")
    got = _noalloc(small)
    _same_bits(got, run_decode(small), "noalloc vs attn_sinks_decode, smaller call")
    compare(got, oracle_full(small), "bf16", "noalloc vs oracle, smaller call")

    note("noalloc: gpt-oss decode workload, window 1000 (split path)")
    got = _noalloc(big, window=1000)
    _same_bits(got, run_decode(big, window=1000), "noalloc vs attn_sinks_decode_window")
    compare(got, oracle_full(big, window=1000), "bf16", "noalloc vs oracle, window 1000")


def test_noalloc_rejects_beyond_scratch():
    require_gpu()
    # 2000 sequences at 64/8 heads, d 64, need more than the 32 MiB scratch
    need = ga.attn_sinks_decode_workspace_bytes(2000, 64, 8, 64, 8192)
    assert need > 32 << 20
    q = torch.zeros(2000, 64, 64, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(1, 8, 16, 64, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(2000, 512, dtype=torch.int32, device="cuda")
    sl = torch.ones(2000, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(ga.AttnSinksError) as e:
        ga.attn_sinks_decode_noalloc(q, kc, kc, bt, sl, None, 0.125, 0, out, 8192)
    assert e.value.status == 7
