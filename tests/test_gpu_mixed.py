"""attn_sinks_mixed: single-token decodes and prefill chunks of one batch.

Its result must equal, bit for bit, attn_sinks_decode over the decode
sequences followed by attn_sinks_prefill over the chunks (the header's
definition), whichever route it takes (one launch, or the two calls); those
two calls are checked against the oracle in test_gpu_parity.py, and the small
batches here are checked against the oracle as well.
"""
import pytest
import torch

import gqa_paged_attention_amd as ga
from gqa_paged_attention_amd import workloads as wl

from .gpu_helpers import check_sampled, compare, note, oracle_full

pytestmark = pytest.mark.gpu


def _mixed(full_cpu, nd, ws_extra=0):
    """attn_sinks_mixed over the whole batch; returns out on the CPU."""
    g = full_cpu.to("cuda")
    out = torch.full_like(g.q, float("nan"))
    dec_max = int(full_cpu.seq_lens[:nd].max()) if nd else 0
    pre_lens = full_cpu.seq_lens[nd:]
    q_lens = (full_cpu.cu_seqlens_q[nd + 1:] - full_cpu.cu_seqlens_q[nd:-1])
    max_q = int(q_lens.max()) if q_lens.numel() else 0
    max_l = int(pre_lens.max()) if pre_lens.numel() else 0
    nbytes = ga.attn_sinks_decode_workspace_bytes(nd, full_cpu.num_q_heads,
                                                  full_cpu.num_kv_heads, full_cpu.head_dim,
                                                  dec_max)
    ws = torch.empty(nbytes + ws_extra, dtype=torch.uint8, device="cuda")
    ga.attn_sinks_mixed(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.cu_seqlens_q,
                        g.sinks, g.scale, out, nd, dec_max, max_q, max_l, ws)
    torch.cuda.synchronize()
    return out.cpu()


def _separate(full_cpu, nd):
    """The definition: attn_sinks_decode on the first nd sequences, then
    attn_sinks_prefill on the rest."""
    parts = []
    if nd:
        dec = full_cpu.rows(0, nd)
        gd = dec.to("cuda")
        out_d = torch.empty_like(gd.q)
        nbytes = ga.attn_sinks_decode_workspace_bytes(nd, dec.num_q_heads, dec.num_kv_heads,
                                                      dec.head_dim, dec.max_seq_len)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ga.decode_batch(gd, out_d, ws)
        parts.append(out_d)
    if nd < full_cpu.num_seqs:
        pre = full_cpu.rows(nd, full_cpu.num_seqs)
        gp = pre.to("cuda")
        out_p = torch.empty_like(gp.q)
        ga.prefill_batch(gp, out_p)
        parts.append(out_p)
    torch.cuda.synchronize()
    return torch.cat([p.cpu() for p in parts])


def test_full_mixed_one_launch_equals_the_two_calls():
    note("mixed call: the full mixed workload (32 decodes, 2 chunks of 2048)")
    full, dec, pre = wl.mixed(0)
    got = _mixed(full, 32)
    want = _separate(full, 32)
    assert torch.equal(got, want), "mixed call differs from decode + prefill"
    note("mixed call: oracle on every decode row and sampled prefill rows")
    compare(got[:32], oracle_full(dec), "bf16", "mixed call, decode rows")
    check_sampled(got[32:], pre, 256, 11, "mixed call, prefill rows (256 sampled)")


# (16, 2) and (4, 1): split workgroups with fewer KV heads than waves, whose
# spare waves return at once beside the prefill's workgroups
@pytest.mark.parametrize("hq,hkv,d", [(64, 4, 128), (16, 8, 64), (32, 8, 64), (16, 2, 64),
                                      (4, 1, 128)])
def test_small_mixed_against_oracle(hq, hkv, d):
    note(f"mixed call: small batch hq={hq} hkv={hkv} d={d}")
    # three decodes past the direct pass's bound (the one-launch route), then
    # chunks over a prefix, a whole sequence and a chunk ending on a page edge
    lens = [700, 1303, 2100, 900, 1000, 512]
    q_lens = [1, 1, 1, 900, 300, 17]
    b = wl.small_batch(3, "bf16", lens, q_lens, hq, hkv, d)
    got = _mixed(b, 3)
    assert torch.equal(got, _separate(b, 3))
    compare(got, oracle_full(b), "bf16", f"mixed call hq={hq} hkv={hkv} d={d}")


@pytest.mark.parametrize("case", ["no_decodes", "no_chunks", "short_decodes", "fp32"])
def test_mixed_other_routes(case):
    note(f"mixed call: {case}")
    if case == "no_decodes":
        b, nd = wl.small_batch(4, "bf16", [800, 300], [800, 100], 64, 8, 64), 0
    elif case == "no_chunks":
        b, nd = wl.small_batch(5, "bf16", [800, 3000, 17], [1, 1, 1], 64, 8, 64), 3
    elif case == "short_decodes":
        b, nd = wl.small_batch(6, "bf16", [100, 512, 700], [1, 1, 700], 64, 8, 64), 2
    else:
        b, nd = wl.small_batch(7, "f32", [600, 900, 400], [1, 1, 400], 8, 2, 64), 2
    got = _mixed(b, nd)
    assert torch.equal(got, _separate(b, nd))
    compare(got, oracle_full(b), b.dtype, f"mixed call, {case}")


def test_mixed_runs_are_deterministic():
    note("mixed call: two runs bit-identical")
    b = wl.small_batch(8, "bf16", [5000, 700, 1200, 2048], [1, 1, 1, 2048], 64, 8, 64)
    assert torch.equal(_mixed(b, 3), _mixed(b, 3, ws_extra=256))
