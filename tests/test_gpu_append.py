"""GPU parity of the KV append and of the append-then-attend calls.

The append ("GPT OSS" model notes, section 3: a layer's K and V are appended
to the cache before the attention step) is pure data movement, so the bar is
bit equality: with the new tokens' slots blanked (NaN), appending them must
rebuild the pool the input generator laid out with the tokens in place, and
match the oracle's append.  The combined calls must then equal the oracle's
attention on that full pool, with and without a sliding window.
"""
import pytest
import torch

import gqa_paged_attention_amd as ga
import oracle
from gqa_paged_attention_amd import workloads as wl
from tests.gpu_helpers import compare, note, oracle_full, require_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [
    # id, dtype, seq_lens, new tokens per sequence, Hkv, d
    ("bf16_d64_ragged", "bf16", [33, 1, 70, 16, 500], [4, 1, 70, 16, 0], 2, 64),
    ("bf16_d128", "bf16", [129, 64, 17], [30, 1, 17], 4, 128),
    ("f32_d64", "f32", [5, 129, 64], [5, 30, 1], 3, 64),
    ("f32_d128_one_each", "f32", [7, 300, 16], [1, 1, 1], 1, 128),
    # a token's rows over 72 heads exceed one workgroup's pass group
    ("f32_d128_72_heads", "f32", [40, 3, 17], [40, 1, 17], 72, 128),
    # long runs of tokens: several tokens a workgroup, a partial last one
    ("bf16_d64_long_runs", "bf16", [3000, 1200, 9], [2501, 700, 9], 1, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_append_rebuilds_the_pool(case):
    name, dt, L, n, Hkv, d = case
    require_gpu()
    full = wl.small_batch(len(name) * 7 + 1, dt, L, n, 4 * Hkv, Hkv, d, sink_mode="normal")
    before, k_new, v_new = wl.split_new_tokens(full)
    ref_k, ref_v = oracle.append_kv(before, k_new, v_new)
    g = before.to("cuda")
    note(f"append {name}: L={L} n={n} Hkv={Hkv} d={d} {dt}")
    ga.attn_sinks_append_kv(k_new.cuda(), v_new.cuda(), g.k_cache, g.v_cache, g.block_table,
                            g.seq_lens, g.cu_seqlens_q, before.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g.k_cache.cpu()), _bits(ref_k)), "K pool differs from the oracle"
    assert torch.equal(_bits(g.v_cache.cpu()), _bits(ref_v)), "V pool differs from the oracle"
    assert torch.equal(_bits(g.k_cache.cpu()), _bits(full.k_cache))
    assert torch.equal(_bits(g.v_cache.cpu()), _bits(full.v_cache))


@pytest.mark.parametrize("window", [0, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_append(dt, window):
    require_gpu()
    full = wl.small_batch(301, dt, [1, 17, 300, 2049], [1, 1, 1, 1], 16, 2, 64,
                          sink_mode="normal")
    before, k_new, v_new = wl.split_new_tokens(full)
    g = before.to("cuda")
    out = torch.empty_like(g.q)
    nbytes = ga.attn_sinks_decode_workspace_bytes(g.num_seqs, g.num_q_heads, g.num_kv_heads,
                                                  g.head_dim, before.max_seq_len)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    note(f"decode_append {dt} window {window}")
    ga.attn_sinks_decode_append(g.q, k_new.cuda(), v_new.cuda(), g.k_cache, g.v_cache,
                                g.block_table, g.seq_lens, g.sinks, g.scale, window, out, ws,
                                before.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g.k_cache.cpu()), _bits(full.k_cache))
    assert torch.equal(_bits(g.v_cache.cpu()), _bits(full.v_cache))
    compare(out.cpu(), oracle_full(full, window=window), dt, f"decode_append window {window}")


@pytest.mark.parametrize("window", [0, 64])
@pytest.mark.parametrize("dt,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_prefill_append(dt, d, window):
    require_gpu()
    full = wl.small_batch(302 + d, dt, [500, 130, 64], [100, 130, 1], 16, 2, d,
                          sink_mode="normal")
    before, k_new, v_new = wl.split_new_tokens(full)
    g = before.to("cuda")
    out = torch.empty_like(g.q)
    note(f"prefill_append {dt} d={d} window {window}")
    ga.attn_sinks_prefill_append(g.q, k_new.cuda(), v_new.cuda(), g.k_cache, g.v_cache,
                                 g.block_table, g.seq_lens, g.cu_seqlens_q, g.sinks, g.scale,
                                 window, out, before.max_q_len, before.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g.k_cache.cpu()), _bits(full.k_cache))
    compare(out.cpu(), oracle_full(full, window=window), dt, f"prefill_append window {window}")


def test_tiny_fp32_prefill_then_append_and_decode():
    """The tiny workload's sequence: prefill 256 tokens, append token 256
    with the decode query, decode at L = 257 (fp32, 1e-5)."""
    require_gpu()
    pre, dec, (page, slot, nk, nv) = wl.tiny_fp32(0)
    g = pre.to("cuda")
    out_p = torch.empty_like(g.q)
    ga.attn_sinks_prefill(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.cu_seqlens_q,
                          g.sinks, g.scale, out_p, pre.max_q_len, pre.max_seq_len)
    d = dec.to("cuda")
    out_d = torch.empty_like(d.q)
    note("tiny fp32: prefill, append + decode")
    ga.attn_sinks_decode_append(d.q, nk[None].cuda(), nv[None].cuda(), g.k_cache, g.v_cache,
                                d.block_table, d.seq_lens, d.sinks, d.scale, 0, out_d, None,
                                dec.max_seq_len)
    torch.cuda.synchronize()
    compare(out_p.cpu(), oracle_full(pre), "f32", "tiny prefill")
    compare(out_d.cpu(), oracle_full(dec), "f32", "tiny append + decode")
    assert torch.equal(_bits(g.k_cache.cpu()), _bits(dec.k_cache))


def test_full_gptoss_prefill_chunk_append():
    """All 32768 tokens x 8 KV heads of the gpt-oss prefill appended into a
    blank pool: bit-identical to the generator's pool."""
    require_gpu()
    full = wl.gptoss_prefill(0)
    before, k_new, v_new = wl.split_new_tokens(full)
    g = before.to("cuda")
    note("full gpt-oss prefill chunk append")
    ga.attn_sinks_append_kv(k_new.cuda(), v_new.cuda(), g.k_cache, g.v_cache, g.block_table,
                            g.seq_lens, g.cu_seqlens_q, before.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g.k_cache), _bits(full.k_cache.cuda()))
    assert torch.equal(_bits(g.v_cache), _bits(full.v_cache.cuda()))
