"""GPU parity of the multi-token decode (a few new query tokens per
sequence, as when speculative or MTP drafts are verified) against the
oracle, which computes it as a causal chunk at the end of each sequence.

Cases cover every packed width (G x Lq query rows per KV head: one, two and
four 16-column blocks at d = 64, one and two at d = 128), shapes that need several
grid layers of such blocks (up to 128 rows), sequences with fewer new
tokens than the batch's maximum, sequences shorter than a 32-token block or
whose new tokens straddle block and page boundaries, and the shapes that
fall back to the prefill kernel (fp32, more packed rows than the split pass
takes).
"""
import pytest
import torch

import gqa_paged_attention_amd as ga
from gqa_paged_attention_amd import workloads as wl
from tests.gpu_helpers import compare, note, oracle_full, require_gpu

pytestmark = pytest.mark.gpu


def run_multi(b):
    require_gpu()
    g = b.to("cuda")
    out = torch.empty_like(g.q)
    nbytes = ga.attn_sinks_decode_multi_workspace_bytes(g.num_seqs, g.num_q_heads,
                                                        g.num_kv_heads, g.head_dim,
                                                        b.max_seq_len, b.max_q_len)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda") if nbytes else None
    ga.attn_sinks_decode_multi(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                               g.cu_seqlens_q, g.sinks, g.scale, out, ws, b.max_q_len,
                               b.max_seq_len)
    torch.cuda.synchronize()
    return out.cpu(), nbytes


CASES = [
    # id, dtype, seq_lens, q_lens, Hq, Hkv, d, packed (uses the split passes)
    ("d64_g8_lq2", "bf16", [2, 33, 100, 1000, 4097], [2, 2, 2, 2, 2], 16, 2, 64, True),
    ("d64_g8_lq4_ragged", "bf16", [4, 31, 35, 500, 3000], [4, 3, 4, 1, 2], 16, 2, 64, True),
    ("d64_g8_lq8", "bf16", [8, 40, 64, 65, 2049], [8, 8, 8, 5, 8], 16, 2, 64, True),
    ("d64_g4_lq3", "bf16", [3, 17, 130], [3, 3, 3], 8, 2, 64, True),
    ("d64_g1_lq6", "bf16", [6, 300], [6, 6], 4, 4, 64, True),
    ("d64_g16_lq4", "bf16", [9, 777], [4, 4], 32, 2, 64, True),
    ("d128_g8_lq2", "bf16", [2, 129, 1500], [2, 2, 1], 16, 2, 128, True),
    ("d128_g16_lq1", "bf16", [300, 33], [1, 1], 32, 2, 128, True),
    ("d128_g16_lq2_two_blocks", "bf16", [50, 600], [2, 2], 32, 2, 128, True),
    ("d128_g8_lq3_two_blocks", "bf16", [3, 70, 1000], [3, 2, 3], 16, 2, 128, True),
    ("d128_g16_lq4_two_layers", "bf16", [4, 33, 2000], [4, 3, 4], 64, 4, 128, True),
    ("d128_g16_lq8_four_layers", "bf16", [8, 1025], [8, 7], 32, 2, 128, True),
    ("d64_g8_lq9_two_layers", "bf16", [9, 200], [9, 9], 16, 2, 64, True),
    ("d64_g16_lq8_two_layers", "bf16", [8, 3000, 70], [8, 8, 2], 32, 2, 64, True),
    ("d64_g16_lq9_fallback", "bf16", [9, 200], [9, 9], 32, 2, 64, False),
    ("d128_g16_lq9_fallback", "bf16", [9, 300], [9, 5], 32, 2, 128, False),
    ("f32_d64_lq4", "f32", [4, 77], [4, 3], 8, 2, 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_multi_token_decode(case):
    name, dt, L, Lq, Hq, Hkv, d, packed = case
    b = wl.small_batch(len(name) * 13 + 5, dt, L, Lq, Hq, Hkv, d, sink_mode="normal")
    note(f"multi-token decode {name}: L={L} Lq={Lq} Hq={Hq} Hkv={Hkv} d={d} {dt}")
    out, nbytes = run_multi(b)
    if dt == "bf16":  # the byte count depends on the shape only; fp32 never uses it
        assert (nbytes > 0) == packed, "packed/prefill choice differs from the documented rule"
    compare(out, oracle_full(b), dt, f"multi-token decode {name}")


def test_multi_with_no_new_tokens_for_some_sequences():
    b = wl.small_batch(411, "bf16", [100, 50, 300], [3, 0, 2], 16, 2, 64, sink_mode="normal")
    note("multi-token decode with an empty sequence")
    out, _ = run_multi(b)
    compare(out, oracle_full(b), "bf16", "multi-token decode, an empty sequence")


def test_multi_deterministic():
    b = wl.small_batch(412, "bf16", [900, 31, 4000], [4, 4, 3], 16, 2, 64, sink_mode="normal")
    a1, _ = run_multi(b)
    a2, _ = run_multi(b)
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))


def test_full_gptoss_shape_four_draft_tokens():
    """The gpt-oss decode shape (64 seqs, 64/8 heads, d 64, L ~ U[1024, 8192])
    with 4 new tokens per sequence: every row against the oracle."""
    gen = torch.Generator().manual_seed(0)
    L = torch.randint(1024, 8193, (64,), generator=gen, dtype=torch.int64).to(torch.int32)
    b = wl.build_batch(gen, "bf16", L, torch.full((64,), 4, dtype=torch.int32), 64, 8, 64,
                       sink_mode="normal")
    note("full gpt-oss shape, 4 draft tokens per sequence")
    out, nbytes = run_multi(b)
    assert nbytes > 0
    compare(out, oracle_full(b), "bf16", "gpt-oss multi-token decode")
