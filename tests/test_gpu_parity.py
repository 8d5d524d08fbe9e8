"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases span several 32-token decode blocks, several splits, several
128-row prefill tiles and 64-key tiles, with ragged tails and NaN-poisoned
unused page slots.  Full-size cases are the five named workloads, compared
on every row where the oracle is quick and on sampled rows otherwise.
"""
import zlib
from dataclasses import replace

import numpy as np
import pytest
import torch

import gqa_paged_attention_amd as ga
import oracle
from gqa_paged_attention_amd import workloads as wl
from tests.gpu_helpers import (aligned_scores as _aligned_scores, check_sampled, compare, note,
                               oracle_full, run_decode, scale_keys as _scale_keys,
                               run_prefill)

pytestmark = pytest.mark.gpu

# --------------------------------------------------------------- small cases

DECODE_CASES = [
    # id, dtype, seq_lens, Hq, Hkv, d, sink_mode, sink_std
    ("d64_g8_ragged", "bf16", [1, 15, 16, 17, 33, 100, 1000, 2049], 16, 2, 64, "normal", 1.0),
    ("d128_g16_ragged", "bf16", [1, 31, 32, 500, 2049, 5000], 32, 2, 128, "normal", 1.0),
    ("d64_g1", "bf16", [7, 300, 64], 4, 4, 64, "normal", 2.0),
    ("d128_g4_nosink", "bf16", [200, 129, 4097], 16, 4, 128, "none", 1.0),
    ("d64_g8_neginf", "bf16", [300, 77], 8, 1, 64, "neginf", 1.0),
    ("d64_g8_long", "bf16", [20000, 12345], 16, 2, 64, "normal", 1.0),
    ("d128_g16_long", "bf16", [33000], 16, 1, 128, "normal", 1.0),
    ("d64_g2_odd", "bf16", [45, 46, 47], 6, 3, 64, "normal", 1.0),
    ("f32_d64", "f32", [1, 17, 300], 8, 2, 64, "normal", 1.0),
    ("f32_d128", "f32", [70, 257], 16, 4, 128, "none", 1.0),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_small(case):
    name, dt, L, Hq, Hkv, d, sm, sd = case
    b = wl.small_batch(zlib.crc32(name.encode()) % 1000, dt, L, [1] * len(L), Hq, Hkv, d, sink_mode=sm,
                       sink_std=sd)
    note(f"decode {name}: L={L} Hq={Hq} Hkv={Hkv} d={d} {dt}")
    compare(run_decode(b), oracle_full(b), dt, f"decode {name}")


PREFILL_CASES = [
    # id, dtype, seq_lens, q_lens, Hq, Hkv, d, sink_mode, sink_std
    ("d64_full_causal", "bf16", [1, 17, 130, 300], [1, 17, 130, 300], 16, 2, 64, "normal", 1.0),
    ("d64_chunks_over_prefix", "bf16", [500, 1000, 64], [100, 257, 1], 16, 2, 64, "normal", 2.0),
    ("d128_full", "bf16", [200, 333], [200, 333], 8, 2, 128, "normal", 1.0),
    ("d128_chunk", "bf16", [700], [129], 16, 1, 128, "none", 1.0),
    # waves whose unmasked steps fill one run of ten (369) and two (736)
    ("d128_full_steady_runs", "bf16", [736, 369], [736, 369], 8, 2, 128, "normal", 1.0),
    ("d64_empty_chunk_between", "bf16", [50, 80, 90], [50, 0, 90], 8, 8, 64, "normal", 1.0),
    ("d64_g1_tail", "bf16", [255, 256, 257], [255, 256, 257], 4, 4, 64, "neginf", 1.0),
    ("f32_d64", "f32", [40, 150], [40, 100], 8, 2, 64, "normal", 1.0),
    ("f32_d128", "f32", [90], [33], 4, 1, 128, "normal", 1.0),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_small(case):
    name, dt, L, Lq, Hq, Hkv, d, sm, sd = case
    b = wl.small_batch(zlib.crc32(name.encode()) % 1000 + 7, dt, L, Lq, Hq, Hkv, d, sink_mode=sm,
                       sink_std=sd)
    note(f"prefill {name}: L={L} Lq={Lq} Hq={Hq} Hkv={Hkv} d={d} {dt}")
    compare(run_prefill(b), oracle_full(b), dt, f"prefill {name}")


# ------------------------------------------------------------ sink behaviour

@pytest.mark.parametrize("d,Hq,Hkv", [(64, 8, 1), (128, 16, 1)])
def test_decode_sink_sensitive(d, Hq, Hkv):
    """Sinks set to the row's own LSE + {-2, 0, +2}: the sink takes 12-88 % of
    the softmax mass, so a kernel that mishandles it fails the bar."""
    b = wl.small_batch(5 + d, "bf16", [3000], [1], Hq, Hkv, d, sink_mode="neginf")
    _, lse = oracle.attention(b, threads=16, with_lse=True)
    deltas = np.array([-2.0, 0.0, 2.0])[np.arange(Hq) % 3]
    b = replace(b, sinks=torch.tensor(lse[0] + deltas, dtype=torch.float32))
    note(f"decode sink-sensitive d={d}")
    ref = oracle_full(b)
    got = run_decode(b)
    compare(got, ref, "bf16", "sink-sensitive decode")
    plain = replace(b, sinks=None)
    diff_ref = ref - oracle_full(plain)
    diff_got = got.double() - run_decode(plain).double()
    compare(diff_got, diff_ref, "bf16", "sink effect (with - without)")


def test_prefill_sink_sensitive():
    b = wl.small_batch(77, "bf16", [400], [400], 8, 2, 64, sink_mode="normal", sink_std=4.0)
    note("prefill sink-sensitive sink_std=4")
    compare(run_prefill(b), oracle_full(b), "bf16", "prefill sink std 4")


def test_null_sinks_equal_neginf_sinks():
    b = wl.small_batch(88, "bf16", [900, 33], [1, 1], 16, 2, 64, sink_mode="neginf")
    note("decode sinks=NULL vs -inf")
    a = run_decode(b)
    c = run_decode(replace(b, sinks=None))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    p = wl.small_batch(89, "bf16", [300], [300], 8, 2, 64, sink_mode="neginf")
    note("prefill sinks=NULL vs -inf")
    assert torch.equal(run_prefill(p).view(torch.int16),
                       run_prefill(replace(p, sinks=None)).view(torch.int16))


@pytest.mark.parametrize("d,L,Lq", [(64, 300, 300), (64, 700, 190), (128, 400, 400)])
def test_prefill_large_late_logits(d, L, Lq):
    """Keys after the first 64 get logits far above every early one (std ~100
    in natural units), beyond what weights relative to the early maximum can
    hold: the kernel must detect it and still match the exact softmax."""
    b = wl.small_batch(100 + d + L, "bf16", [L], [Lq], 8, 2, d)
    b = _scale_keys(b, 64, 100.0)
    note(f"prefill large late logits d={d} L={L} Lq={Lq}")
    compare(run_prefill(b), oracle_full(b), "bf16", f"prefill large late logits d={d}")
    note(f"decode large late logits d={d} L={L}")
    dec = replace(b, cu_seqlens_q=torch.tensor([0, 1], dtype=torch.int32), q=b.q[-1:].contiguous())
    compare(run_decode(dec), oracle_full(dec), "bf16", f"decode large late logits d={d}")


@pytest.mark.parametrize("d,L,Lq", [(64, 300, 300), (64, 700, 190), (128, 400, 400)])
def test_prefill_all_logits_far_below_zero(d, L, Lq):
    """Every logit near -150 (natural units) and no sink: the unshifted
    weights 2^s would underflow to 0, yet the softmax is a proper average of
    V.  The kernel must find the rows out of range and recompute them."""
    b = wl.small_batch(200 + d + L, "bf16", [L], [Lq], 8, 2, d, sink_mode="none")
    b = _aligned_scores(b, 7 + d, 30.0, 150.0 / (30.0 * b.scale))
    note(f"prefill logits near -150, no sink, d={d} L={L} Lq={Lq}")
    compare(run_prefill(b), oracle_full(b), "bf16", f"prefill low logits d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_all_logits_large(d):
    """All keys scaled by 100 (logits of std ~100 from the first key on):
    unshifted weights overflow in most rows, which must be recomputed."""
    b = wl.small_batch(300 + d, "bf16", [500, 129], [500, 64], 8, 2, d)
    b = _scale_keys(b, 0, 100.0)
    note(f"prefill all logits large d={d}")
    compare(run_prefill(b), oracle_full(b), "bf16", f"prefill large logits d={d}")


# -------------------------------------------------------- structural checks

def _permuted(b, seed):
    gen = torch.Generator().manual_seed(seed)
    perm = torch.randperm(b.num_pages, generator=gen)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(b.num_pages)
    k2 = torch.empty_like(b.k_cache)
    v2 = torch.empty_like(b.v_cache)
    k2[inv] = b.k_cache
    v2[inv] = b.v_cache
    bt = b.block_table.clone().to(torch.int64)
    valid = bt >= 0
    bt[valid] = inv[bt[valid]]
    return replace(b, k_cache=k2, v_cache=v2, block_table=bt.to(torch.int32))


def test_page_permutation_and_determinism_bitwise():
    b = wl.small_batch(91, "bf16", [3000, 17, 999], [1, 1, 1], 16, 2, 64)
    note("decode: determinism and page permutation")
    a1 = run_decode(b)
    a2 = run_decode(b)
    a3 = run_decode(_permuted(b, 5))
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16)), "decode not deterministic"
    assert torch.equal(a1.view(torch.int16), a3.view(torch.int16)), "page permutation changed decode"
    p = wl.small_batch(92, "bf16", [600, 200], [300, 200], 16, 2, 64)
    note("prefill: determinism and page permutation")
    c1 = run_prefill(p)
    c2 = run_prefill(p)
    c3 = run_prefill(_permuted(p, 6))
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16)), "prefill not deterministic"
    assert torch.equal(c1.view(torch.int16), c3.view(torch.int16)), "page permutation changed prefill"


def test_split_count_does_not_change_decode():
    """A larger max_seq_len bound changes the split length and the number of
    splits; results stay within the bar of each other and of the oracle."""
    b = wl.small_batch(93, "bf16", [5000, 4000], [1, 1], 16, 2, 64)
    ref = oracle_full(b)
    for msl in (5000, 9000, 40000, 300000):
        note(f"decode with max_seq_len bound {msl}")
        bb = replace(b, block_table=torch.nn.functional.pad(b.block_table,
                                                            (0, msl // 16 + 1 - b.max_pages_per_seq),
                                                            value=-1))
        compare(run_decode(bb, max_seq_len=msl), ref, "bf16", f"decode bound {msl}")


def test_prefill_rows_match_decode():
    b = wl.small_batch(94, "bf16", [700], [200], 16, 2, 64)
    note("prefill rows vs decode at the same positions")
    pre = run_prefill(b)
    for i in (0, 63, 64, 127, 128, 199):
        L = 700 - 200 + i + 1
        d = replace(b, seq_lens=torch.tensor([L], dtype=torch.int32),
                    cu_seqlens_q=torch.tensor([0, 1], dtype=torch.int32),
                    q=b.q[i:i + 1].contiguous())
        dec = run_decode(d)
        compare(pre[i:i + 1], dec.double().numpy(), "bf16", f"row {i} prefill vs decode")


def test_stage_entry_points_equal_decode():
    """attn_sinks_decode == attn_sinks_decode_partials + attn_sinks_decode_merge."""
    b = wl.small_batch(98, "bf16", [5000, 1, 700], [1, 1, 1], 16, 2, 128).to("cuda")
    note("decode stages vs one-call decode")
    ref = ga.decode_batch(b)
    nbytes = ga.attn_sinks_decode_workspace_bytes(3, 16, 2, 128, b.max_seq_len)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(b.q)
    ga.attn_sinks_decode_partials(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, b.scale,
                                  ws, b.max_seq_len)
    ga.attn_sinks_decode_merge(b.seq_lens, b.sinks, ws, out, b.num_kv_heads, b.max_seq_len)
    out32 = torch.empty(out.shape, dtype=torch.float32, device="cuda")
    ga.attn_sinks_decode_merge(b.seq_lens, b.sinks, ws, out32, b.num_kv_heads, b.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(out32.to(torch.bfloat16).view(torch.int16), ref.view(torch.int16))


def test_short_contexts_take_the_direct_pass():
    """With max_seq_len <= 512 attn_sinks_decode runs one direct pass; its
    results meet the bar against the oracle and against the two stage
    entry points on the same inputs."""
    for d, L in ((64, [1, 31, 32, 33, 500, 512]), (128, [7, 200, 512])):
        b = wl.small_batch(410 + d, "bf16", L, [1] * len(L), 32, 2, d, sink_mode="normal")
        note(f"short-context decode d={d} L={L}")
        got = run_decode(b)
        compare(got, oracle_full(b), "bf16", f"direct decode d={d}")
        g = b.to("cuda")
        ws = torch.empty(ga.attn_sinks_decode_workspace_bytes(g.num_seqs, g.num_q_heads,
                                                              g.num_kv_heads, d, b.max_seq_len),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty_like(g.q)
        ga.attn_sinks_decode_partials(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                                      g.scale, ws, b.max_seq_len)
        ga.attn_sinks_decode_merge(g.seq_lens, g.sinks, ws, out, g.num_kv_heads, b.max_seq_len)
        torch.cuda.synchronize()
        compare(got, out.cpu().double().numpy(), "bf16", f"direct vs stages d={d}")


def test_empty_sequences_give_zero():
    b = wl.small_batch(95, "bf16", [1, 40], [1, 1], 8, 2, 64)
    b = replace(b, seq_lens=torch.tensor([0, 40], dtype=torch.int32))
    note("decode with an empty sequence")
    got = run_decode(b)
    assert torch.all(got[0] == 0)
    compare(got, oracle_full(b), "bf16", "decode with empty sequence")


def test_tiny_fp32_prefill_append_decode():
    """256-token causal prefill, append token 256 on the GPU, decode at 257."""
    pre, dec, (page, slot, nk, nv) = wl.tiny_fp32(0)
    note("tiny fp32 prefill")
    compare(run_prefill(pre), oracle_full(pre), "f32", "tiny fp32 prefill")
    g = pre.to("cuda")
    g.k_cache[page, :, slot, :] = nk.cuda()
    g.v_cache[page, :, slot, :] = nv.cuda()
    gd = replace(g, q=dec.q.cuda(), cu_seqlens_q=dec.cu_seqlens_q.cuda(),
                 seq_lens=dec.seq_lens.cuda(), meta={"max_q_len": 1, "max_seq_len": 257})
    note("tiny fp32 decode after append")
    out = ga.decode_batch(gd)
    torch.cuda.synchronize()
    compare(out.cpu(), oracle_full(dec), "f32", "tiny fp32 decode")


def test_graph_capture_replays():
    b = wl.small_batch(96, "bf16", [2000, 300], [1, 1], 16, 2, 64).to("cuda")
    p = wl.small_batch(97, "bf16", [400], [150], 16, 2, 64).to("cuda")
    out_d = torch.empty_like(b.q)
    out_p = torch.empty_like(p.q)
    nbytes = ga.attn_sinks_decode_workspace_bytes(2, 16, 2, 64, b.max_seq_len)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    note("graph capture: eager reference")
    ga.decode_batch(b, out_d, ws)
    ga.prefill_batch(p, out_p)
    torch.cuda.synchronize()
    ref_d, ref_p = out_d.clone(), out_p.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        out_d.zero_()
        out_p.zero_()
        note("graph capture: capturing")
        with torch.cuda.graph(graph, stream=s):
            ga.decode_batch(b, out_d, ws)
            ga.prefill_batch(p, out_p)
    torch.cuda.synchronize()
    for rep in range(3):
        out_d.fill_(7.0)
        out_p.fill_(7.0)
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d.view(torch.int16), ref_d.view(torch.int16))
        assert torch.equal(out_p.view(torch.int16), ref_p.view(torch.int16))


# ----------------------------------------------------------- full workloads

def test_full_tiny_fp32():
    pre, dec, _ = wl.tiny_fp32(0)
    note("full: tiny fp32 (prefill, decode)")
    compare(run_prefill(pre), oracle_full(pre), "f32", "tiny prefill")
    compare(run_decode(dec), oracle_full(dec), "f32", "tiny decode")


def test_full_gptoss_decode():
    note("full: gpt-oss decode, generating")
    b = wl.gptoss_decode(0)
    note("full: gpt-oss decode, running")
    got = run_decode(b)
    note("full: gpt-oss decode, oracle on every row")
    compare(got, oracle_full(b), "bf16", "gpt-oss decode (all rows)")


def test_full_gptoss_prefill():
    note("full: gpt-oss prefill, generating")
    b = wl.gptoss_prefill(0)
    note("full: gpt-oss prefill, running")
    got = run_prefill(b)
    note("full: gpt-oss prefill, oracle on sampled rows")
    check_sampled(got, b, 512, 3, "gpt-oss prefill (512 sampled rows)")


@pytest.mark.timeout(900)
def test_full_qwen_decode():
    note("full: qwen decode, generating (about a minute)")
    b = wl.qwen_decode(0)
    note("full: qwen decode, running")
    got = run_decode(b)
    note("full: qwen decode, oracle on sampled rows")
    check_sampled(got, b, 256, 4, "qwen decode (256 sampled rows)")
    note("full: qwen decode with sinks=NULL")
    got2 = run_decode(replace(b, sinks=None))
    assert torch.equal(got.view(torch.int16), got2.view(torch.int16))


def test_full_mixed():
    note("full: mixed batch, generating")
    full, dec, pre = wl.mixed(0)
    gd = dec.to("cuda")
    gp = pre.to("cuda")
    out_d = torch.empty_like(gd.q)
    out_p = torch.empty_like(gp.q)
    nbytes = ga.attn_sinks_decode_workspace_bytes(32, 64, 8, 64, dec.max_seq_len)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    note("full: mixed batch, decode then prefill on one stream")
    ga.decode_batch(gd, out_d, ws)
    ga.prefill_batch(gp, out_p)
    torch.cuda.synchronize()
    got = torch.cat([out_d.cpu(), out_p.cpu()])
    note("full: mixed batch, oracle on every decode row and sampled prefill rows")
    compare(got[:32], oracle_full(dec), "bf16", "mixed decode (all rows)")
    check_sampled(got[32:], pre, 384, 5, "mixed prefill (384 sampled rows)")
