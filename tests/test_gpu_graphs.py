"""HIP-graph capture and replay of the entry points beyond plain decode and
prefill: every call enqueues only kernels (no allocation, no host sync, no
memset node), so one graph holding the windowed decode (direct path) and
prefill, the multi-token decode, the ragged call, the KV append and the
fused RoPE append must replay to the eager results, bit for bit, with eager
work between the replays."""
import pytest
import torch

import gqa_paged_attention_amd as ga
from gqa_paged_attention_amd import workloads as wl
from tests.gpu_helpers import note, require_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_graph_of_every_next_entry_point():
    require_gpu()
    dec = wl.small_batch(701, "bf16", [2000, 300, 129], [1, 1, 1], 16, 2, 64).to("cuda")
    pre = wl.small_batch(702, "bf16", [400, 90], [150, 90], 16, 2, 64).to("cuda")
    mul = wl.small_batch(703, "bf16", [900, 37], [4, 3], 16, 2, 64).to("cuda")
    rag = wl.ragged_batch(704, "bf16", [300, 77], [300, 40], 16, 2, 64)
    rq, rk, rv = rag.q.cuda(), rag.k.cuda(), rag.v.cuda()
    rcq, rckv = rag.cu_seqlens_q.cuda(), rag.cu_seqlens_kv.cuda()
    rsinks = rag.sinks.cuda()
    full = wl.small_batch(705, "bf16", [40, 5, 17], [7, 5, 1], 16, 2, 64)
    before, k_new, v_new = wl.split_new_tokens(full)
    app = before.to("cuda")
    k0, v0 = app.k_cache.clone(), app.v_cache.clone()
    q0 = full.q.cuda()
    qw = q0.clone()
    kn, vn = k_new.cuda(), v_new.cuda()
    pos = torch.arange(q0.shape[0], dtype=torch.int32, device="cuda") * 37

    outs = {
        "win_dec": torch.empty_like(dec.q), "win_pre": torch.empty_like(pre.q),
        "multi": torch.empty_like(mul.q), "ragged": torch.empty_like(rq),
        "lse": torch.empty(rq.shape[0], rq.shape[1], dtype=torch.float32, device="cuda"),
    }
    ws_dec = torch.empty(max(ga.attn_sinks_decode_workspace_bytes(
        dec.num_seqs, dec.num_q_heads, dec.num_kv_heads, dec.head_dim, dec.max_seq_len), 16),
        dtype=torch.uint8, device="cuda")
    ws_mul = torch.empty(max(ga.attn_sinks_decode_multi_workspace_bytes(
        mul.num_seqs, mul.num_q_heads, mul.num_kv_heads, mul.head_dim, mul.max_seq_len,
        mul.max_q_len), 16), dtype=torch.uint8, device="cuda")

    def work():
        ga.decode_batch(dec, outs["win_dec"], ws_dec, window=128)
        ga.prefill_batch(pre, outs["win_pre"], window=64)
        ga.attn_sinks_decode_multi(mul.q, mul.k_cache, mul.v_cache, mul.block_table,
                                   mul.seq_lens, mul.cu_seqlens_q, mul.sinks, mul.scale,
                                   outs["multi"], ws_mul, mul.max_q_len, mul.max_seq_len)
        ga.attn_sinks_ragged(rq, rk, rv, rcq, rckv, rsinks, rag.scale, True, outs["ragged"],
                             outs["lse"], 300, 300)
        # the appends write the pool and q: start each run from the same state
        app.k_cache.copy_(k0)
        app.v_cache.copy_(v0)
        qw.copy_(q0)
        ga.attn_sinks_append_kv(kn, vn, app.k_cache, app.v_cache, app.block_table,
                                app.seq_lens, app.cu_seqlens_q, before.max_seq_len)
        ga.attn_sinks_rope_append(qw, kn, vn, pos, app.k_cache, app.v_cache, app.block_table,
                                  app.seq_lens, app.cu_seqlens_q, before.max_seq_len, 10000.0,
                                  32.0)

    note("graph of the next entry points: eager reference")
    work()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    ref_q, ref_k, ref_v = qw.clone(), app.k_cache.clone(), app.v_cache.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        note("graph of the next entry points: capturing")
        with torch.cuda.graph(graph, stream=s):
            work()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs.values():
            t.fill_(7.0)
        qw.fill_(3.0)
        app.k_cache.fill_(5.0)
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(_bits(t), _bits(ref[name])), f"replay {rep}: {name} differs"
        assert torch.equal(_bits(qw), _bits(ref_q)), f"replay {rep}: rotated q differs"
        assert torch.equal(_bits(app.k_cache), _bits(ref_k)), f"replay {rep}: K pool differs"
        assert torch.equal(_bits(app.v_cache), _bits(ref_v)), f"replay {rep}: V pool differs"
