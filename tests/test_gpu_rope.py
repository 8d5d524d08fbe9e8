"""GPU parity of the fused rotary-embedding append (attn_sinks_rope_append)
against the fp64 oracle of oracle/rope.py.

"GPT OSS" model notes, sections 3 and 4.1: Q and K are rotated (NeoX RoPE,
YaRN scaling, original context 4096, beta_fast 32, beta_slow 1) before K is
appended.  The rotated q and the rotated K written to the cache must meet
the tolerance bar against the oracle's fp64 rotation; V and every slot the
append does not own must be bit-identical to the oracle's append.  The base
and the scale are call parameters (the notes give neither); the cases use
base 10000 with scale 1 (plain RoPE) and 32, at cache positions and at far
positions up to 2^20.
"""
import numpy as np
import pytest
import torch
from dataclasses import replace

import gqa_paged_attention_amd as ga
from oracle import rope as R
from gqa_paged_attention_amd import workloads as wl
from tests.gpu_helpers import compare, note, oracle_full, require_gpu

pytestmark = pytest.mark.gpu

BASE, ORIG, BF, BS = 10000.0, 4096, 32.0, 1.0


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [
    # id, dtype, seq_lens, new tokens per sequence, Hq, Hkv, d
    ("bf16_d64_ragged", "bf16", [33, 1, 70, 16, 500], [4, 1, 70, 16, 0], 16, 2, 64),
    ("bf16_d128", "bf16", [129, 64, 17], [30, 1, 17], 16, 4, 128),
    ("f32_d64", "f32", [5, 129, 64], [5, 30, 1], 12, 3, 64),
    ("f32_d128_one_each", "f32", [7, 300, 16], [1, 1, 1], 4, 1, 128),
]


def _positions(full, kind, seed):
    cu = full.cu_seqlens_q.tolist()
    if kind == "cache":
        pos = []
        for b in range(full.num_seqs):
            n = cu[b + 1] - cu[b]
            pos += [int(full.seq_lens[b]) - n + i for i in range(n)]
        return torch.tensor(pos, dtype=torch.int32)
    gen = torch.Generator().manual_seed(seed)
    pos = torch.randint(0, 1 << 20, (cu[-1],), generator=gen, dtype=torch.int64)
    pos[: min(3, len(pos))] = torch.tensor([0, 131071, 4096])[: min(3, len(pos))]
    return pos.to(torch.int32)


def _run(full, pos, scale):
    before, k_new, v_new = wl.split_new_tokens(full)
    g = before.to("cuda")
    q = full.q.cuda().clone()
    ga.attn_sinks_rope_append(q, k_new.cuda(), v_new.cuda(), pos.cuda(), g.k_cache, g.v_cache,
                              g.block_table, g.seq_lens, g.cu_seqlens_q, before.max_seq_len,
                              BASE, scale, ORIG, BF, BS)
    torch.cuda.synchronize()
    ref = R.rope_append(before, full.q, k_new, v_new, pos, BASE, scale, ORIG, BF, BS)
    return before, g, q.cpu(), ref


def _new_slots(batch):
    cu = batch.cu_seqlens_q.tolist()
    out = []
    for b in range(batch.num_seqs):
        L, n = int(batch.seq_lens[b]), cu[b + 1] - cu[b]
        for i in range(n):
            p = L - n + i
            out.append((int(batch.block_table[b, p // 16]), p % 16))
    return out


@pytest.mark.parametrize("kind", ["cache", "far"])
@pytest.mark.parametrize("scale", [1.0, 32.0])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rope_append_matches_oracle(case, scale, kind):
    name, dt, L, n, Hq, Hkv, d = case
    require_gpu()
    full = wl.small_batch(len(name) * 11 + d, dt, L, n, Hq, Hkv, d, sink_mode="normal")
    pos = _positions(full, kind, 7)
    note(f"rope_append {name} scale {scale} positions {kind}")
    before, g, q_gpu, (q_rot, k_rot, kc, vc) = _run(full, pos, scale)
    compare(q_gpu, q_rot, dt, f"rotated q {name}")
    k_gpu = g.k_cache.cpu()
    slots = _new_slots(before)
    got_k = torch.stack([k_gpu[pg, :, sl, :] for pg, sl in slots])
    compare(got_k, k_rot, dt, f"rotated K in the cache {name}")
    # everything else in the pool, and V, exactly as the oracle's append
    for pg, sl in slots:
        k_gpu[pg, :, sl, :] = kc[pg, :, sl, :]
    assert torch.equal(_bits(k_gpu), _bits(kc)), "K slots outside the new tokens changed"
    assert torch.equal(_bits(g.v_cache.cpu()), _bits(vc)), "V differs from the oracle's append"


@pytest.mark.parametrize("dt,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_rope_append_then_prefill(dt, d):
    """The step the notes describe: rotate, append, attend.  The GPU attends
    with its own rotated q and cache; the oracle with its own (rounded to
    the dtype), and the outputs meet the bar."""
    require_gpu()
    full = wl.small_batch(500 + d, dt, [300, 77, 130], [120, 77, 1], 16, 2, d,
                          sink_mode="normal")
    pos = _positions(full, "cache", 0)
    before, g, q_gpu, (q_rot, k_rot, kc, vc) = _run(full, pos, 32.0)
    out = torch.empty_like(g.q)
    ga.attn_sinks_prefill(q_gpu.cuda(), g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                          g.cu_seqlens_q, g.sinks, g.scale, out, before.max_q_len,
                          before.max_seq_len)
    torch.cuda.synchronize()
    rotated = replace(before, q=torch.from_numpy(q_rot).to(full.q.dtype), k_cache=kc,
                      v_cache=vc)
    note(f"rope_append then prefill {dt} d={d}")
    compare(out.cpu(), oracle_full(rotated), dt, f"rope + append + prefill {dt} d={d}")


def test_full_gptoss_prefill_chunk_rope_append():
    """All 32768 tokens of the gpt-oss prefill shape, scale 32, at their cache
    positions: sampled rows of q and K against the oracle, V bit-exact."""
    require_gpu()
    full = wl.gptoss_prefill(0)
    pos = _positions(full, "cache", 0)
    before, k_new, v_new = wl.split_new_tokens(full)
    g = before.to("cuda")
    q = full.q.cuda().clone()
    note("full gpt-oss prefill chunk rope_append")
    ga.attn_sinks_rope_append(q, k_new.cuda(), v_new.cuda(), pos.cuda(), g.k_cache, g.v_cache,
                              g.block_table, g.seq_lens, g.cu_seqlens_q, before.max_seq_len,
                              BASE, 32.0, ORIG, BF, BS)
    torch.cuda.synchronize()
    rows = torch.randperm(q.shape[0], generator=torch.Generator().manual_seed(3))[:512]
    f = R.yarn_frequencies(64, BASE, 32.0, ORIG, BF, BS)
    ms = R.yarn_mscale(32.0)
    compare(q.cpu()[rows], R.rope(full.q[rows], pos[rows], f, ms), "bf16", "sampled q rows")
    slots = _new_slots(before)
    k_gpu = g.k_cache.cpu()
    got = torch.stack([k_gpu[slots[t][0], :, slots[t][1], :] for t in rows.tolist()])
    compare(got, R.rope(k_new[rows], pos[rows], f, ms), "bf16", "sampled K rows")
    assert torch.equal(_bits(g.v_cache.cpu()), _bits(full.v_cache))
