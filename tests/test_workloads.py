"""The seeded synthetic workloads are the five configurations they stand for.

Each generator in gqa_paged_attention_amd.workloads is checked against the
shape of its configuration: sequence count, query and KV heads, head_dim,
length distribution, 16-token HND pages behind a random page table, the sink
distribution and the scale.  The pool's unused slots and spare pages hold NaN,
so a kernel that reads past a sequence or through a wrong table entry cannot
pass a parity test by accident; this file checks that they do.  The Qwen-shaped
decode pool (4.7 GB) is too large for the CPU suite: its generator is checked
through the arguments it hands to build_batch, and the GPU parity tests run it
whole.
"""
import math

import pytest
import torch

from gqa_paged_attention_amd import workloads as wl

PAGE = 16


def _check_layout(b, *, dtype, n_seqs, hq, hkv, d, spare_min, tails_unset=True):
    """Page table, pool and slack of one PagedBatch."""
    assert b.dtype == dtype
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    assert b.q.dtype == b.k_cache.dtype == b.v_cache.dtype == tdt
    assert b.page_size == PAGE
    assert (b.num_q_heads, b.num_kv_heads, b.head_dim) == (hq, hkv, d)
    assert b.num_seqs == n_seqs
    assert b.scale == pytest.approx(1.0 / math.sqrt(d))
    n_pages = b.k_cache.shape[0]
    # HND pages: [page][kv head][16 tokens][d]
    assert tuple(b.k_cache.shape) == (n_pages, hkv, PAGE, d)
    assert b.v_cache.shape == b.k_cache.shape
    assert int(b.cu_seqlens_q[0]) == 0
    assert int(b.cu_seqlens_q[-1]) == b.q.shape[0]
    assert tuple(b.q.shape[1:]) == (hq, d)

    used = []
    for s in range(n_seqs):
        L = int(b.seq_lens[s])
        n = (L + PAGE - 1) // PAGE
        row = b.block_table[s]
        assert torch.all(row[:n] >= 0) and torch.all(row[:n] < n_pages)
        if tails_unset:
            assert torch.all(row[n:] == -1), "table tails are -1"
        used += row[:n].tolist()
        # the slack of the last page is NaN
        if L % PAGE:
            last = int(row[n - 1])
            assert torch.isnan(b.k_cache[last, :, L % PAGE:].float()).all()
            assert torch.isnan(b.v_cache[last, :, L % PAGE:].float()).all()
        # the visible keys are finite
        pages = row[:n].long()
        k = b.k_cache[pages].transpose(1, 2).reshape(n * PAGE, hkv, d)[:L]
        assert torch.isfinite(k.float()).all()
    assert len(set(used)) == len(used), "no page is shared"
    spare = sorted(set(range(n_pages)) - set(used))
    assert len(spare) >= spare_min
    if spare:
        assert torch.isnan(b.k_cache[spare].float()).all()
    # the table is a permutation, not the identity layout
    if len(used) > 8:
        assert used != sorted(used)
    return used


def test_tiny_fp32_config():
    pre, dec, (page, slot, new_k, new_v) = wl.tiny_fp32(0)
    # 1 seq, 4 q / 1 KV head, head_dim 64, 256-token prefill then 1 decode step, scale 1/8
    # (the prefill's table already holds the page the decode token is appended to)
    _check_layout(pre, dtype="f32", n_seqs=1, hq=4, hkv=1, d=64, spare_min=0,
                  tails_unset=False)
    _check_layout(dec, dtype="f32", n_seqs=1, hq=4, hkv=1, d=64, spare_min=0)
    assert int(pre.seq_lens[0]) == 256 and pre.q.shape[0] == 256
    assert int(dec.seq_lens[0]) == 257 and dec.q.shape[0] == 1
    assert pre.scale == 0.125
    assert pre.sinks is not None and torch.isfinite(pre.sinks).all()
    # the decode step's key sits where the append writes it; the prefill pool holds NaN there
    assert page == int(dec.block_table[0, 256 // PAGE]) and slot == 256 % PAGE
    assert torch.isnan(pre.k_cache[page, :, slot]).all()
    assert torch.equal(dec.k_cache[page, :, slot], new_k)
    assert torch.equal(dec.v_cache[page, :, slot], new_v)


def test_gptoss_decode_config():
    b = wl.gptoss_decode(0)
    _check_layout(b, dtype="bf16", n_seqs=64, hq=64, hkv=8, d=64, spare_min=1)
    L = b.seq_lens
    assert int(L.min()) >= 1024 and int(L.max()) <= 8192
    assert len(set(L.tolist())) > 32, "lengths are drawn, not fixed"
    assert torch.equal(b.cu_seqlens_q, torch.arange(65, dtype=torch.int32))
    assert b.sinks.shape == (64,) and torch.isfinite(b.sinks).all()
    # q, K, V and sinks are N(0, 1)
    assert abs(float(b.q.float().std()) - 1.0) < 0.02
    assert abs(float(b.q.float().mean())) < 0.02
    assert 0.5 < float(b.sinks.std()) < 1.6


def test_gptoss_prefill_config():
    b = wl.gptoss_prefill(0)
    _check_layout(b, dtype="bf16", n_seqs=8, hq=64, hkv=8, d=64, spare_min=1)
    assert torch.equal(b.seq_lens, torch.full((8,), 4096, dtype=torch.int32))
    assert torch.equal(b.cu_seqlens_q, torch.arange(9, dtype=torch.int32) * 4096)
    assert torch.isfinite(b.sinks).all()


def test_mixed_config():
    full, dec, pre = wl.mixed(0)
    _check_layout(full, dtype="bf16", n_seqs=34, hq=64, hkv=8, d=64, spare_min=1)
    Ld = dec.seq_lens
    assert dec.num_seqs == 32 and int(Ld.min()) >= 2048 and int(Ld.max()) <= 16384
    assert torch.equal(dec.cu_seqlens_q, torch.arange(33, dtype=torch.int32))
    # 2 prefill chunks of 2048 tokens on 8192-token cached prefixes
    assert pre.num_seqs == 2
    assert torch.equal(pre.seq_lens, torch.full((2,), 8192 + 2048, dtype=torch.int32))
    assert torch.equal(pre.cu_seqlens_q, torch.tensor([0, 2048, 4096], dtype=torch.int32))
    # the parts share one pool and one table
    assert dec.k_cache.data_ptr() == pre.k_cache.data_ptr() == full.k_cache.data_ptr()
    # sinks ~ N(0, 2)
    assert 1.2 < float(full.sinks.std()) < 3.0


def test_qwen_decode_config(monkeypatch):
    seen = {}

    def fake_build(gen, dtype, seq_lens, q_lens, hq, hkv, d, **kw):
        seen.update(dtype=dtype, L=torch.as_tensor(seq_lens), Lq=torch.as_tensor(q_lens),
                    heads=(hq, hkv, d), **kw)
        return wl.PagedBatch(dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                             page_size=PAGE, seq_lens=torch.as_tensor(seq_lens),
                             cu_seqlens_q=torch.zeros(1), q=torch.zeros(1),
                             k_cache=torch.zeros(1), v_cache=torch.zeros(1),
                             block_table=torch.zeros(1), sinks=None, scale=1.0)

    monkeypatch.setattr(wl, "build_batch", fake_build)
    wl.qwen_decode(0)
    # 128 seqs x 1 token, 64 q / 4 KV heads, head_dim 128, ctx U[4096, 32768], sinks -inf
    assert seen["dtype"] == "bf16" and seen["heads"] == (64, 4, 128)
    assert seen["L"].numel() == 128 and torch.all(seen["Lq"] == 1)
    assert int(seen["L"].min()) >= 4096 and int(seen["L"].max()) <= 32768
    assert len(set(seen["L"].tolist())) > 64
    assert seen["sink_mode"] == "neginf"


def test_generators_are_seeded():
    a, _, _ = wl.tiny_fp32(0)
    b, _, _ = wl.tiny_fp32(0)
    c, _, _ = wl.tiny_fp32(1)
    for x, y in ((a.q, b.q), (a.k_cache, b.k_cache), (a.block_table, b.block_table),
                 (a.sinks, b.sinks)):
        assert torch.equal(x.nan_to_num(), y.nan_to_num())
    assert not torch.equal(a.q, c.q)
