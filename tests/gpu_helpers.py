"""Shared pieces of the GPU parity tests: running the C ABI, comparing to the
oracle at the stated tolerances, and sampling rows at full sizes."""
from __future__ import annotations

import sys

from dataclasses import replace

import numpy as np

import torch

import gqa_paged_attention_amd as ga
import oracle

# Elementwise bar: |gpu - oracle| <= atol + rtol * |oracle|, no NaN/Inf.
TOL = {"bf16": (1e-2, 2e-2), "f32": (1e-5, 1e-5)}
# rms(err) / rms(ref) bar for bf16, which a kernel that drops the sink fails on
# the sink-sensitive cases.
RMS_BAR = {"bf16": 1e-2, "f32": 1e-5}
ORACLE_THREADS = 16


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")
    ga.library()  # raises if the HIP library is missing


def run_decode(batch_cpu, max_seq_len=None, sync=True, window=None):
    """attn_sinks_decode through the C ABI (attn_sinks_decode_window when
    `window` is given); returns the output on the CPU."""
    require_gpu()
    g = batch_cpu.to("cuda")
    out = torch.empty_like(g.q)
    msl = batch_cpu.max_seq_len if max_seq_len is None else max_seq_len
    nbytes = ga.attn_sinks_decode_workspace_bytes(g.num_seqs, g.num_q_heads, g.num_kv_heads,
                                                  g.head_dim, msl)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    args = (g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.sinks, g.scale)
    if window is None:
        ga.attn_sinks_decode(*args, out, ws, msl)
    else:
        ga.attn_sinks_decode_window(*args, window, out, ws, msl)
    if sync:
        torch.cuda.synchronize()
    return out.cpu()


def run_prefill(batch_cpu, sync=True, window=None):
    """attn_sinks_prefill through the C ABI (attn_sinks_prefill_window when
    `window` is given); returns the output on the CPU."""
    require_gpu()
    g = batch_cpu.to("cuda")
    out = torch.empty_like(g.q)
    args = (g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.cu_seqlens_q, g.sinks,
            g.scale)
    if window is None:
        ga.attn_sinks_prefill(*args, out, batch_cpu.max_q_len, batch_cpu.max_seq_len)
    else:
        ga.attn_sinks_prefill_window(*args, window, out, batch_cpu.max_q_len,
                                     batch_cpu.max_seq_len)
    if sync:
        torch.cuda.synchronize()
    return out.cpu()


def compare(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str) -> dict:
    """Assert the tolerance bar; return the error statistics."""
    atol, rtol = TOL[dtype]
    g = got.double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    assert np.all(np.isfinite(g)), f"{what}: NaN/Inf in the GPU output"
    err = np.abs(g - r)
    bad = err > atol + rtol * np.abs(r)
    big = np.abs(r) >= atol
    stats = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_rel": float((err[big] / np.abs(r[big])).max()) if big.any() else 0.0,
        "rms_ratio": float(np.sqrt((err ** 2).mean()) / max(np.sqrt((r ** 2).mean()), 1e-30))
        if err.size else 0.0,
    }
    note(f"  {what}: max_abs={stats['max_abs']:.3e} max_rel={stats['max_rel']:.3e} "
         f"rms_ratio={stats['rms_ratio']:.3e}")
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance, first at "
                             f"{idx}: gpu={g[idx]!r} oracle={r[idx]!r}")
    assert stats["rms_ratio"] <= RMS_BAR[dtype], f"{what}: rms ratio {stats['rms_ratio']:.3e}"
    return stats


def oracle_full(batch_cpu, window=0):
    return oracle.attention(batch_cpu, threads=ORACLE_THREADS, window=window)


def sample_rows(batch_cpu, n_rows: int, seed: int):
    """(token, head) pairs: every sequence's first and last query row, plus a
    seeded random sample; heads cycle so every head is covered."""
    rng = np.random.default_rng(seed)
    cu = batch_cpu.cu_seqlens_q.numpy()
    toks = []
    for b in range(batch_cpu.num_seqs):
        if cu[b + 1] > cu[b]:
            toks += [cu[b], cu[b + 1] - 1]
    extra = max(n_rows - len(toks), 0)
    toks += list(rng.integers(0, batch_cpu.total_q, size=extra))
    toks = np.asarray(toks, dtype=np.int64)
    heads = (np.arange(toks.size) * 7 + rng.integers(0, batch_cpu.num_q_heads)) % \
        batch_cpu.num_q_heads
    return toks, heads.astype(np.int32)


def check_sampled(got: torch.Tensor, batch_cpu, n_rows: int, seed: int, what: str,
                  window: int = 0) -> dict:
    toks, heads = sample_rows(batch_cpu, n_rows, seed)
    ref = oracle.attention_rows(batch_cpu, toks, heads, threads=ORACLE_THREADS, window=window)
    return compare(got[torch.as_tensor(toks), torch.as_tensor(heads.astype(np.int64))], ref,
                   batch_cpu.dtype, what)


def scale_keys(b, first_token, factor):
    """Multiply the stored K rows of tokens >= first_token of every sequence by
    `factor` (the oracle reads the same stored values)."""
    k = b.k_cache.clone()
    for s in range(b.num_seqs):
        for t in range(first_token, int(b.seq_lens[s])):
            page = int(b.block_table[s, t // 16])
            k[page, :, t % 16, :] = (k[page, :, t % 16, :].float() * factor).to(k.dtype)
    return replace(b, k_cache=k)


def aligned_scores(b, seed, q_norm, k_norm):
    """Every query of KV head g is q_norm u_g (+ noise 0.1) and every stored
    key of it is -k_norm u_g (+ noise 0.5), u_g a random unit vector: all
    logits near -scale q_norm k_norm, spread by a few units."""
    gen = torch.Generator().manual_seed(seed)
    G = b.num_q_heads // b.num_kv_heads
    u = torch.randn(b.num_kv_heads, b.head_dim, generator=gen)
    u = u / u.norm(dim=1, keepdim=True)
    q = (q_norm * u.repeat_interleave(G, dim=0)[None] +
         0.1 * torch.randn(b.q.shape, generator=gen)).to(b.q.dtype)
    k = b.k_cache.float().clone()
    for s_ in range(b.num_seqs):
        for t in range(int(b.seq_lens[s_])):
            page = int(b.block_table[s_, t // 16])
            k[page, :, t % 16, :] = -k_norm * u + 0.5 * torch.randn(u.shape, generator=gen)
    return replace(b, q=q, k_cache=k.to(b.k_cache.dtype))
