#!/usr/bin/env python3
"""Benchmark of paged GQA attention with per-head sinks on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--only all|decode|prefill|mixed|next|qwen]

One step is one decode pass (split pass + merge pass) of the gpt-oss-20b-shaped
decode workload: 64 sequences x 1 query token, 64 q / 8 KV heads, head_dim 64,
context lengths uniform in [1024, 8192], 16-token HND pages, bf16, seeded
synthetic data.  Inputs are resident in HBM before timing starts.  L2 and the
Infinity Cache are flushed (a 1 GiB write) before every step, outside the
timed events.  The headline value is decode KV-read GB/s; the same line also
carries the causal prefill (TFLOP/s), the Qwen3-235B-shaped decode and
causal prefill (head_dim 128), the mixed batch and the sliding-window, multi-token, ragged, KV-append and
RoPE-append legs, each against its own roofline, plus the fp64 CPU oracle
timed on the host cores (a baseline, not a target).  Every leg reports the
mean step time with the median and minimum beside it.  The RoPE-append leg
rotates the same q in place every step: its values drift, its work does not.

Modes used to make the committed profiles:
    --profile-run            the selected legs (--only; default every leg),
                             no oracle, no warm pass (run under rocprofv3)
    --summarize-trace DIR NAME              kernel durations -> profiles/NAME.txt
    --summarize-traffic FDIR WDIR KERNEL NAME
                                            FETCH/WRITE_SIZE -> HBM bytes per launch
    --summarize-counters DIR KERNEL NAME    any --pmc counters -> per-dispatch
                                            averages and derived busy fractions
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, TFLOP/s (256 CU x 2.4 GHz x 4096)
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "decode_split_bf16_gptoss_decode_traffic.txt")
PREFILL_TRAFFIC_FILE = os.path.join(PROFILES, "prefill_bf16_gptoss_prefill_traffic.txt")
PREFILL_COUNTER_FILE = os.path.join(PROFILES, "prefill_bf16_gptoss_prefill_counters.txt")
# (api.cpp decides the launch shapes, kernels.h holds the constants they use)
DECODE_SOURCES = ["gqa_paged_attention_amd/csrc/decode.hip", "gqa_paged_attention_amd/csrc/split.h",
                  "gqa_paged_attention_amd/csrc/common.h",
                  "gqa_paged_attention_amd/csrc/kernels.h", "gqa_paged_attention_amd/csrc/api.cpp"]
PREFILL_SOURCES = ["gqa_paged_attention_amd/csrc/prefill.hip", "gqa_paged_attention_amd/csrc/split.h",
                   "gqa_paged_attention_amd/csrc/common.h",
                   "gqa_paged_attention_amd/csrc/kernels.h", "gqa_paged_attention_amd/csrc/api.cpp"]


def kernel_sources(kernel: str):
    """The source files a profiled kernel is built from (for the hash that
    ties a committed counter summary to the code it measured)."""
    return PREFILL_SOURCES if "prefill" in kernel else DECODE_SOURCES


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ algorithmic work

def decode_bytes(batch) -> int:
    """Bytes a decode pass must move: K and V of every visible token, q, out,
    the used page-table entries, seq_lens and sinks."""
    elem = 4 if batch.dtype == "f32" else 2
    L = batch.seq_lens.to("cpu").long()
    kv = int(L.sum()) * batch.num_kv_heads * batch.head_dim * 2 * elem
    qo = 2 * batch.num_seqs * batch.num_q_heads * batch.head_dim * elem
    table = int(((L + 15) // 16).sum()) * 4
    return kv + qo + table + 4 * batch.num_seqs + 4 * batch.num_q_heads


def prefill_flops(batch) -> int:
    """4 * d * Hq per visible (query, key) pair (QK^T and PV, 2 flops per MAC)."""
    L = batch.seq_lens.to("cpu").long()
    Lq = batch.q_lens.to("cpu").long()
    pairs = int((Lq * (L - Lq) + Lq * (Lq + 1) // 2).sum())
    return 4 * batch.head_dim * batch.num_q_heads * pairs


def window_decode_bytes(batch, window: int) -> int:
    """Bytes a sliding-window decode pass must move: K and V of the last
    `window` keys of every sequence, q, out, the table entries of the pages
    holding them, seq_lens and sinks."""
    elem = 4 if batch.dtype == "f32" else 2
    L = batch.seq_lens.to("cpu").long()
    lo = (L - window).clamp(min=0)
    kv = int((L - lo).sum()) * batch.num_kv_heads * batch.head_dim * 2 * elem
    qo = 2 * batch.num_seqs * batch.num_q_heads * batch.head_dim * elem
    table = int(((L - 1) // 16 - lo // 16 + 1).clamp(min=0).sum()) * 4
    return kv + qo + table + 4 * batch.num_seqs + 4 * batch.num_q_heads


def window_prefill_work(batch, window: int):
    """(flops, bytes) of a sliding-window prefill: 4 d Hq per visible
    (query, key) pair; q and out once, and K and V of every key some row of
    the chunk sees, once."""
    elem = 4 if batch.dtype == "f32" else 2
    flops = kv = 0
    L = batch.seq_lens.tolist()
    Lq = batch.q_lens.tolist()
    for l, lq in zip(L, Lq):
        flops += sum(min(p + 1, window) for p in range(l - lq, l))
        kv += l - max(l - lq - window + 1, 0)
    flops *= 4 * batch.head_dim * batch.num_q_heads
    qo = 2 * batch.total_q * batch.num_q_heads * batch.head_dim * elem
    return flops, qo + kv * batch.num_kv_heads * batch.head_dim * 2 * elem


# ------------------------------------------------------------------ timing

class Timer:
    """Per-stage HIP-event timing of a list of launches on the current stream."""

    # Warm-up runs at least this long as well as at least W steps: after the
    # host-side work between legs (seconds of workload generation) the GPU
    # needs some tens of milliseconds of load before its clocks settle.
    MIN_WARMUP_S = 0.25

    def __init__(self, torch, flush_buf):
        self.torch = torch
        self.flush_buf = flush_buf

    def run(self, stages, steps, warmup, flush=True):
        """Time `steps` steps twice after the warm-up: once with events only
        around each whole step (step_ms: nothing recorded between its
        launches), once with an event after every stage (stage_ms)."""
        torch = self.torch
        n = len(stages)
        t_w = time.perf_counter()
        done = 0
        while done < warmup or time.perf_counter() - t_w < self.MIN_WARMUP_S:
            if flush:
                self.flush_buf.fill_(1)
            for _, fn in stages:
                fn()
            torch.cuda.synchronize()
            done += 1
        walls = []
        totals = []
        per_stage = {name: [] for name, _ in stages}
        for instrumented in (False, True):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
                  for _ in range(steps)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(steps):
                if flush:
                    self.flush_buf.fill_(k & 0xff)
                ev[k][0].record()
                for i, (_, fn) in enumerate(stages):
                    fn()
                    if instrumented or i == n - 1:
                        ev[k][i + 1 if instrumented else n].record()
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t0)
            if instrumented:
                for i, (name, _) in enumerate(stages):
                    per_stage[name] = [ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(steps)]
            else:
                totals = [ev[k][0].elapsed_time(ev[k][n]) for k in range(steps)]
        return {"stage_ms": {k: sum(v) / len(v) for k, v in per_stage.items()},
                "stage_ms_min": {k: min(v) for k, v in per_stage.items()},
                "step_ms": sum(totals) / len(totals),
                "step_ms_median": _median(totals),
                "step_ms_min": min(totals),
                "wall_s": walls[0]}


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def spread(r) -> dict:
    """Median and minimum step time beside the mean (ms)."""
    return {"ms_median": round(r["step_ms_median"], 4), "ms_min": round(r["step_ms_min"], 4)}


class leg_range:
    """A named range around one leg (roctx through torch), so that a
    rocprofv3 --marker-trace run can attribute each kernel dispatch to its
    leg; the GPU is synchronised before the range closes."""

    def __init__(self, torch, name):
        self.torch, self.name = torch, name

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.torch.cuda.nvtx.range_push(self.name)

    def __exit__(self, *exc):
        self.torch.cuda.synchronize()
        self.torch.cuda.nvtx.range_pop()


# --------------------------------------------------------------- workloads

def decode_stages(ga, g, out, ws):
    msl = g.max_seq_len
    return [
        ("decode_split", lambda: ga.attn_sinks_decode_partials(
            g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.scale, ws, msl)),
        ("decode_merge", lambda: ga.attn_sinks_decode_merge(
            g.seq_lens, g.sinks, ws, out, g.num_kv_heads, msl)),
    ]


def decode_workspace(torch, ga, g):
    n = ga.attn_sinks_decode_workspace_bytes(g.num_seqs, g.num_q_heads, g.num_kv_heads,
                                             g.head_dim, g.max_seq_len)
    return torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")


def bench_decode(torch, ga, timer, batch_cpu, steps, warmup, label, with_warm=True):
    g = batch_cpu.to("cuda")
    out = torch.empty_like(g.q)
    ws = decode_workspace(torch, ga, g)
    nbytes = decode_bytes(batch_cpu)
    cold = timer.run(decode_stages(ga, g, out, ws), steps, warmup, flush=True)
    warm = timer.run(decode_stages(ga, g, out, ws), steps, warmup, flush=False) if with_warm \
        else cold
    gbs = nbytes / (cold["step_ms"] * 1e-3) / 1e9
    split_gbs = nbytes / (cold["stage_ms"]["decode_split"] * 1e-3) / 1e9
    res = {
        "workload": label,
        "algorithmic_bytes": nbytes,
        "ms": round(cold["step_ms"], 4),
        **spread(cold),
        "GB_per_s": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "split_ms": round(cold["stage_ms"]["decode_split"], 4),
        "merge_ms": round(cold["stage_ms"]["decode_merge"], 4),
        "split_GB_per_s": round(split_gbs, 1),
        "warm_GB_per_s": round(nbytes / (warm["step_ms"] * 1e-3) / 1e9, 1),
    }
    return res, out, (g, ws)


def bench_prefill(torch, ga, timer, batch_cpu, steps, warmup, label):
    g = batch_cpu.to("cuda")
    out = torch.empty_like(g.q)
    mq, ms = batch_cpu.max_q_len, batch_cpu.max_seq_len
    stage = [("prefill", lambda: ga.attn_sinks_prefill(
        g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.cu_seqlens_q, g.sinks, g.scale,
        out, mq, ms))]
    r = timer.run(stage, steps, warmup, flush=True)
    flops = prefill_flops(batch_cpu)
    tf = flops / (r["step_ms"] * 1e-3) / 1e12
    return {"workload": label, "algorithmic_flops": flops, "ms": round(r["step_ms"], 4),
            **spread(r), "TFLOP_per_s": round(tf, 1),
            "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}, out


def bench_window(torch, ga, timer, steps, warmup, wl, window=128):
    """The gpt-oss decode and prefill workloads under a sliding window of 128
    (the local layers of the "GPT OSS" notes, section 4.1): each call timed
    whole, against the HBM roofline (decode) and against the larger of the
    HBM and MFMA times (prefill)."""
    dec = wl.gptoss_decode(0)
    g = dec.to("cuda")
    out = torch.empty_like(g.q)
    ws = decode_workspace(torch, ga, g)
    r = timer.run([("decode_window", lambda: ga.attn_sinks_decode_window(
        g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.sinks, g.scale, window, out,
        ws, g.max_seq_len))], steps, warmup, flush=True)
    nb = window_decode_bytes(dec, window)
    d_gbs = nb / (r["step_ms"] * 1e-3) / 1e9
    del g, out, ws
    pre = wl.gptoss_prefill(0)
    gp = pre.to("cuda")
    outp = torch.empty_like(gp.q)
    rp = timer.run([("prefill_window", lambda: ga.attn_sinks_prefill_window(
        gp.q, gp.k_cache, gp.v_cache, gp.block_table, gp.seq_lens, gp.cu_seqlens_q, gp.sinks,
        gp.scale, window, outp, pre.max_q_len, pre.max_seq_len))], steps, warmup, flush=True)
    fl, pb = window_prefill_work(pre, window)
    t = rp["step_ms"] * 1e-3
    t_hbm, t_mfma = pb / (HBM_PEAK_GBS * 1e9), fl / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    return {
        "window": window,
        "decode": {"workload": f"gpt-oss decode workload, sliding window {window}",
                   "algorithmic_bytes": nb, "ms": round(r["step_ms"], 4),
                   "GB_per_s": round(d_gbs, 1), "hbm_frac": round(d_gbs / HBM_PEAK_GBS, 4)},
        "prefill": {"workload": f"gpt-oss prefill workload, sliding window {window}",
                    "algorithmic_flops": fl, "algorithmic_bytes": pb,
                    "ms": round(rp["step_ms"], 4),
                    "TFLOP_per_s": round(fl / t / 1e12, 1), "GB_per_s": round(pb / t / 1e9, 1),
                    "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                    "roofline_frac": round(max(t_hbm, t_mfma) / t, 4)},
    }


def bench_append(torch, ga, timer, steps, warmup, wl):
    """KV append ("GPT OSS" notes, section 3) of the gpt-oss prefill chunk
    (32768 tokens x 8 KV heads into their pages: read once, written once,
    against the HBM roofline), and the gpt-oss decode step with its append
    (attn_sinks_decode_append) next to the decode alone."""
    pre = wl.gptoss_prefill(0)
    before, k_new, v_new = wl.split_new_tokens(pre)
    g = before.to("cuda")
    kn, vn = k_new.cuda(), v_new.cuda()
    r = timer.run([("append", lambda: ga.attn_sinks_append_kv(
        kn, vn, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.cu_seqlens_q,
        before.max_seq_len))], steps, warmup, flush=True)
    nb = 2 * 2 * k_new.numel() * k_new.element_size()  # K and V, read and written
    nb += 4 * (g.num_seqs * 2 + 1)
    a_gbs = nb / (r["step_ms"] * 1e-3) / 1e9
    del g, kn, vn, before, pre
    dec = wl.gptoss_decode(0)
    dbefore, dk, dv = wl.split_new_tokens(dec)
    gd = dbefore.to("cuda")
    out = torch.empty_like(gd.q)
    ws = decode_workspace(torch, ga, gd)
    dkc, dvc = dk.cuda(), dv.cuda()
    rd = timer.run([("decode_append", lambda: ga.attn_sinks_decode_append(
        gd.q, dkc, dvc, gd.k_cache, gd.v_cache, gd.block_table, gd.seq_lens, gd.sinks,
        gd.scale, 0, out, ws, gd.max_seq_len))], steps, warmup, flush=True)
    return {
        "prefill_chunk_append": {
            "workload": "gpt-oss prefill chunk: 32768 tokens x 8 KV heads x 64, bf16",
            "bytes": nb, "ms": round(r["step_ms"], 4), "GB_per_s": round(a_gbs, 1),
            "hbm_frac": round(a_gbs / HBM_PEAK_GBS, 4)},
        "decode_step_with_append": {
            "workload": "gpt-oss decode workload, its 64 tokens appended first",
            "ms": round(rd["step_ms"], 4),
            "GB_per_s": round(decode_bytes(dec) / (rd["step_ms"] * 1e-3) / 1e9, 1)},
    }


def bench_rope(torch, ga, timer, steps, warmup, wl):
    """RoPE with YaRN scaling fused into the KV append ("GPT OSS" notes,
    sections 3 and 4.1) on the gpt-oss prefill chunk (32768 tokens, 64 q / 8
    KV heads, d 64, base 10000, scale 32, cache positions): q read and
    written in place, K and V read and written into their pages, against
    the HBM roofline."""
    pre = wl.gptoss_prefill(0)
    before, k_new, v_new = wl.split_new_tokens(pre)
    g = before.to("cuda")
    q = pre.q.cuda()
    kn, vn = k_new.cuda(), v_new.cuda()
    cu = pre.cu_seqlens_q.tolist()
    pos = []
    for b in range(pre.num_seqs):
        n = cu[b + 1] - cu[b]
        pos += [int(pre.seq_lens[b]) - n + i for i in range(n)]
    pos = torch.tensor(pos, dtype=torch.int32, device="cuda")
    r = timer.run([("rope_append", lambda: ga.attn_sinks_rope_append(
        q, kn, vn, pos, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.cu_seqlens_q,
        before.max_seq_len, 10000.0, 32.0))], steps, warmup, flush=True)
    nb = 2 * q.numel() * q.element_size() + 2 * 2 * kn.numel() * kn.element_size() + \
        pos.numel() * 4 + 4 * (g.num_seqs * 2 + 1)
    gbs = nb / (r["step_ms"] * 1e-3) / 1e9
    return {"workload": "gpt-oss prefill chunk: 32768 tokens, q 64 heads rotated in place, "
                        "K rotated and V appended into 8 KV heads' pages, d 64, bf16, YaRN "
                        "scale 32",
            "bytes": nb, "ms": round(r["step_ms"], 4), "GB_per_s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def bench_multi(torch, ga, timer, steps, warmup, wl, q_len=4):
    """Multi-token decode: the gpt-oss decode shape (64 seqs, L ~ U[1024,
    8192], 64/8 heads, d 64) with `q_len` new tokens per sequence, through
    attn_sinks_decode_multi (packed split passes) and, for comparison, the
    same call through attn_sinks_prefill.  Bytes: K and V of every key once,
    plus q and out of every new token."""
    gen = torch.Generator().manual_seed(0)
    L = torch.randint(1024, 8193, (64,), generator=gen, dtype=torch.int64).to(torch.int32)
    b = wl.build_batch(gen, "bf16", L, torch.full((64,), q_len, dtype=torch.int32), 64, 8, 64,
                       sink_mode="normal")
    g = b.to("cuda")
    out = torch.empty_like(g.q)
    nb = ga.attn_sinks_decode_multi_workspace_bytes(g.num_seqs, g.num_q_heads, g.num_kv_heads,
                                                    g.head_dim, b.max_seq_len, b.max_q_len)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    args = (g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.cu_seqlens_q, g.sinks,
            g.scale)
    r = timer.run([("multi", lambda: ga.attn_sinks_decode_multi(
        *args, out, ws, b.max_q_len, b.max_seq_len))], steps, warmup, flush=True)
    rp = timer.run([("as_prefill", lambda: ga.attn_sinks_prefill(
        *args, out, b.max_q_len, b.max_seq_len))], steps, warmup, flush=True)
    nbytes = b.algorithmic_kv_bytes() + 2 * b.q.numel() * 2 + \
        int(((L.long() + 15) // 16).sum()) * 4 + 4 * (2 * 64 + 1) + 4 * 64
    gbs = nbytes / (r["step_ms"] * 1e-3) / 1e9
    return {"workload": f"gpt-oss decode shape, {q_len} new tokens per sequence",
            "algorithmic_bytes": nbytes, "ms": round(r["step_ms"], 4),
            "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "same_call_as_prefill_ms": round(rp["step_ms"], 4)}


def bench_ragged(torch, ga, timer, steps, warmup, wl):
    """Ragged cache-free attention (contiguous K/V, LSE written) on the
    gpt-oss prefill shape, causal and unmasked, against the MFMA roofline."""
    r = wl.ragged_batch(0, "bf16", [4096] * 8, [4096] * 8, 64, 8, 64, sink_mode="normal")
    g = r.to("cuda")
    out = torch.empty_like(g.q)
    lse = torch.empty(g.q.shape[0], g.q.shape[1], dtype=torch.float32, device="cuda")
    res = {}
    for causal in (True, False):
        t = timer.run([("ragged", lambda: ga.attn_sinks_ragged(
            g.q, g.k, g.v, g.cu_seqlens_q, g.cu_seqlens_kv, g.sinks, g.scale, causal, out, lse,
            r.max_q_len, r.max_kv_len))], steps, warmup, flush=True)
        pairs = 8 * (4096 * 4097 // 2 if causal else 4096 * 4096)
        fl = 4 * 64 * 64 * pairs
        tf = fl / (t["step_ms"] * 1e-3) / 1e12
        res["causal" if causal else "unmasked"] = {
            "workload": "8 seqs x 4096 tokens, 64/8 heads, d 64, bf16, contiguous K/V, LSE out",
            "algorithmic_flops": fl, "ms": round(t["step_ms"], 4), "TFLOP_per_s": round(tf, 1),
            "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    return res


def bench_mixed(torch, ga, timer, steps, warmup, wl):
    """The mixed batch: the decode rows (split + merge) and the two prefill
    chunks, one after the other on one stream, and again with the decode half
    on a second stream beside the prefill half, and as one attn_sinks_mixed
    call (one launch for both halves, then the merge).  The decode half and the
    prefill half are each timed on their own as well as the whole step, with
    events only around what is timed (none between its launches)."""
    full, dec, pre = wl.mixed(0)
    gd, gp = dec.to("cuda"), pre.to("cuda")
    out_d, out_p = torch.empty_like(gd.q), torch.empty_like(gp.q)
    ws = decode_workspace(torch, ga, gd)
    dstages = decode_stages(ga, gd, out_d, ws)
    pstage = [("prefill", lambda: ga.attn_sinks_prefill(
        gp.q, gp.k_cache, gp.v_cache, gp.block_table, gp.seq_lens, gp.cu_seqlens_q, gp.sinks,
        gp.scale, out_p, pre.max_q_len, pre.max_seq_len))]
    rd = timer.run(dstages, steps, warmup, flush=True)
    rp = timer.run(pstage, steps, warmup, flush=True)
    r = timer.run(dstages + pstage, steps, warmup, flush=True)
    # The same step with the decode half on a second stream (default
    # priority), started together with the prefill half and joined before
    # the step's end event: the memory-bound decode's workgroups run beside
    # the compute-bound prefill's instead of before them.
    side = torch.cuda.Stream()

    def overlapped():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            for _, f in dstages:
                f()
        for _, f in pstage:
            f()
        main.wait_stream(side)

    ro = timer.run([("overlapped", overlapped)], steps, warmup, flush=True)
    # The same step as one attn_sinks_mixed call over the whole batch: the
    # decode rows' split pass and the chunks' prefill in one launch (the split
    # workgroups first), then the merge.
    gf = full.to("cuda")
    out_f = torch.empty_like(gf.q)
    ws_f = torch.empty(ga.attn_sinks_decode_workspace_bytes(
        dec.num_seqs, dec.num_q_heads, dec.num_kv_heads, dec.head_dim, dec.max_seq_len),
        dtype=torch.uint8, device="cuda")
    rm = timer.run([("one_launch", lambda: ga.attn_sinks_mixed(
        gf.q, gf.k_cache, gf.v_cache, gf.block_table, gf.seq_lens, gf.cu_seqlens_q, gf.sinks,
        gf.scale, out_f, dec.num_seqs, dec.max_seq_len, pre.max_q_len, pre.max_seq_len,
        ws_f))], steps, warmup, flush=True)
    if not (torch.equal(out_f[:dec.num_seqs], out_d) and torch.equal(out_f[dec.num_seqs:], out_p)):
        raise RuntimeError("attn_sinks_mixed differs from the decode and prefill calls")
    nb, fl = decode_bytes(dec), prefill_flops(pre)
    dec_ms, pre_ms = rd["step_ms"], rp["step_ms"]
    bound_ms = (nb / (HBM_PEAK_GBS * 1e9) + fl / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3
    return {"workload": "mixed: 32 decode seqs (ctx U[2048,16384]) + 2 prefill chunks of 2048 "
                        "on 8192-token prefixes, 64/8 heads, d=64, bf16, sinks N(0,2)",
            "ms": round(r["step_ms"], 4), **spread(r),
            "decode_ms": round(dec_ms, 4),
            "decode_split_ms": round(rd["stage_ms"]["decode_split"], 4),
            "decode_merge_ms": round(rd["stage_ms"]["decode_merge"], 4),
            "decode_algorithmic_bytes": nb,
            "decode_GB_per_s": round(nb / (dec_ms * 1e-3) / 1e9, 1),
            "decode_hbm_frac": round(nb / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "prefill_ms": round(pre_ms, 4),
            "prefill_algorithmic_flops": fl,
            "prefill_TFLOP_per_s": round(fl / (pre_ms * 1e-3) / 1e12, 1),
            "prefill_mfma_frac": round(fl / (pre_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "serial_bound_ms": round(bound_ms, 4),
            "frac_of_serial_bound": round(bound_ms / r["step_ms"], 4),
            "two_stream_ms": round(ro["step_ms"], 4),
            "two_stream_ms_median": round(ro["step_ms_median"], 4),
            "two_stream_frac_of_serial_bound": round(bound_ms / ro["step_ms"], 4),
            "one_launch_ms": round(rm["step_ms"], 4), "one_launch_ms_median":
            round(rm["step_ms_median"], 4),
            "one_launch_frac_of_serial_bound": round(bound_ms / rm["step_ms"], 4)}


# ------------------------------------------------------------ cpu baseline

def cpu_baseline(batch_cpu, gpu_out, sample_seqs, min_seconds=10.0):
    """The fp64 oracle on the first `sample_seqs` sequences of the decode
    workload, timed on this host's cores; the GPU output is checked on the
    same rows (the correctness gate before the timings are reported)."""
    import numpy as np
    import oracle
    sub = batch_cpu.rows(0, sample_seqs)
    threads = oracle.default_threads()
    oracle.attention(sub.rows(0, 1), threads=threads)  # load + warm
    # the whole sample, repeated until at least min_seconds of host work
    runs, t0 = 0, time.perf_counter()
    while True:
        ref = oracle.attention(sub, threads=threads)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    got = gpu_out[:sample_seqs].double().cpu().numpy()
    err = np.abs(got - ref)
    ok = bool(np.all(np.isfinite(got)) and np.all(err <= 1e-2 + 2e-2 * np.abs(ref)))
    nbytes = decode_bytes(sub)
    return {"value": round(nbytes * runs / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {sample_seqs} of 64 sequences of the gpt-oss decode workload "
                      f"({nbytes / 1e6:.1f} MB of K/V), all 64 heads, fp64, {runs} runs in "
                      f"{dt:.1f} s",
            "cpu_model": cpu_model(),
            "seconds": round(dt, 3),
            "gpu_matches_oracle": ok, "gpu_max_abs_err": float(err.max())}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _summary_fields(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def read_traffic(path, sources):
    """HBM traffic per launch from a committed counter summary, or None when
    the summary is missing or the kernel's sources changed since."""
    return read_counter(path, sources, "traffic_bytes_per_launch")


def read_counter(path, sources, field):
    if not os.path.exists(path):
        return None
    kv = _summary_fields(path)
    if kv.get("kernel_source_sha256_16") != source_hash(sources):
        return None
    try:
        return float(kv[field].split()[0])
    except (KeyError, ValueError, IndexError):
        return None


# ---------------------------------------------------- profile summarising

def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    import re
    name = name.replace("(anonymous namespace)::", "")
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\(.*$", "", name)[:80]


def _find(outdir, suffix):
    hits = glob.glob(os.path.join(outdir, "**", "*" + suffix), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {outdir}")
    return hits[0]


def summarize_trace(outdir: str, name: str, command: str):
    """profiles/<name>.txt: per-kernel durations from a --kernel-trace --stats run."""
    rows = _read_csv(_find(outdir, "kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel-trace summary: {name}", f"command: {command}", "",
             "kernel | calls | avg_us | min_us | max_us | total_ms | pct"]
    for r in rows:
        lines.append(f"{_short(r['Name'])} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}")
    hits = glob.glob(os.path.join(outdir, "**", "*kernel_trace.csv"), recursive=True)
    if hits:
        # the same kernels split by launch shape, so that each workload's
        # launches can be told apart; scratch 0 means no register spills
        shapes = {}
        for r in _read_csv(hits[0]):
            key = (_short(r["Kernel_Name"]), r["Grid_Size_X"], r["Grid_Size_Y"],
                   r["Grid_Size_Z"], r["Workgroup_Size_X"], r["VGPR_Count"],
                   r["Accum_VGPR_Count"], r["Scratch_Size"], r["LDS_Block_Size"])
            shapes.setdefault(key, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += ["", "by launch shape:",
                  "kernel | grid (threads) | block | vgpr | agpr | scratch | lds | calls | avg_us | min_us"]
        for key, ds in sorted(shapes.items(), key=lambda kv: -sum(kv[1])):
            k, gx, gy, gz, bx, vg, ag, sc, lds = key
            lines.append(f"{k} | {gx}x{gy}x{gz} | {bx} | {vg} | {ag} | {sc} | {lds} | "
                         f"{len(ds)} | {sum(ds) / len(ds):.2f} | {min(ds):.2f}")
    markers = glob.glob(os.path.join(outdir, "**", "*marker_api_trace.csv"), recursive=True)
    if hits and markers:
        # each dispatch attributed to the leg range (bench.py leg_range) that
        # holds its start
        # (the range's name is in "Function" in rocprofv3's marker csv)
        ranges = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                   r.get("Message") or r.get("Function"))
                  for r in _read_csv(markers[0]) if r.get("Message") or r.get("Function")]
        legs = {}
        for r in _read_csv(hits[0]):
            t0 = int(r["Start_Timestamp"])
            leg = next((m for a, b, m in ranges if a <= t0 <= b), None)
            if leg is None or "FillFunctor" in r["Kernel_Name"] or "copyBuffer" in r["Kernel_Name"]:
                continue
            key = (leg, _short(r["Kernel_Name"]), r["Grid_Size_X"], r["Grid_Size_Y"],
                   r["Grid_Size_Z"])
            legs.setdefault(key, []).append((int(r["End_Timestamp"]) - t0) / 1e3)
        lines += ["", "by leg (bench.py leg ranges; flush fills and copies left out):",
                  "leg | kernel | grid (threads) | calls | avg_us | median_us | min_us"]
        for key, ds in legs.items():
            leg, k, gx, gy, gz = key
            ds = sorted(ds)
            lines.append(f"{leg} | {k} | {gx}x{gy}x{gz} | {len(ds)} | {sum(ds) / len(ds):.2f} | "
                         f"{ds[len(ds) // 2]:.2f} | {ds[0]:.2f}")
    _write_profile(name, lines)


def summarize_traffic(fetch_dir: str, write_dir: str, kernel: str, name: str, command: str):
    """profiles/<name>.txt: HBM bytes per launch of `kernel` from one FETCH_SIZE
    and one WRITE_SIZE run, each scaled by what the counter reads for the
    1 GiB device copy made by --profile-run."""
    calib = 1 << 30
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _read_csv(_find(d, "counter_collection.csv"))
                if r["Counter_Name"] == counter]
        copy = max((float(r["Counter_Value"]) for r in rows
                    if "copyBuffer" in r["Kernel_Name"]), default=0.0)
        vals = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
        if not copy or not vals:
            raise SystemExit(f"{counter}: copy or {kernel} dispatches missing")
        factor = calib / (copy * 1024.0)
        out[counter] = (sum(vals) / len(vals), len(vals), copy, factor)
    fetch, write = out["FETCH_SIZE"], out["WRITE_SIZE"]
    traffic = (fetch[0] * fetch[3] + write[0] * write[3]) * 1024.0
    lines = [f"# rocprofv3 HBM traffic summary: {name}", f"command: {command}",
             f"kernel: {kernel}",
             f"kernel_source_sha256_16: {source_hash(kernel_sources(kernel))}",
             f"copy_calibration_bytes: {calib}",
             f"fetch_kib_copy: {fetch[2]:.1f}",
             f"fetch_scale: {fetch[3]:.4f}",
             f"write_kib_copy: {write[2]:.1f}",
             f"write_scale: {write[3]:.4f}",
             f"fetch_kib_per_dispatch: {fetch[0]:.1f}  ({fetch[1]} dispatches)",
             f"write_kib_per_dispatch: {write[0]:.1f}  ({write[1]} dispatches)",
             f"traffic_bytes_per_launch: {traffic:.0f}"]
    _write_profile(name, lines)


# MI355X: 8 XCDs of 32 CUs, 4 SIMDs per CU.
XCDS, SIMDS = 8, 1024


def summarize_counters(outdir: str, kernel: str, name: str, command: str):
    """profiles/<name>.txt: per-dispatch averages of every counter collected
    for `kernel` (rocprofv3 --pmc runs under DIR), with derived figures.

    rocprofv3's csv gives each counter summed over its hardware instances.
    GRBM_GUI_ACTIVE counts every XCD's busy cycles, so /8 is the kernel's span
    in cycles; SQ_VALU_MFMA_BUSY_CYCLES counts each SIMD's matrix-core busy
    cycles, so over (SIMDs x span) it is the matrix cores' busy fraction.  The
    SQ_* wave counters (SQ_WAVE_CYCLES, SQ_ACTIVE_INST_*) count in units of 4
    cycles, summed over waves."""
    files = glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {outdir}")
    vals, durs = {}, []
    for f in files:
        for r in _read_csv(f):
            if kernel not in r["Kernel_Name"]:
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            durs.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if not vals:
        raise SystemExit(f"no dispatch of {kernel} under {outdir}")
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    dur_ns = sum(durs) / len(durs)
    lines = [f"# rocprofv3 counter summary: {name}", f"command: {command}", f"kernel: {kernel}",
             f"kernel_source_sha256_16: {source_hash(kernel_sources(kernel))}",
             f"dispatch_avg_ns_under_counters: {dur_ns:.0f}", "",
             "counter | per-dispatch average | dispatches"]
    for k in sorted(avg):
        lines.append(f"{k} | {avg[k]:.6g} | {len(vals[k])}")
    lines.append("")
    span = avg.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
    if span:
        lines.append(f"span_cycles: {span:.0f}  (GRBM_GUI_ACTIVE / 8 XCDs)")
        lines.append(f"implied_clock_ghz: {span / dur_ns:.3f}  (span / dispatch duration)")
    if span and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        lines.append(f"mfma_busy_frac: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * span):.4f}"
                     "  (SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x span))")
    if span and "SQ_ACTIVE_INST_VALU" in avg:
        lines.append(f"valu_active_frac_per_simd: "
                     f"{4 * avg['SQ_ACTIVE_INST_VALU'] / (SIMDS * span):.4f}"
                     "  (4 x SQ_ACTIVE_INST_VALU / (1024 SIMDs x span); summed over the "
                     "SIMD's waves, MFMA issue included)")
    if span and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
        lines.append(f"valu_mfma_coexec_frac: "
                     f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / (SIMDS * span):.4f}"
                     "  (SQ_VALU_MFMA_COEXEC_CYCLES / (1024 SIMDs x span))")
    if "SQ_INSTS_VALU" in avg and avg.get("SQ_INSTS_MFMA"):
        lines.append(f"valu_insts_per_mfma_inst: "
                     f"{(avg['SQ_INSTS_VALU'] - avg['SQ_INSTS_MFMA']) / avg['SQ_INSTS_MFMA']:.2f}"
                     "  ((SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA)")
    _write_profile(name, lines)


def _write_profile(name, lines):
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, name + ".txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# -------------------------------------------------------------------- main

LEGS = ("decode", "prefill", "mixed", "next", "qwen")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", *LEGS], default="all",
                    help="run only the headline decode plus this leg (with --profile-run: "
                         "only this leg); next = the window, multi-token, ragged, KV-append "
                         "and RoPE-append legs")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "NAME"))
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "KERNEL", "NAME"))
    ap.add_argument("--summarize-counters", nargs=3, metavar=("DIR", "KERNEL", "NAME"))
    ap.add_argument("--command", default="", help="command line recorded in the summary")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.command)
        return 0
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.command)
        return 0
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.command)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library's path runs on a single MI355X "
              "and has no multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import gqa_paged_attention_amd as ga
    from gqa_paged_attention_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    ga.library()
    torch.cuda.set_device(0)
    flush_buf = torch.empty(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB
    timer = Timer(torch, flush_buf)
    K, W = args.steps, args.warmup
    legs = set(LEGS) if args.only == "all" else {args.only}
    # the headline decode always runs, except in a profile run of another leg
    run_headline = not args.profile_run or args.only in ("all", "decode")

    label = ("gpt-oss-20b-shaped decode, bf16: 64 seqs x 1 token, 64 q / 8 KV heads, "
             "head_dim 64, ctx U[1024,8192], 16-token HND pages, random page table, "
             "q/k/v/sinks N(0,1), seed 0")
    d_res = d_out = dec = None
    if run_headline:
        log("generating gpt-oss decode workload")
        dec = wl.gptoss_decode(0)
        log("timing decode")
        with leg_range(torch, "gptoss_decode"):
            d_res, d_out, _ = bench_decode(torch, ga, timer, dec, K, W, label,
                                           with_warm=not args.profile_run)
        log(json.dumps(d_res))

    extra = {}
    if "prefill" in legs:
        log("generating gpt-oss prefill workload")
        pre = wl.gptoss_prefill(0)
        with leg_range(torch, "gptoss_prefill"):
            p_res, _ = bench_prefill(torch, ga, timer, pre, K, W,
                                     "gpt-oss-shaped causal prefill, bf16: 8 seqs x 4096 "
                                     "tokens, 64 q / 8 KV heads, head_dim 64, sinks N(0,1), "
                                     "seed 0")
        del pre
        log(json.dumps(p_res))
        extra["prefill"] = p_res
    if "mixed" in legs:
        log("generating mixed workload")
        with leg_range(torch, "mixed"):
            extra["mixed"] = bench_mixed(torch, ga, timer, K, W, wl)
        log(json.dumps(extra["mixed"]))
    if "next" in legs:
        log("sliding-window legs (window 128)")
        with leg_range(torch, "window128"):
            extra["sliding_window"] = bench_window(torch, ga, timer, K, W, wl)
        log(json.dumps(extra["sliding_window"]))
        log("multi-token decode leg")
        with leg_range(torch, "multi_token_decode"):
            extra["multi_token_decode"] = bench_multi(torch, ga, timer, K, W, wl)
        log(json.dumps(extra["multi_token_decode"]))
        log("ragged cache-free legs")
        with leg_range(torch, "ragged"):
            extra["ragged"] = bench_ragged(torch, ga, timer, K, W, wl)
        log(json.dumps(extra["ragged"]))
        log("KV append legs")
        with leg_range(torch, "kv_append"):
            extra["kv_append"] = bench_append(torch, ga, timer, K, W, wl)
        log(json.dumps(extra["kv_append"]))
        log("RoPE + KV append leg")
        with leg_range(torch, "rope_append"):
            extra["rope_append"] = bench_rope(torch, ga, timer, K, W, wl)
        log(json.dumps(extra["rope_append"]))
    if "qwen" in legs:
        log("generating qwen decode workload (about a minute)")
        qw = wl.qwen_decode(0)
        with leg_range(torch, "qwen_decode"):
            q_res, _, keep = bench_decode(torch, ga, timer, qw, max(K // 2, 3),
                                          max(W // 2, 1),
                                          "Qwen3-235B-shaped decode, bf16: 128 seqs x 1 token, "
                                          "64 q / 4 KV heads, head_dim 128, ctx "
                                          "U[4096,32768], sinks -inf, seed 0",
                                          with_warm=not args.profile_run)
        del keep, qw
        extra["qwen_decode"] = q_res
        log(json.dumps(q_res))
        qp = wl.qwen_prefill(0)
        with leg_range(torch, "qwen_prefill"):
            qp_res, _ = bench_prefill(torch, ga, timer, qp, max(K // 2, 3), max(W // 2, 1),
                                      "Qwen3-235B-shaped causal prefill, bf16: 4 seqs x 4096 "
                                      "tokens, 64 q / 4 KV heads, head_dim 128, sinks -inf, "
                                      "seed 0")
        del qp
        extra["qwen_prefill"] = qp_res
        log(json.dumps(qp_res))

    if args.profile_run:
        # a plain 1 GiB device copy: its FETCH_SIZE / WRITE_SIZE counters give
        # the factor between counter units and bytes
        src = torch.empty(1 << 28, dtype=torch.int32, device="cuda").fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(json.dumps({"profile_run": True, "decode": d_res, **extra,
                        "copy_calibration_bytes": src.numel() * 4}))
        return 0

    log("cpu baseline: oracle on the host cores")
    cpu = cpu_baseline(dec, d_out.cpu(), sample_seqs=64)
    log(json.dumps(cpu))
    if not cpu["gpu_matches_oracle"]:
        print("GPU decode output does not match the oracle; refusing to report", file=sys.stderr)
        return 1

    traffic = read_traffic(TRAFFIC_FILE, DECODE_SOURCES)
    split_launch_bytes = d_res["algorithmic_bytes"]
    achieved = d_res["split_GB_per_s"]
    line = {
        "metric": "decode KV-read GB/s (% HBM peak); prefill attention TFLOPS (% MFMA peak)",
        "value": d_res["GB_per_s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": d_res["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": label, "parallelism": "single GPU",
                   "hbm_frac": d_res["hbm_frac"], "warm_GB_per_s": d_res["warm_GB_per_s"],
                   "ms_median": d_res["ms_median"], "ms_min": d_res["ms_min"],
                   "split_ms": d_res["split_ms"], "merge_ms": d_res["merge_ms"]},
        "roofline": {"bound": "hbm", "kernel": "decode_split_bf16<64>",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": split_launch_bytes},
        "cpu_baseline": {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
        **extra,
    }
    if "prefill" in extra:
        p = extra["prefill"]
        line["prefill_roofline"] = {
            "bound": "mfma", "kernel": "prefill_bf16<64>", "achieved": p["TFLOP_per_s"],
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": p["mfma_frac"],
            "traffic": read_traffic(PREFILL_TRAFFIC_FILE, PREFILL_SOURCES),
            "mfma_busy": read_counter(PREFILL_COUNTER_FILE, PREFILL_SOURCES, "mfma_busy_frac")}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
