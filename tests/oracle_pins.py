"""Pins that tie the oracle to facts other than its own code.

Each pin takes `attn(batch, with_lse=False, window=0)` -- a callable with the
oracle's signature -- and raises AssertionError when the callable disagrees with what
the pages or the mathematics fix.  test_oracle.py runs them on the oracle;
test_oracle_mutants.py runs them on copies of oracle.c with planted mistakes
and checks that every mistake is caught by at least one pin.

The facts used:
  * hand-worked cases (tests/golden/handworked.json) from the definition in the
    "GPT OSS" model notes, section 3 and sections 1 / 4.1;
  * the pure-Python virtual-token brute force (oracle/brute.py);
  * sink = -inf is plain softmax attention: torch's fp64 CPU
    scaled_dot_product_attention with GQA and a bottom-right causal mask;
  * closed form: with a sink, out = SDPA * sigmoid(LSE - sink), where LSE is
    the log-sum-exp of the visible logits (torch.logsumexp);
  * sink = LSE halves the output; a sink far above LSE drives it to 0;
  * a single visible key gives v_0 * sigmoid(s_0 - sink);
  * permuting physical pages leaves the result bit-identical;
  * a prefill row equals a decode call truncated at that row's position;
  * sliding window ("GPT OSS" model notes, section 4.1: a local window of W
    positions on even layers; section 11: the window is passed per call):
    a window at least as long as the sequence changes nothing; the brute
    force with the same window; plain softmax attention under a band mask
    (torch SDPA) times sigmoid(LSE - sink); W = 1 is the single-key closed
    form on the query's own key; and a windowed decode equals an unwindowed
    decode over a pool that holds only the last W tokens;
  * without the causal mask (ragged, cache-free attention of embedding
    models, "Fast embeddings on GPUs"): the brute force and unmasked SDPA
    times sigmoid(LSE - sink);
  * the LSE the oracle reports is log(sum_j e^(s_j) + e^sink), i.e.
    torch.logaddexp(torch.logsumexp(visible logits), sink);
  * KV append (model notes, section 3: K and V are appended before the
    attention step): appending the newest tokens into a pool where their
    slots are blank rebuilds, bit for bit, the pool the input generator laid
    out with those tokens already in place; the tiny workload's documented
    slot of token 256 is the one written.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

from dataclasses import replace

import numpy as np
import torch
import torch.nn.functional as F

from gqa_paged_attention_amd import workloads as wl
from oracle.brute import brute_force

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "handworked.json")


# ---------------------------------------------------------------- references

def sdpa_reference(batch, window=0, causal=True):
    """Plain softmax attention (no sink) and per-row LSE, via torch fp64 CPU.

    Uses the logical K/V rows kept by the generator, GQA through
    enable_gqa=True, and an explicit bottom-right causal mask (a band of the
    last `window` positions when window > 0; every key when causal=False).
    Returns (out [total_q][Hq][d], lse [total_q][Hq]) as numpy fp64.
    """
    assert batch.k_logical is not None, "build the batch with keep_logical=True"
    outs, lses = [], []
    cu = batch.cu_seqlens_q.tolist()
    offs = batch.kv_offsets.tolist()
    for b in range(batch.num_seqs):
        L = int(batch.seq_lens[b])
        nq = cu[b + 1] - cu[b]
        if nq == 0:
            continue
        q = batch.q[cu[b]:cu[b + 1]].double().permute(1, 0, 2).unsqueeze(0)   # 1,Hq,nq,d
        k = batch.k_logical[offs[b]:offs[b] + L].double().permute(1, 0, 2).unsqueeze(0)
        v = batch.v_logical[offs[b]:offs[b] + L].double().permute(1, 0, 2).unsqueeze(0)
        i = torch.arange(nq).unsqueeze(1)
        j = torch.arange(L).unsqueeze(0)
        mask = j <= (L - nq + i)                                               # nq, L
        if not causal:
            mask = torch.ones_like(mask)
        if window > 0:
            mask = mask & (j > (L - nq + i) - window)
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=batch.scale,
                                           enable_gqa=True)
        G = batch.num_q_heads // batch.num_kv_heads
        kk = k.repeat_interleave(G, dim=1)
        logits = torch.matmul(q, kk.transpose(-1, -2).contiguous()) * batch.scale
        logits = logits.masked_fill(~mask, float("-inf"))
        lse = torch.logsumexp(logits, dim=-1)                                  # 1,Hq,nq
        outs.append(o[0].permute(1, 0, 2))
        lses.append(lse[0].permute(1, 0))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.abs(a - b)
    bad = err > atol + rtol * np.abs(b)
    assert not bad.any(), f"{what}: max abs err {err.max():.3e} at {np.argwhere(bad)[0]}"


# -------------------------------------------------------------------- inputs

def _val(x, ln):
    if isinstance(x, str):
        if x == "-inf":
            return float("-inf")
        if x.startswith("2ln"):
            return 2.0 * ln[x[1:]]
        return ln[x]
    return float(x)


def golden_cases():
    data = json.load(open(GOLDEN))
    ln = data["ln"]
    out = []
    for c in data["cases"]:
        conv = lambda a: [[[_val(x, ln) for x in row] for row in tok] for tok in a]
        q = torch.tensor(conv(c["q"]), dtype=torch.float64)
        k = torch.tensor(conv(c["k"]), dtype=torch.float64)
        v = torch.tensor(conv(c["v"]), dtype=torch.float64)
        sinks = [_val(x, ln) for x in c["sinks"]]
        expected = np.array([[[float(Fraction(x)) for x in row] for row in tok]
                             for tok in c["expected"]])
        out.append((c["name"], q, k, v, c["seq_lens"], c["q_lens"], sinks, c["scale"], expected))
    return out


def tiny_batches():
    """Small mixed decode/prefill batches with random page tables."""
    cases = []
    specs = [
        # seed, dtype, seq_lens, q_lens, Hq, Hkv, d, sink_mode, sink_std
        (1, "f32", [5, 17], [1, 1], 4, 2, 8, "normal", 1.0),
        (2, "bf16", [33, 1, 16], [4, 1, 16], 4, 1, 4, "normal", 3.0),
        (3, "f32", [40], [40], 2, 2, 8, "neginf", 1.0),
        (4, "bf16", [20, 31], [2, 7], 6, 3, 4, "none", 1.0),
        (5, "f32", [12, 29], [1, 29], 4, 4, 8, "normal", 0.5),
    ]
    for seed, dt, L, Lq, Hq, Hkv, d, sm, sd in specs:
        cases.append(wl.small_batch(seed, dt, L, Lq, Hq, Hkv, d, sink_mode=sm, sink_std=sd,
                                    keep_logical=True))
    return cases


def medium_batch(seed, sink_mode="normal", dtype="f32", sink_std=1.0):
    return wl.small_batch(seed, dtype, [70, 129, 16, 1], [1, 33, 16, 1], 8, 2, 64,
                          sink_mode=sink_mode, sink_std=sink_std, keep_logical=True)


# ---------------------------------------------------------------------- pins

def pin_golden(attn):
    for name, q, k, v, L, Lq, sinks, scale, expected in golden_cases():
        for perm_seed in (0, 1, 2):
            b = wl.from_logical("f32", q, k, v, L, Lq, sinks, scale, perm_seed=perm_seed,
                                spare_pages=2)
            _close(attn(b), expected, 1e-6, 1e-7, f"golden {name} (perm {perm_seed})")


def pin_brute(attn):
    for b in tiny_batches():
        ref = np.array(brute_force(b))
        _close(attn(b), ref, 1e-12, 1e-13, f"brute force {b.dtype} L={b.seq_lens.tolist()}")


def pin_plain_is_sdpa(attn):
    for seed, mode in ((11, "neginf"), (12, "none")):
        for dt in ("f32", "bf16"):
            b = medium_batch(seed, sink_mode=mode, dtype=dt)
            ref, _ = sdpa_reference(b)
            _close(attn(b), ref, 1e-12, 1e-13, f"sink=-inf vs SDPA ({mode}, {dt})")


def pin_closed_form(attn):
    for seed, std in ((21, 1.0), (22, 4.0)):
        b = medium_batch(seed, sink_std=std)
        ref, lse = sdpa_reference(b)
        sink = b.sinks.double().numpy()[None, :]
        expect = ref * sigmoid(lse - sink)[..., None]
        _close(attn(b), expect, 1e-11, 1e-13, f"closed form (sink std {std})")


def pin_large_and_half_sink(attn):
    # decode batch: one row per head, so a per-head sink can be set per row
    base = wl.small_batch(31, "f32", [90], [1], 8, 2, 64, sink_mode="neginf", keep_logical=True)
    ref, lse = sdpa_reference(base)
    lse = lse[0]
    # sink = LSE: the sink takes exactly half of the softmax mass
    half = wl.small_batch(31, "f32", [90], [1], 8, 2, 64, sink_mode="neginf", keep_logical=True)
    half.sinks = torch.tensor(lse, dtype=torch.float32)
    lse32 = half.sinks.double().numpy()
    expect = ref * sigmoid(lse - lse32)[None, :, None]
    _close(attn(half), expect, 1e-11, 1e-13, "sink = LSE")
    _close(attn(half), ref / 2.0, 1e-6, 1e-8, "sink = LSE halves the output")
    # sink = LSE + 50: |out| <= exp(LSE - sink) * max|v|
    big = wl.small_batch(31, "f32", [90], [1], 8, 2, 64, sink_mode="neginf", keep_logical=True)
    big.sinks = torch.tensor(lse + 50.0, dtype=torch.float32)
    got = attn(big)
    bound = math.exp(-49.0) * float(big.v_logical.abs().max())
    assert np.all(np.abs(got) <= bound), f"large sink: max |out| {np.abs(got).max():.3e}"
    assert np.any(np.abs(got) > 0.0), "large sink: output vanished exactly (sink too strong?)"


def pin_single_key(attn):
    # prefill with Lq = L: row 0 of each sequence sees exactly key 0
    b = wl.small_batch(41, "f32", [9, 25], [9, 25], 4, 2, 16, sink_mode="normal",
                       sink_std=1.5, keep_logical=True)
    got = attn(b)
    G = b.num_q_heads // b.num_kv_heads
    for s, row in ((0, 0), (1, 9)):
        k0 = b.k_logical[int(b.kv_offsets[s])].double()
        v0 = b.v_logical[int(b.kv_offsets[s])].double()
        for h in range(b.num_q_heads):
            s0 = float(b.scale * (b.q[row, h].double() @ k0[h // G]))
            w = 1.0 / (1.0 + math.exp(float(b.sinks[h]) - s0))
            _close(got[row, h], (v0[h // G] * w).numpy(), 1e-12, 1e-14, "single key")


def pin_page_permutation(attn):
    b = medium_batch(51)
    ref = attn(b)
    gen = torch.Generator().manual_seed(52)
    perm = torch.randperm(b.num_pages, generator=gen)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(b.num_pages)
    # move physical page p to slot inv[p]; rewrite the table accordingly
    k2 = torch.empty_like(b.k_cache)
    v2 = torch.empty_like(b.v_cache)
    k2[inv] = b.k_cache
    v2[inv] = b.v_cache
    bt = b.block_table.clone().to(torch.int64)
    valid = bt >= 0
    bt[valid] = inv[bt[valid]]
    from dataclasses import replace
    b2 = replace(b, k_cache=k2, v_cache=v2, block_table=bt.to(torch.int32))
    got = attn(b2)
    assert np.array_equal(got, ref), "page permutation changed the result"


def pin_prefill_row_is_decode(attn):
    b = wl.small_batch(61, "bf16", [48], [20], 4, 2, 32, sink_mode="normal", keep_logical=True)
    full = attn(b)
    from dataclasses import replace
    for i in (0, 7, 19):
        L = 48 - 20 + i + 1
        d = replace(b, seq_lens=torch.tensor([L], dtype=torch.int32),
                    cu_seqlens_q=torch.tensor([0, 1], dtype=torch.int32),
                    q=b.q[i:i + 1].contiguous())
        assert np.array_equal(attn(d)[0], full[i]), f"prefill row {i} differs from decode"


def pin_gqa_groups(attn):
    b = wl.small_batch(71, "f32", [37], [1], 8, 2, 16, sink_mode="normal", keep_logical=True)
    G = 4
    b.q[:, 1] = b.q[:, 0]          # heads 0, 1 share KV head 0
    b.q[:, 4] = b.q[:, 0]          # head 4 uses KV head 1
    b.sinks[1] = b.sinks[0]
    b.sinks[4] = b.sinks[0]
    got = attn(b)
    assert np.array_equal(got[0, 0], got[0, 1]), "heads of one group differ"
    assert not np.allclose(got[0, 0], got[0, G]), "heads of different groups agree"


def pin_empty_rows(attn):
    b = wl.small_batch(81, "f32", [0, 5], [0, 1], 2, 1, 8, sink_mode="normal", keep_logical=True)
    got = attn(b)
    assert got.shape[0] == 1 and np.all(np.isfinite(got))
    # a decode row whose only visible set is empty: seq_lens 0 with a query row
    e = wl.small_batch(82, "f32", [1], [1], 2, 1, 8, sink_mode="normal")
    from dataclasses import replace
    e = replace(e, seq_lens=torch.tensor([0], dtype=torch.int32))
    assert np.all(attn(e) == 0.0), "empty visible set with a finite sink must give 0"
    e = replace(e, sinks=None)
    assert np.all(attn(e) == 0.0), "empty visible set with no sink must give 0"


# ------------------------------------------------------------ sliding window

def pin_window_wide_is_full(attn):
    b = medium_batch(101)
    full = attn(b)
    for w in (int(b.seq_lens.max()), int(b.seq_lens.max()) + 7, 10 ** 6):
        assert np.array_equal(attn(b, window=w), full), f"window {w} >= L changed the result"


def pin_window_brute(attn):
    for b, w in zip(tiny_batches(), (1, 3, 7, 16, 5)):
        ref = np.array(brute_force(b, window=w))
        _close(attn(b, window=w), ref, 1e-12, 1e-13, f"brute force, window {w}")


def pin_window_band_sdpa(attn):
    for seed, w, mode in ((111, 5, "normal"), (112, 24, "normal"), (113, 9, "neginf")):
        b = medium_batch(seed, sink_mode=mode)
        ref, lse = sdpa_reference(b, window=w)
        if mode == "normal":
            sink = b.sinks.double().numpy()[None, :]
            ref = ref * sigmoid(lse - sink)[..., None]
        _close(attn(b, window=w), ref, 1e-11, 1e-13, f"band-masked SDPA, window {w}")


def pin_window_one(attn):
    # W = 1: every row sees only its own position's key
    b = wl.small_batch(121, "f32", [30, 12], [6, 12], 4, 2, 16, sink_mode="normal",
                       sink_std=1.5, keep_logical=True)
    got = attn(b, window=1)
    G = b.num_q_heads // b.num_kv_heads
    cu, offs = b.cu_seqlens_q.tolist(), b.kv_offsets.tolist()
    for s in range(b.num_seqs):
        L, nq = int(b.seq_lens[s]), cu[s + 1] - cu[s]
        for i in range(nq):
            kp = b.k_logical[offs[s] + L - nq + i].double()
            vp = b.v_logical[offs[s] + L - nq + i].double()
            for h in range(b.num_q_heads):
                sp = float(b.scale * (b.q[cu[s] + i, h].double() @ kp[h // G]))
                wgt = 1.0 / (1.0 + math.exp(float(b.sinks[h]) - sp))
                _close(got[cu[s] + i, h], (vp[h // G] * wgt).numpy(), 1e-12, 1e-14,
                       "window 1")


def pin_window_truncation(attn):
    # a windowed decode equals an unwindowed decode whose pool holds only
    # the last W tokens of each sequence
    b = wl.small_batch(131, "bf16", [70, 9, 129, 33], [1, 1, 1, 1], 8, 2, 32,
                       sink_mode="normal", keep_logical=True)
    offs = b.kv_offsets.tolist()
    for w in (1, 16, 40):
        ks, vs, lens = [], [], []
        for s in range(b.num_seqs):
            L = int(b.seq_lens[s])
            lo = max(0, L - w)
            ks.append(b.k_logical[offs[s] + lo:offs[s] + L])
            vs.append(b.v_logical[offs[s] + lo:offs[s] + L])
            lens.append(L - lo)
        t = wl.from_logical("bf16", b.q.float(), torch.cat(ks).float(), torch.cat(vs).float(),
                            lens, [1] * b.num_seqs, b.sinks, b.scale, perm_seed=w,
                            spare_pages=3)
        _close(attn(b, window=w), attn(t), 1e-12, 1e-14, f"window {w} vs truncated pool")


# ------------------------------------------------------ no causal mask, LSE

def pin_noncausal_brute(attn):
    for b in tiny_batches():
        ref = np.array(brute_force(b, causal=False))
        _close(attn(b, causal=False), ref, 1e-12, 1e-13, f"brute force, no mask {b.dtype}")


def pin_noncausal_sdpa(attn):
    for seed, mode in ((151, "normal"), (152, "neginf")):
        b = medium_batch(seed, sink_mode=mode)
        ref, lse = sdpa_reference(b, causal=False)
        if mode == "normal":
            ref = ref * sigmoid(lse - b.sinks.double().numpy()[None, :])[..., None]
        _close(attn(b, causal=False), ref, 1e-11, 1e-13, f"unmasked SDPA ({mode})")


def pin_lse(attn):
    for seed, causal in ((161, True), (162, False)):
        b = medium_batch(seed)
        _, lse = attn(b, with_lse=True, causal=causal)
        _, lse_keys = sdpa_reference(b, causal=causal)
        expect = np.logaddexp(lse_keys, b.sinks.double().numpy()[None, :])
        _close(lse, expect, 1e-12, 1e-12, f"LSE with the sink (causal {causal})")
        nb = replace(b, sinks=None)
        _, lse0 = attn(nb, with_lse=True, causal=causal)
        _close(lse0, lse_keys, 1e-12, 1e-12, f"LSE without a sink (causal {causal})")


# ----------------------------------------------------------------- KV append

def _same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def check_append(append):
    """`append(batch, k_new, v_new) -> (k_cache, v_cache)` against the pools
    the generator lays out directly."""
    for seed, dt, L, Lq, Hkv, d in ((141, "bf16", [33, 1, 70, 16], [4, 1, 70, 16], 2, 64),
                                     (142, "f32", [5, 129, 64], [5, 30, 1], 3, 128),
                                     (143, "bf16", [0, 17, 40], [0, 17, 2], 1, 64)):
        full = wl.small_batch(seed, dt, L, Lq, 4 * Hkv, Hkv, d, sink_mode="normal")
        before, k_new, v_new = wl.split_new_tokens(full)
        assert not _same_bits(before.k_cache, full.k_cache) or sum(Lq) == 0
        k, v = append(before, k_new, v_new)
        assert _same_bits(k, full.k_cache), f"append K differs (seed {seed})"
        assert _same_bits(v, full.v_cache), f"append V differs (seed {seed})"
    pre, dec, (page, slot, nk, nv) = wl.tiny_fp32(0)
    q1 = replace(dec, cu_seqlens_q=torch.tensor([0, 1], dtype=torch.int32))
    k, v = append(replace(q1, k_cache=pre.k_cache, v_cache=pre.v_cache), nk[None], nv[None])
    assert _same_bits(k[page, :, slot], nk) and _same_bits(v[page, :, slot], nv)
    assert _same_bits(k, dec.k_cache) and _same_bits(v, dec.v_cache)


def pin_append(attn):
    """The oracle's append (independent of `attn`, which it does not use)."""
    import oracle
    check_append(oracle.append_kv)


ALL_PINS = [pin_golden, pin_brute, pin_plain_is_sdpa, pin_closed_form, pin_large_and_half_sink,
            pin_single_key, pin_page_permutation, pin_prefill_row_is_decode, pin_gqa_groups,
            pin_empty_rows, pin_window_wide_is_full, pin_window_brute, pin_window_band_sdpa,
            pin_window_one, pin_window_truncation, pin_append, pin_noncausal_brute,
            pin_noncausal_sdpa, pin_lse]
