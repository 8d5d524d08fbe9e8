"""GPU parity of the sliding-window entry points against the windowed oracle.

The window follows the "GPT OSS" model notes (section 4.1: even layers
attend within a local window, 128 by default; section 11: the window is
passed per call): the query at position p sees keys p - W + 1 .. p and the
sink.  Cases cover windows shorter than, equal to and longer than the
32-token decode blocks and 16-token pages, windows that start mid-page,
sequences shorter than the window, chunks over cached prefixes, both head
dims and fp32, plus the full-size gpt-oss shapes at W = 128.
"""
import zlib
from dataclasses import replace

import pytest
import torch

import gqa_paged_attention_amd as ga
from gqa_paged_attention_amd import workloads as wl
from tests.gpu_helpers import (aligned_scores, check_sampled, compare, note, oracle_full,
                               run_decode, run_prefill, scale_keys)

pytestmark = pytest.mark.gpu

WINDOWS = [1, 5, 16, 31, 32, 33, 100, 128, 1000]

DECODE_CASES = [
    # id, dtype, seq_lens, Hq, Hkv, d, sink_mode
    ("d64_g8", "bf16", [1, 15, 16, 17, 33, 100, 129, 1000, 2049], 16, 2, 64, "normal"),
    ("d128_g16", "bf16", [1, 31, 32, 200, 2049], 32, 2, 128, "normal"),
    ("d64_g1_nosink", "bf16", [7, 300, 64, 4097], 4, 4, 64, "none"),
    ("f32_d64", "f32", [1, 17, 300], 8, 2, 64, "normal"),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_window(case):
    name, dt, L, Hq, Hkv, d, sm = case
    b = wl.small_batch(zlib.crc32(name.encode()) % 1000 + 3, dt, L, [1] * len(L), Hq, Hkv, d,
                       sink_mode=sm)
    for w in WINDOWS:
        note(f"decode window {w} {name}: L={L} Hq={Hq} Hkv={Hkv} d={d} {dt}")
        compare(run_decode(b, window=w), oracle_full(b, window=w), dt,
                f"decode {name} window {w}")


PREFILL_CASES = [
    # id, dtype, seq_lens, q_lens, Hq, Hkv, d, sink_mode
    ("d64_full_causal", "bf16", [1, 17, 130, 300, 600], [1, 17, 130, 300, 600], 16, 2, 64,
     "normal"),
    ("d64_chunks_over_prefix", "bf16", [500, 1000, 64], [100, 257, 1], 16, 2, 64, "normal"),
    ("d128_full", "bf16", [200, 333], [200, 333], 8, 2, 128, "normal"),
    ("d128_chunk", "bf16", [700], [129], 16, 1, 128, "none"),
    ("f32_d64", "f32", [40, 150], [40, 100], 8, 2, 64, "normal"),
]


# bf16 windowed prefill at d 64 with a group size divisible by 4 runs on the
# causal kernel's pipeline; a debug setting sends it to the kernel whose
# waves stream their own blocks, which every other shape takes.
WINDOW_ROUTES = {
    "pipelined": {},
    "streamed": {ga.ATTN_DEBUG_PREFILL_WINDOW_STREAMED: 1},
}


def _with_settings(settings, fn):
    prev = {k: ga.attn_sinks_set_debug(k, v) for k, v in settings.items()}
    try:
        return fn()
    finally:
        for k, v in prev.items():
            ga.attn_sinks_set_debug(k, v)


@pytest.fixture(params=list(WINDOW_ROUTES))
def window_route(request):
    settings = WINDOW_ROUTES[request.param]
    prev = {k: ga.attn_sinks_set_debug(k, v) for k, v in settings.items()}
    yield request.param
    for k, v in prev.items():
        ga.attn_sinks_set_debug(k, v)


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_window(case, window_route):
    name, dt, L, Lq, Hq, Hkv, d, sm = case
    b = wl.small_batch(zlib.crc32(name.encode()) % 1000 + 11, dt, L, Lq, Hq, Hkv, d,
                       sink_mode=sm)
    for w in (1, 17, 32, 64, 128, 300):
        note(f"prefill window {w} {name} ({window_route}): L={L} Lq={Lq} Hq={Hq} "
             f"Hkv={Hkv} d={d} {dt}")
        compare(run_prefill(b, window=w), oracle_full(b, window=w), dt,
                f"prefill {name} window {w}")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_no_window_and_wide_window_are_the_plain_calls(dt):
    """window 0, and any window of at least max_seq_len, give the bits of the
    unwindowed entry points."""
    d = wl.small_batch(201, dt, [900, 33, 2049], [1, 1, 1], 16, 2, 64, sink_mode="normal")
    note(f"decode window 0 / wide vs plain {dt}")
    plain = run_decode(d)
    for w in (0, d.max_seq_len, d.max_seq_len + 5):
        assert torch.equal(_bits(run_decode(d, window=w)), _bits(plain)), f"decode window {w}"
    p = wl.small_batch(202, dt, [300, 500], [300, 200], 8, 2, 64, sink_mode="normal")
    note(f"prefill window 0 / wide vs plain {dt}")
    plain = run_prefill(p)
    for w in (0, p.max_seq_len, 10 ** 6):
        assert torch.equal(_bits(run_prefill(p, window=w)), _bits(plain)), f"prefill window {w}"


def test_window_runs_are_deterministic():
    d = wl.small_batch(203, "bf16", [3000, 129, 77], [1, 1, 1], 16, 2, 64, sink_mode="normal")
    p = wl.small_batch(204, "bf16", [700, 300], [700, 100], 16, 2, 64, sink_mode="normal")
    note("window determinism")
    assert torch.equal(_bits(run_decode(d, window=128)), _bits(run_decode(d, window=128)))
    assert torch.equal(_bits(run_prefill(p, window=128)), _bits(run_prefill(p, window=128)))


@pytest.mark.parametrize("d,L,Lq", [(64, 700, 700), (128, 500, 300)])
def test_window_large_late_logits(d, L, Lq, window_route):
    """Keys from position 200 on get logits far above the earlier ones (std
    ~100 in natural units): rows whose window holds both kinds must raise
    their maximum well past the lazy slack and rescale.  Prefill at W = 128;
    decode at W = 600, whose window spans both kinds (the split passes)."""
    b = wl.small_batch(600 + d + L, "bf16", [L], [Lq], 8, 2, d)
    b = scale_keys(b, 200, 100.0)
    note(f"window prefill large late logits d={d} L={L} Lq={Lq}")
    compare(run_prefill(b, window=128), oracle_full(b, window=128), "bf16",
            f"window prefill large late logits d={d}")
    dec = replace(b, cu_seqlens_q=torch.tensor([0, 1], dtype=torch.int32),
                  q=b.q[-1:].contiguous())
    note(f"window decode large late logits d={d} L={L}")
    compare(run_decode(dec, window=600), oracle_full(dec, window=600), "bf16",
            f"window decode large late logits d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_window_prefill_logits_far_below_zero(d, window_route):
    """Every logit near -150 (natural units) and no sink: weights against a
    zero reference would underflow to 0; each row's maximum has to come from
    its own first visible block."""
    b = wl.small_batch(700 + d, "bf16", [600], [600], 8, 2, d, sink_mode="none")
    b = aligned_scores(b, 9 + d, 30.0, 150.0 / (30.0 * b.scale))
    note(f"window prefill logits near -150, no sink, d={d}")
    compare(run_prefill(b, window=128), oracle_full(b, window=128), "bf16",
            f"window prefill low logits d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_window_tail_on_partial_last_page(d, window_route):
    """Chunks of a few rows at the very end of their sequence, whose windows
    all start on the sequence's last, partly filled page: the pages below
    are read as rows of that page, and those rows have to stay inside the
    sequence (the rest of the page holds NaN).  Lengths put the oldest key
    in either half of its 32-token block and in either block of a 64-key
    tile; the windows are shorter than a page, one past a block's half,
    and longer."""
    L = [97, 100, 289, 310, 1000, 1007, 1010, 1025, 96, 1008]
    Lq = [1, 4, 1, 8, 1, 8, 3, 2, 1, 9]
    b = wl.small_batch(321 + d, "bf16", L, Lq, 16, 2, d, sink_mode="normal")
    for w in (1, 2, 8, 9, 17, 40):
        note(f"prefill window {w} tails on partial pages d={d} ({window_route}): "
             f"L={L} Lq={Lq}")
        compare(run_prefill(b, window=w), oracle_full(b, window=w), "bf16",
                f"prefill tails d={d} window {w}")


def test_prefill_window_block_edges_pipelined():
    """The pipelined windowed prefill skips, per row block, the 32-key blocks
    none of its rows sees (the block past row block 0's last row, the blocks
    below row block 1's window), and runs its middle steps without those
    tests.  Windows just below, at and above multiples of the block, and
    chunks whose first row sits at every offset class within a block (the
    prefix lengths 0, 5, 17, 31 and 870), put the first and last visible
    block of each row block at every step position."""
    L = [150, 205, 337, 351, 1000]
    Lq = [150, 200, 320, 320, 130]
    b = wl.small_batch(777, "bf16", L, Lq, 16, 2, 64, sink_mode="normal")
    for w in (31, 32, 33, 63, 64, 65, 95, 96, 97, 160):
        note(f"prefill window {w} block edges, pipelined: L={L} Lq={Lq}")
        compare(run_prefill(b, window=w), oracle_full(b, window=w), "bf16",
                f"prefill block edges window {w}")


PIPELINED_CASES = [
    # id, seq_lens, q_lens, Hq, Hkv, window, late-key scale: chunks over
    # prefixes; rows whose windows span small and much larger logits (their
    # rows take the exact recompute); few-row tails on partial last pages
    ("chunks", [500, 1000, 64, 2100], [100, 257, 1, 2100], 16, 2, 128, None),
    ("late_logits", [700, 900], [700, 600], 8, 2, 128, 100.0),
    ("tails", [97, 310, 1000, 1007, 1010], [1, 8, 1, 8, 3], 16, 2, 1, None),
]


@pytest.mark.parametrize("case", PIPELINED_CASES, ids=[c[0] for c in PIPELINED_CASES])
def test_prefill_window_pipelined_wait_all_bit_identical(case):
    """The pipelined windowed prefill with its hand-counted tile waits and
    with waits that take every load in flight: the same bits (a wait that
    missed a load would let a wave read a stage before it lands), and within
    the bar of the oracle."""
    name, L, Lq, Hq, Hkv, w, late = case
    b = wl.small_batch(zlib.crc32(name.encode()) % 1000 + 41, "bf16", L, Lq, Hq, Hkv, 64,
                       sink_mode="normal")
    if late is not None:
        b = scale_keys(b, 200, late)
    note(f"window {w} pipelined, counted and wait-all tile waits, {name}: L={L} Lq={Lq} "
         f"Hq={Hq} Hkv={Hkv}")
    outs = {}
    for route, settings in [("counted", {}), ("wait_all", {ga.ATTN_DEBUG_PREFILL_WAIT_ALL: 1})]:
        outs[route] = _with_settings(settings, lambda: run_prefill(b, window=w))
    assert torch.equal(outs["counted"].view(torch.int16), outs["wait_all"].view(torch.int16))
    compare(outs["counted"], oracle_full(b, window=w), "bf16", f"window {w} {name}")


def test_full_gptoss_decode_window128():
    b = wl.gptoss_decode(0)
    note("full gpt-oss decode, window 128 (every row)")
    compare(run_decode(b, window=128), oracle_full(b, window=128), "bf16",
            "gpt-oss decode window 128")


def test_full_gptoss_prefill_window128(window_route):
    b = wl.gptoss_prefill(0)
    note("full gpt-oss prefill, window 128 (sampled rows)")
    check_sampled(run_prefill(b, window=128), b, 3000, 5, "gpt-oss prefill window 128",
                  window=128)


def _redirect_below(b, first_page):
    """The batch with every table entry of sequence s below page first_page[s]
    pointing at a spare (NaN-filled, never referenced) page: a cache that
    has released the pages a window no longer reaches."""
    used = set(b.block_table[b.block_table >= 0].tolist())
    spare = next(p for p in range(b.k_cache.shape[0]) if p not in used)
    assert torch.isnan(b.k_cache[spare].float()).all(), "spare pages hold NaN"
    bt = b.block_table.clone()
    moved = 0
    for s, p in enumerate(first_page):
        if p > 0:
            bt[s, :p] = spare
            moved += p
    assert moved > 0
    return replace(b, block_table=bt)


WINDOW_PAGE_CASES = [
    # id, seq_lens, Hq, Hkv, d, window: the oldest visible key of some
    # sequence sits at offset >= 16 of its 32-token block, so that block
    # begins with a page wholly below the window
    ("d64_w80", [1000, 300, 2049, 97], 16, 2, 64, 80),
    ("d64_w590_split", [2049, 1300, 3000], 16, 2, 64, 590),
    ("d128_w100", [1000, 517, 2049], 32, 2, 128, 100),
]


@pytest.mark.parametrize("case", WINDOW_PAGE_CASES, ids=[c[0] for c in WINDOW_PAGE_CASES])
def test_decode_window_reads_no_page_below_it(case):
    name, L, Hq, Hkv, d, w = case
    b = wl.small_batch(zlib.crc32(name.encode()) % 1000 + 29, "bf16", L, [1] * len(L), Hq, Hkv,
                       d, sink_mode="normal")
    assert any((l - w) % 32 >= 16 for l in L if l > w)
    moved = _redirect_below(b, [max(l - w, 0) // 16 for l in L])
    note(f"decode window {w}, pages below the window redirected, {name}: L={L} d={d}")
    got = run_decode(moved, window=w)
    compare(got, oracle_full(b, window=w), "bf16", f"decode {name}, released pages")
    same = run_decode(b, window=w)
    assert torch.equal(got.view(torch.int16), same.view(torch.int16))


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_window_reads_no_page_below_it(d, window_route):
    L, Lq, w = [1400, 700, 3000], [300, 200, 1000], 100
    b = wl.small_batch(71 + d, "bf16", L, Lq, 16, 2, d, sink_mode="normal")
    first = [max(l - lq - w + 1, 0) // 16 for l, lq in zip(L, Lq)]
    moved = _redirect_below(b, first)
    note(f"prefill window {w}, pages below every row's window redirected: L={L} Lq={Lq} d={d}")
    got = run_prefill(moved, window=w)
    compare(got, oracle_full(b, window=w), "bf16", f"prefill d={d}, released pages")
    same = run_prefill(b, window=w)
    assert torch.equal(got.view(torch.int16), same.view(torch.int16))
