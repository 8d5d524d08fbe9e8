"""The oracle against its pins (CPU only).  See oracle_pins.py for the facts."""
import numpy as np
import pytest

import oracle
from gqa_paged_attention_amd import workloads as wl
from tests import oracle_pins as pins


def _attn(batch, with_lse=False, window=0, causal=True):
    return oracle.attention(batch, threads=4, with_lse=with_lse, window=window, causal=causal)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_attn)


def test_rows_subset_matches_full():
    b = pins.medium_batch(91)
    full = _attn(b)
    tok = np.array([0, 5, 40, 50], dtype=np.int64)
    head = np.array([7, 0, 3, 5], dtype=np.int32)
    sub = oracle.attention_rows(b, tok, head, threads=2)
    assert np.array_equal(sub, full[tok, head])


def test_thread_count_does_not_change_bits():
    b = pins.medium_batch(92, dtype="bf16")
    assert np.array_equal(oracle.attention(b, threads=1), oracle.attention(b, threads=8))


def test_tiny_fp32_prefill_then_decode():
    pre, dec, (page, slot, nk, nv) = wl.tiny_fp32(0, keep_logical=True)
    assert pre.total_q == 256 and dec.total_q == 1 and int(dec.seq_lens[0]) == 257
    assert pre.num_pages == 17 and int(dec.block_table[0, 16]) == page
    out_pre = _attn(pre)
    assert np.all(np.isfinite(out_pre))
    # the decode pool holds the appended token; the prefill pool holds NaN there
    assert np.isnan(pre.k_cache[page, :, slot].numpy()).all()
    out_dec = _attn(dec)
    assert np.all(np.isfinite(out_dec))
