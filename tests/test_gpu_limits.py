"""GPU parity at the edges of the supported shapes: very long sequences,
many sequences, the largest group size, long prefill chunks over long
prefixes (sampled rows where the oracle would be slow)."""
import numpy as np
import pytest
import torch

from gqa_paged_attention_amd import workloads as wl
from tests.gpu_helpers import check_sampled, compare, note, oracle_full, run_decode, run_prefill

pytestmark = pytest.mark.gpu


def test_decode_very_long_sequence_g16_d128():
    # one 131072-token sequence, 16 query heads on one KV head
    b = wl.small_batch(601, "bf16", [131072, 5], [1, 1], 16, 1, 128, sink_mode="normal")
    note("decode L=131072, G=16, d=128")
    compare(run_decode(b), oracle_full(b), "bf16", "decode 128K tokens")


def test_decode_many_sequences():
    gen = torch.Generator().manual_seed(602)
    L = torch.randint(1, 300, (4096,), generator=gen, dtype=torch.int64).to(torch.int32)
    b = wl.build_batch(gen, "bf16", L, torch.ones(4096, dtype=torch.int32), 8, 1, 64,
                       sink_mode="normal")
    note("decode 4096 sequences")
    compare(run_decode(b), oracle_full(b), "bf16", "decode 4096 sequences")


def test_decode_g16_d64_and_length_bound_above_lengths():
    # the host length bound may exceed every actual length
    b = wl.small_batch(603, "bf16", [100, 2000, 33], [1, 1, 1], 32, 2, 64, sink_mode="normal")
    note("decode G=16 d=64 with max_seq_len above the lengths")
    got = run_decode(b, max_seq_len=b.max_pages_per_seq * 16)
    compare(got, oracle_full(b), "bf16", "decode G=16, loose length bound")


def test_prefill_long_chunk_over_long_prefix():
    # 16384 new rows over a 16384-token prefix, sampled rows
    b = wl.small_batch(604, "bf16", [32768], [16384], 16, 2, 64, sink_mode="normal")
    note("prefill 16384 rows over a 16384-token prefix (sampled)")
    check_sampled(run_prefill(b), b, 1500, 7, "long prefill chunk")


def test_prefill_d128_g16_long():
    b = wl.small_batch(605, "bf16", [9000], [9000], 16, 1, 128, sink_mode="normal")
    note("prefill d=128 G=16 9000 tokens (sampled)")
    check_sampled(run_prefill(b), b, 1500, 8, "prefill d128 G16")
