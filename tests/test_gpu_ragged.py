"""GPU parity of the ragged, cache-free attention (contiguous K/V per
sequence, "Fast embeddings on GPUs": ragged inputs and no KV cache) with
and without the causal mask, and of the row LSE it reports, against the
oracle (which reads the same values laid out in pages)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import gqa_paged_attention_amd as ga
import oracle
from gqa_paged_attention_amd import workloads as wl
from tests.gpu_helpers import ORACLE_THREADS, compare, note, require_gpu, scale_keys

pytestmark = pytest.mark.gpu

LSE_TOL = (5e-3, 1e-3)  # abs, rel: weights enter the row sum as bf16


def run_ragged(r, causal, with_lse=True):
    require_gpu()
    g = r.to("cuda")
    out = torch.empty_like(g.q)
    lse = torch.empty(g.q.shape[0], g.q.shape[1], dtype=torch.float32, device="cuda") \
        if with_lse else None
    ga.attn_sinks_ragged(g.q, g.k, g.v, g.cu_seqlens_q, g.cu_seqlens_kv, g.sinks, g.scale,
                         causal, out, lse, r.max_q_len, r.max_kv_len)
    torch.cuda.synchronize()
    return out.cpu(), None if lse is None else lse.cpu()


def check_lse(got, ref, what):
    g, r = got.double().numpy(), np.asarray(ref)
    fin = np.isfinite(r)
    assert np.array_equal(np.isfinite(g), fin), f"{what}: finiteness differs"
    err = np.abs(g[fin] - r[fin])
    note(f"  {what}: lse max abs err {err.max() if err.size else 0:.3e}")
    assert np.all(err <= LSE_TOL[0] + LSE_TOL[1] * np.abs(r[fin])), f"{what}: LSE off"


CASES = [
    # id, kv_lens, q_lens, Hq, Hkv, d, sink_mode
    ("d64_g8_ragged", [1, 17, 130, 300, 600], [1, 17, 130, 300, 600], 16, 2, 64, "normal"),
    ("d64_chunks", [500, 1000, 64], [100, 257, 1], 16, 2, 64, "normal"),
    ("d128_g4", [200, 333], [200, 333], 8, 2, 128, "normal"),
    ("d64_g1_nosink", [255, 256, 257], [255, 256, 257], 4, 4, 64, "none"),
    ("d128_neginf", [700], [129], 16, 1, 128, "neginf"),
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "unmasked"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ragged(case, causal):
    name, L, Lq, Hq, Hkv, d, sm = case
    r = wl.ragged_batch(len(name) * 17 + int(causal), "bf16", L, Lq, Hq, Hkv, d, sink_mode=sm)
    note(f"ragged {name} causal={causal}: L={L} Lq={Lq} Hq={Hq} Hkv={Hkv} d={d}")
    out, lse = run_ragged(r, causal)
    ref, ref_lse = oracle.attention(r.paged, threads=ORACLE_THREADS, with_lse=True,
                                    causal=causal)
    compare(out, ref, "bf16", f"ragged {name} causal={causal}")
    check_lse(lse, ref_lse, f"ragged {name} causal={causal}")


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "unmasked"])
def test_ragged_large_late_logits(causal):
    """Keys from position 64 on get logits far above the earlier ones (std ~100
    in natural units): weights against the reference taken from the first
    keys cannot hold them, so the exact recompute runs; its outputs and LSE
    meet the bar.  The contiguous K rows and the oracle's paged copy are
    scaled alike."""
    r = wl.ragged_batch(503 + int(causal), "bf16", [300, 700], [300, 190], 8, 2, 64,
                        sink_mode="normal")
    k = r.k.clone()
    cu = r.cu_seqlens_kv
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]) + 64, int(cu[s + 1])
        k[lo:hi] = (k[lo:hi].float() * 100.0).to(k.dtype)
    r = replace(r, k=k, paged=scale_keys(r.paged, 64, 100.0))
    note(f"ragged large late logits causal={causal}")
    out, lse = run_ragged(r, causal)
    ref, ref_lse = oracle.attention(r.paged, threads=ORACLE_THREADS, with_lse=True,
                                    causal=causal)
    compare(out, ref, "bf16", f"ragged large late logits causal={causal}")
    check_lse(lse, ref_lse, f"ragged large late logits causal={causal}")


def test_ragged_unmasked_more_rows_than_keys_and_empty_sequences():
    r = wl.ragged_batch(501, "bf16", [0, 40, 3], [5, 70, 9], 8, 2, 64, sink_mode="normal")
    note("ragged unmasked, Lq > L and an empty key set")
    out, lse = run_ragged(r, False)
    ref, ref_lse = oracle.attention(r.paged, threads=ORACLE_THREADS, with_lse=True,
                                    causal=False)
    compare(out, ref, "bf16", "ragged unmasked Lq > L")
    check_lse(lse, ref_lse, "ragged unmasked Lq > L")


def test_ragged_causal_equals_paged_prefill():
    """The ragged causal call and the paged prefill of the same values agree
    (both within tolerance of the oracle; here to each other, closely)."""
    r = wl.ragged_batch(502, "bf16", [300, 77], [300, 40], 16, 2, 64, sink_mode="normal")
    out, _ = run_ragged(r, True, with_lse=False)
    g = r.paged.to("cuda")
    o2 = torch.empty_like(g.q)
    ga.attn_sinks_prefill(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.cu_seqlens_q,
                          g.sinks, g.scale, o2, r.paged.max_q_len, r.paged.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o2.cpu().view(torch.int16))


def test_full_gptoss_prefill_shape_ragged():
    """The gpt-oss prefill shape (8 x 4096, 64/8, d 64) as ragged causal
    attention; sampled rows and their LSE against the oracle."""
    r = wl.ragged_batch(0, "bf16", [4096] * 8, [4096] * 8, 64, 8, 64, sink_mode="normal")
    note("full gpt-oss prefill shape, ragged causal")
    out, lse = run_ragged(r, True)
    rng = np.random.default_rng(3)
    tok = rng.integers(0, r.q.shape[0], size=2000)
    head = rng.integers(0, 64, size=2000).astype(np.int32)
    ref, ref_lse = oracle.attention_rows(r.paged, tok, head, threads=ORACLE_THREADS,
                                         with_lse=True)
    compare(out[torch.as_tensor(tok), torch.as_tensor(head.astype(np.int64))], ref, "bf16",
            "gpt-oss ragged causal (sampled)")
    check_lse(lse[torch.as_tensor(tok), torch.as_tensor(head.astype(np.int64))], ref_lse,
              "gpt-oss ragged causal (sampled)")
