"""Pure-Python brute force of sink attention, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

This follows the "virtual token" description of the sink in the "GPT OSS"
model notes (TensorSharp docs, sections 1 and 4.1): for each query row the
visible keys are gathered one by one from the HND page pool, their logits are
listed, and one more entry is appended whose logit is the head's sink and
whose value vector is all zeros.  A textbook max-subtracted softmax over that
list (math.fsum for every sum) then weights the values.  It shares no code
with oracle.c and uses no numpy or torch arithmetic.
"""
from __future__ import annotations

import math


def _tolist(t):
    return t.tolist() if hasattr(t, "tolist") else list(t)


def brute_force(batch, window: int = 0, causal: bool = True):
    """Return nested lists out[total_q][Hq][d] for a small CPU PagedBatch.

    With window > 0 the query at position p lists only the keys at positions
    p - window + 1 .. p (the sliding window of the model notes, section 4.1);
    with causal=False every row lists all keys of its sequence."""
    q = _tolist(batch.q.double())
    k_pool = _tolist(batch.k_cache.double())
    v_pool = _tolist(batch.v_cache.double())
    table = _tolist(batch.block_table)
    seq_lens = _tolist(batch.seq_lens)
    cu = _tolist(batch.cu_seqlens_q)
    sinks = None if batch.sinks is None else _tolist(batch.sinks.double())
    Hq, Hkv, d, P = batch.num_q_heads, batch.num_kv_heads, batch.head_dim, batch.page_size
    per_kv = Hq // Hkv
    scale = float(batch.scale)

    out = [None] * len(q)
    for b in range(len(seq_lens)):
        n_q = cu[b + 1] - cu[b]
        for i in range(n_q):
            t = cu[b] + i
            # the row's last visible key: its own position, or the last key
            newest = seq_lens[b] - n_q + i if causal else seq_lens[b] - 1
            rows = []
            for h in range(Hq):
                kv_head = h // per_kv
                keys, values = [], []
                oldest = max(0, newest + 1 - window) if window > 0 else 0
                for j in range(oldest, newest + 1):
                    page = table[b][j // P]
                    keys.append(k_pool[page][kv_head][j % P])
                    values.append(v_pool[page][kv_head][j % P])
                logits = [scale * math.fsum(a * c for a, c in zip(q[t][h], key)) for key in keys]
                # the virtual sink token: its logit is the sink, its value is zero
                logits.append(sinks[h] if sinks is not None else -math.inf)
                values.append([0.0] * d)
                top = max(logits)
                if top == -math.inf:
                    rows.append([0.0] * d)
                    continue
                weights = [math.exp(x - top) for x in logits]
                total = math.fsum(weights)
                rows.append([math.fsum(w * val[c] for w, val in zip(weights, values)) / total
                             for c in range(d)])
            out[t] = rows
    return out
