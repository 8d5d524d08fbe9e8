"""Each plausible mistake planted in a copy of oracle.c must fail some pin.

The copies are compiled to a temporary directory on the CPU; the oracle's own
source is never modified.  A mutant that no pin rejects means the pins are
too weak to vouch for the oracle.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "sink dropped from the denominator": ("den += exp(sink - m);", "den += 0.0;"),
    "sink sign flipped": ("den += exp(sink - m);", "den += exp(-sink - m);"),
    "sink scaled like a logit": ("den += exp(sink - m);", "den += exp(scale * sink - m);"),
    "scale dropped": ("scores[j] = scale * dot;", "scores[j] = dot;"),
    "GQA head mapping h % Hkv": ("const int g = h / group;", "const int g = h % num_kv_heads;"),
    "top-left causal alignment": ("const int pos = seq_lens[b] - q_len + i;", "const int pos = i;"),
    "last key excluded": ("const int n_vis = last + 1 < 0 ? 0 : last + 1;",
                          "const int n_vis = last < 0 ? 0 : last;"),
    "causal flag ignored": ("const int last = causal ? pos : seq_lens[b] - 1;",
                            "const int last = pos;"),
    "unmasked rows stop at the chunk start": ("const int last = causal ? pos : seq_lens[b] - 1;",
                                              "const int last = causal ? pos : seq_lens[b] - q_len;"),
    "page slot from the wrong index": ("* page_size + (j % page_size)) * head_dim;",
                                       "* page_size + (j / page_size) % page_size) * head_dim;"),
    "K and V swapped": ("dot += qrow[c] * widen(k_cache, row + c, dtype);",
                        "dot += qrow[c] * widen(v_cache, row + c, dtype);"),
    "bf16 widened from the wrong half": ("<< 16;", "<< 0;"),
    "exponent not shifted by the max": ("double e = exp(scores[j] - m);",
                                        "double e = exp(scores[j]);"),
    "query row of the wrong head": ("((size_t)t * num_q_heads + h) * head_dim + c",
                                    "((size_t)t * num_q_heads + h / group) * head_dim + c"),
    "window one key too wide": ("? n_vis - window : 0;", "? n_vis - window - 1 : 0;"),
    "window ignored": ("const int j0 = (window > 0 &&", "const int j0 = 0 * (window > 0 &&"),
    "window anchored at the chunk's first query": (
        "const int j0 = (window > 0 && n_vis - window > 0) ? n_vis - window : 0;",
        "const int j0 = (window > 0 && n_vis - i - window > 0) ? n_vis - i - window : 0;"),
}


def _build(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not unique: {old!r}"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", str(src), "-o", str(lib),
                    "-lm"], check=True)
    return oracle.load_library(str(lib))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build(tmp_path, name, old, new)

    def attn(batch, with_lse=False, window=0, causal=True):
        return oracle.attention(batch, threads=4, with_lse=with_lse, lib=lib, window=window,
                                causal=causal)

    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(attn)
        except (AssertionError, RuntimeError, ValueError):
            failures.append(pin.__name__)
    assert failures, f"no pin rejects the mutant '{name}'"


# Plausible mistakes in a KV append, each of which check_append must reject.
def _append_mutant(kind):
    def append(batch, k_new, v_new):
        k = batch.k_cache.clone()
        v = batch.v_cache.clone()
        cu = batch.cu_seqlens_q.tolist()
        P = batch.page_size
        for b in range(batch.num_seqs):
            L = int(batch.seq_lens[b])
            n = cu[b + 1] - cu[b]
            for i in range(n):
                p = L - n + i
                if kind == "off by one":
                    p = L - n + i - 1 if L - n + i > 0 else 0
                if kind == "anchored at 0":
                    p = i
                page = int(batch.block_table[b, p // P])
                slot = p % P if kind != "slot from page index" else (p // P) % P
                src = cu[b] + i if kind != "rows of the wrong order" else cu[b] + n - 1 - i
                k[page, :, slot, :] = k_new[src]
                v[page, :, slot, :] = (v_new if kind != "K written as V" else k_new)[src]
        return k, v
    return append


@pytest.mark.parametrize("kind", ["off by one", "anchored at 0", "slot from page index",
                                  "rows of the wrong order", "K written as V"])
def test_append_mutant_is_caught(kind):
    with pytest.raises(AssertionError):
        pins.check_append(_append_mutant(kind))
