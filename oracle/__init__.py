"""fp64 CPU oracle for paged grouped-query attention with per-head sinks.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its binding) never imports, links or calls it, and it never touches the
GPU or the HIP library.

Two independent implementations of one definition live here (plus the KV
append of ``append_kv``, which the attention step follows):

* ``attention_rows`` / ``attention`` -- ctypes binding of ``oracle.c``: fp64,
  OpenMP over (query token, head) rows, two passes over the keys in logical
  order (max with the sink, then exponentials, denominator and values).
* ``brute.brute_force`` -- pure Python on nested lists: per row it lists the
  visible logits, appends the sink as a virtual token whose value vector is
  zero ("GPT OSS" model notes, sections 1 and 4.1), and applies a textbook
  softmax with math.fsum.  For tiny inputs only.

The definition both follow is written out in the header of oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "oracle.c")
_LIB_PATH = os.path.join(_DIR, "liboracle.so")
_lib = None

DTYPE_CODE = {"f32": 0, "bf16": 1}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """ctypes handle of a compiled oracle with its signature declared."""
    lib = ctypes.CDLL(path)
    f = lib.oracle_attention_rows
    P = ctypes.c_void_p
    f.argtypes = [ctypes.c_int] * 7 + [P] * 6 + [P, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int64, P, P, P, P, ctypes.c_int]
    f.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = load_library(_LIB_PATH)
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def attention_rows(batch, row_token: Sequence[int], row_head: Sequence[int],
                   threads: Optional[int] = None, with_lse: bool = False, lib=None,
                   window: int = 0, causal: bool = True):
    """fp64 outputs for the listed (query token, query head) pairs.

    `batch` is a workloads.PagedBatch on the CPU.  Returns an array
    [n_rows][head_dim] (and the natural-log LSE per row when asked).
    `window` > 0 limits each query at position p to keys p - window + 1 .. p;
    causal=False lets every row see all keys of its sequence.  The LSE is
    the natural log of the row's softmax denominator, sink included.
    `lib` selects another compiled copy of oracle.c (used by the tests that
    check the pins catch planted mistakes).
    """
    lib = lib or _load()
    dev = batch.q.device
    if dev.type != "cpu":
        raise ValueError("the oracle reads CPU tensors only")
    rt = torch.as_tensor(np.asarray(row_token, dtype=np.int64)).contiguous()
    rh = torch.as_tensor(np.asarray(row_head, dtype=np.int32)).contiguous()
    n = int(rt.numel())
    if rh.numel() != n:
        raise ValueError("row_token and row_head differ in length")
    out = torch.empty(n, batch.head_dim, dtype=torch.float64)
    lse = torch.empty(n, dtype=torch.float64) if with_lse else None
    q = batch.q.contiguous()
    kc = batch.k_cache.contiguous()
    vc = batch.v_cache.contiguous()
    bt = batch.block_table.to(torch.int32).contiguous()
    sl = batch.seq_lens.to(torch.int32).contiguous()
    cu = batch.cu_seqlens_q.to(torch.int32).contiguous()
    sinks = None if batch.sinks is None else batch.sinks.to(torch.float32).contiguous()
    rc = lib.oracle_attention_rows(
        DTYPE_CODE[batch.dtype], batch.num_seqs, batch.num_q_heads, batch.num_kv_heads,
        batch.head_dim, batch.page_size, batch.max_pages_per_seq,
        _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(sl), _ptr(cu), _ptr(sinks),
        ctypes.c_double(batch.scale), int(window), int(bool(causal)), ctypes.c_int64(n),
        _ptr(rt), _ptr(rh),
        _ptr(out), _ptr(lse), int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_rows failed with code {rc}")
    return (out.numpy(), lse.numpy()) if with_lse else out.numpy()


def attention(batch, threads: Optional[int] = None, with_lse: bool = False, lib=None,
              window: int = 0, causal: bool = True):
    """fp64 output for every query row: array [total_q][Hq][head_dim]."""
    T, H = batch.total_q, batch.num_q_heads
    tok = np.repeat(np.arange(T, dtype=np.int64), H)
    head = np.tile(np.arange(H, dtype=np.int32), T)
    res = attention_rows(batch, tok, head, threads=threads, with_lse=with_lse, lib=lib,
                         window=window, causal=causal)
    if with_lse:
        out, lse = res
        return out.reshape(T, H, batch.head_dim), lse.reshape(T, H)
    return res.reshape(T, H, batch.head_dim)


def append_kv(batch, k_new: torch.Tensor, v_new: torch.Tensor):
    """The cache after appending the newest tokens ("GPT OSS" model notes,
    section 3: the layer's (K, V) are appended to the KV cache before the
    attention step; section 11: paged K/V per layer).

    Token i of the n_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] new tokens of
    sequence b sits at position p = L_b - n_b + i (seq_lens already count
    them); its rows go to page block_table[b][p // page_size], slot
    p % page_size, of every KV head.  k_new / v_new are [total_q][Hkv][d] in
    query order.  Returns new (k_cache, v_cache) CPU tensors; nothing else
    changes.  Plain Python loop over the tokens.
    """
    k = batch.k_cache.clone()
    v = batch.v_cache.clone()
    cu = batch.cu_seqlens_q.tolist()
    table = batch.block_table.tolist()
    P = batch.page_size
    for b in range(batch.num_seqs):
        L = int(batch.seq_lens[b])
        n = cu[b + 1] - cu[b]
        for i in range(n):
            p = L - n + i
            page = table[b][p // P]
            k[page, :, p % P, :] = k_new[cu[b] + i]
            v[page, :, p % P, :] = v_new[cu[b] + i]
    return k, v
