"""Seeded synthetic inputs for paged grouped-query attention with sinks.

This module draws random tensors and lays them out; it does no attention
arithmetic.  Both the HIP path and the fp64 oracle consume what it builds.

Layout produced (the HND page layout of "Hosting Qwen on Blackwell": heads
major, the tokens of one head contiguous inside a page):

    k_cache, v_cache   [num_pages][num_kv_heads][page_size][head_dim]
    block_table        [num_seqs][max_pages_per_seq] int32, -1 past the end
    seq_lens           [num_seqs] int32   visible KV tokens, new tokens included
    cu_seqlens_q       [num_seqs + 1] int32   ragged query offsets
    q                  [total_q][num_q_heads][head_dim]
    sinks              [num_q_heads] float32, or None (every sink is -inf)

Recipe (fixed draw order from one CPU generator seeded per workload):
  1. sequence lengths (integers, uniform, inclusive bounds), when drawn;
  2. a random permutation of all pool pages (used pages + ~1 % spare);
  3. q, then K, then V as float32 N(0, 1) in logical [token][head][dim]
     order, then rounded to the storage dtype (round-to-nearest-even);
  4. sinks as float32 N(0, 1) * sink_std (never rounded to bf16).
K/V rows are then scattered into the permuted pool, so which physical page
holds a token never changes the values.  Unused slots of each sequence's last
page and every spare page hold NaN, so a kernel that reads past a sequence's
end poisons its output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

PAGE_SIZE = 16

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class PagedBatch:
    """One call's worth of inputs, all CPU tensors unless moved by the caller."""

    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    seq_lens: torch.Tensor
    cu_seqlens_q: torch.Tensor
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    sinks: Optional[torch.Tensor]
    scale: float
    # Logical K/V rows ([sum L_b][Hkv][d]) and their per-sequence offsets, kept
    # only when asked for; tests use them to build library-routine references.
    k_logical: Optional[torch.Tensor] = None
    v_logical: Optional[torch.Tensor] = None
    kv_offsets: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.numel())

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def q_lens(self) -> torch.Tensor:
        return (self.cu_seqlens_q[1:] - self.cu_seqlens_q[:-1]).to(torch.int32)

    @property
    def max_q_len(self) -> int:
        if "max_q_len" in self.meta:
            return self.meta["max_q_len"]
        return int(self.q_lens.max().item()) if self.num_seqs else 0

    @property
    def max_seq_len(self) -> int:
        if "max_seq_len" in self.meta:
            return self.meta["max_seq_len"]
        return int(self.seq_lens.max().item()) if self.num_seqs else 0

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def is_decode(self) -> bool:
        return bool(torch.all(self.q_lens == 1).item())

    def to(self, device) -> "PagedBatch":
        """Copy every tensor to `device` (the logical K/V stay on the CPU).

        The host-side maxima are computed first and kept, so a GPU batch never
        needs a device-to-host read to size a call."""
        mv = lambda t: None if t is None else t.to(device)
        meta = dict(self.meta)
        meta["max_q_len"] = self.max_q_len
        meta["max_seq_len"] = self.max_seq_len
        return replace(
            self,
            meta=meta,
            seq_lens=mv(self.seq_lens),
            cu_seqlens_q=mv(self.cu_seqlens_q),
            q=mv(self.q),
            k_cache=mv(self.k_cache),
            v_cache=mv(self.v_cache),
            block_table=mv(self.block_table),
            sinks=mv(self.sinks),
        )

    def rows(self, start: int, stop: int) -> "PagedBatch":
        """Sequences [start, stop) as a batch that shares the same page pool."""
        cu = self.cu_seqlens_q
        q0, q1 = int(cu[start]), int(cu[stop])
        meta = {k: v for k, v in self.meta.items() if k not in ("max_q_len", "max_seq_len")}
        return replace(
            self,
            meta=meta,
            seq_lens=self.seq_lens[start:stop].contiguous(),
            cu_seqlens_q=(cu[start:stop + 1] - q0).to(torch.int32).contiguous(),
            q=self.q[q0:q1].contiguous(),
            block_table=self.block_table[start:stop].contiguous(),
            k_logical=None,
            v_logical=None,
            kv_offsets=None,
        )

    def algorithmic_kv_bytes(self) -> int:
        """K + V bytes of the visible tokens (what a decode pass must read)."""
        elem = 4 if self.dtype == "f32" else 2
        return int(self.seq_lens.to(torch.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * elem


def _draw_lengths(gen: torch.Generator, n: int, lo: int, hi: int) -> torch.Tensor:
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int64).to(torch.int32)


def build_batch(
    gen: torch.Generator,
    dtype: str,
    seq_lens,
    q_lens,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    sink_mode: str = "normal",
    sink_std: float = 1.0,
    scale: Optional[float] = None,
    spare_frac: float = 0.01,
    page_size: int = PAGE_SIZE,
    keep_logical: bool = False,
    poison: bool = True,
    causal_rows: bool = True,
) -> PagedBatch:
    """Draw q/K/V/sinks (steps 2-4 of the recipe) and lay them out in pages.

    sink_mode: "normal" (N(0,1) * sink_std), "neginf" (an explicit -inf array)
    or "none" (sinks=None, which the kernels read as every sink = -inf).
    """
    if dtype not in _TORCH_DTYPE:
        raise ValueError(f"dtype must be one of {sorted(_TORCH_DTYPE)}")
    tdt = _TORCH_DTYPE[dtype]
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32).flatten()
    q_lens = torch.as_tensor(q_lens, dtype=torch.int32).flatten()
    if seq_lens.numel() != q_lens.numel():
        raise ValueError("seq_lens and q_lens differ in length")
    if causal_rows and torch.any(q_lens > seq_lens):
        # (rows without the causal mask may outnumber the keys)
        raise ValueError("a sequence has more query tokens than visible keys")
    B = seq_lens.numel()
    pages_per_seq = [(int(L) + page_size - 1) // page_size for L in seq_lens]
    used = sum(pages_per_seq)
    spare = int(math.ceil(used * spare_frac)) if spare_frac > 0 else 0
    num_pages = max(used + spare, 1)
    max_pages = max(max(pages_per_seq, default=0), 1)

    # 2. pool permutation
    perm = torch.randperm(num_pages, generator=gen).to(torch.int32)

    total_q = int(q_lens.sum())
    total_kv = int(seq_lens.to(torch.int64).sum())
    # 3. q, K, V in logical order, drawn in fp32 then rounded to the dtype
    q = torch.randn(total_q, num_q_heads, head_dim, generator=gen).to(tdt)
    k = torch.randn(total_kv, num_kv_heads, head_dim, generator=gen).to(tdt)
    v = torch.randn(total_kv, num_kv_heads, head_dim, generator=gen).to(tdt)
    # 4. sinks
    if sink_mode == "normal":
        sinks = torch.randn(num_q_heads, generator=gen) * float(sink_std)
    elif sink_mode == "neginf":
        sinks = torch.full((num_q_heads,), float("-inf"))
    elif sink_mode == "none":
        sinks = None
    else:
        raise ValueError(f"unknown sink_mode {sink_mode!r}")

    return _lay_out(dtype, seq_lens, q_lens, perm, pages_per_seq, max_pages, q, k, v,
                    None if sinks is None else sinks.to(torch.float32),
                    float(scale) if scale is not None else 1.0 / math.sqrt(head_dim),
                    page_size, keep_logical, poison)


def _lay_out(dtype, seq_lens, q_lens, perm, pages_per_seq, max_pages, q, k, v, sinks, scale,
             page_size, keep_logical, poison) -> PagedBatch:
    """Scatter logical K/V rows into the permuted HND pool and build the table."""
    tdt = _TORCH_DTYPE[dtype]
    B = seq_lens.numel()
    num_pages = perm.numel()
    num_kv_heads, head_dim = k.shape[1], k.shape[2]
    block_table = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(pages_per_seq):
        block_table[b, :n] = perm[off:off + n]
        off += n
    fill = float("nan") if poison else 0.0
    k_cache = torch.full((num_pages, num_kv_heads, page_size, head_dim), fill, dtype=tdt)
    v_cache = torch.full_like(k_cache, fill)
    kv_offsets = torch.zeros(B + 1, dtype=torch.int64)
    kv_offsets[1:] = torch.cumsum(seq_lens.to(torch.int64), 0)
    # sequence by sequence: logical rows -> [pages][16][Hkv][d] -> HND pages
    for b in range(B):
        L, n = int(seq_lens[b]), pages_per_seq[b]
        if L == 0:
            continue
        o = int(kv_offsets[b])
        ids = block_table[b, :n].to(torch.int64)
        for src, dst in ((k, k_cache), (v, v_cache)):
            blk = torch.full((n * page_size, num_kv_heads, head_dim), fill, dtype=tdt)
            blk[:L] = src[o:o + L]
            dst[ids] = blk.view(n, page_size, num_kv_heads, head_dim).transpose(1, 2)

    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(q_lens, 0).to(torch.int32)
    return PagedBatch(
        dtype=dtype,
        num_q_heads=int(q.shape[1]),
        num_kv_heads=int(num_kv_heads),
        head_dim=int(head_dim),
        page_size=page_size,
        seq_lens=seq_lens.contiguous(),
        cu_seqlens_q=cu,
        q=q.contiguous(),
        k_cache=k_cache,
        v_cache=v_cache,
        block_table=block_table,
        sinks=None if sinks is None else sinks.contiguous(),
        scale=float(scale),
        k_logical=k if keep_logical else None,
        v_logical=v if keep_logical else None,
        kv_offsets=kv_offsets if keep_logical else None,
    )


def from_logical(dtype: str, q, k, v, seq_lens, q_lens, sinks, scale: float,
                 perm_seed: int = 0, spare_pages: int = 0, page_size: int = PAGE_SIZE,
                 poison: bool = True) -> PagedBatch:
    """Lay out given logical rows (q [total_q][Hq][d], k/v [sum L][Hkv][d])
    into a randomly permuted page pool; used for hand-worked cases."""
    tdt = _TORCH_DTYPE[dtype]
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32).flatten()
    q_lens = torch.as_tensor(q_lens, dtype=torch.int32).flatten()
    pages_per_seq = [(int(L) + page_size - 1) // page_size for L in seq_lens]
    num_pages = max(sum(pages_per_seq) + spare_pages, 1)
    gen = torch.Generator().manual_seed(perm_seed)
    perm = torch.randperm(num_pages, generator=gen).to(torch.int32)
    max_pages = max(max(pages_per_seq, default=0), 1)
    return _lay_out(dtype, seq_lens, q_lens, perm, pages_per_seq, max_pages,
                    torch.as_tensor(q).to(tdt), torch.as_tensor(k).to(tdt),
                    torch.as_tensor(v).to(tdt),
                    None if sinks is None else torch.as_tensor(sinks, dtype=torch.float32),
                    scale, page_size, True, poison)


def split_new_tokens(batch: PagedBatch):
    """For a batch whose query rows are the newest tokens of each sequence
    (the last Lq_b of its L_b keys), return (pool_before, k_new, v_new):
    the same batch with those tokens' K/V slots overwritten with NaN (the pool
    as it stands before the append), and the tokens' K/V rows
    [total_q][Hkv][d] in query order.  Pure data movement, for the append
    tests; it needs nothing but the table and the pool."""
    cu = batch.cu_seqlens_q.tolist()
    P = batch.page_size
    k_old = batch.k_cache.clone()
    v_old = batch.v_cache.clone()
    k_new = torch.empty(batch.total_q, batch.num_kv_heads, batch.head_dim, dtype=k_old.dtype)
    v_new = torch.empty_like(k_new)
    for b in range(batch.num_seqs):
        L = int(batch.seq_lens[b])
        n = cu[b + 1] - cu[b]
        for i in range(n):
            pos = L - n + i
            page, slot = int(batch.block_table[b, pos // P]), pos % P
            k_new[cu[b] + i] = batch.k_cache[page, :, slot]
            v_new[cu[b] + i] = batch.v_cache[page, :, slot]
            k_old[page, :, slot] = float("nan")
            v_old[page, :, slot] = float("nan")
    return replace(batch, k_cache=k_old, v_cache=v_old), k_new, v_new


@dataclass
class RaggedBatch:
    """Ragged inputs without a KV cache: q [total_q][Hq][d], k/v
    [total_kv][Hkv][d] contiguous per sequence, offsets cu_seqlens_q /
    cu_seqlens_kv.  `paged` holds the same values laid out in a paged pool
    (for the oracle, which reads pages)."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens_q: torch.Tensor
    cu_seqlens_kv: torch.Tensor
    sinks: Optional[torch.Tensor]
    scale: float
    paged: PagedBatch

    @property
    def max_q_len(self) -> int:
        return int((self.cu_seqlens_q[1:] - self.cu_seqlens_q[:-1]).max().item())

    @property
    def max_kv_len(self) -> int:
        return int((self.cu_seqlens_kv[1:] - self.cu_seqlens_kv[:-1]).max().item())

    def to(self, device) -> "RaggedBatch":
        mv = lambda t: None if t is None else t.to(device)
        return replace(self, q=mv(self.q), k=mv(self.k), v=mv(self.v),
                       cu_seqlens_q=mv(self.cu_seqlens_q), cu_seqlens_kv=mv(self.cu_seqlens_kv),
                       sinks=mv(self.sinks))


def ragged_batch(seed: int, dtype: str, kv_lens, q_lens, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, sink_mode: str = "normal", sink_std: float = 1.0) -> RaggedBatch:
    """Same recipe as build_batch (lengths given; q, K, V, sinks drawn in that
    order), K/V kept contiguous per sequence."""
    gen = torch.Generator().manual_seed(seed)
    b = build_batch(gen, dtype, kv_lens, q_lens, num_q_heads, num_kv_heads, head_dim,
                    sink_mode=sink_mode, sink_std=sink_std, keep_logical=True,
                    causal_rows=False)
    cu_kv = b.kv_offsets.to(torch.int32)
    return RaggedBatch(q=b.q, k=b.k_logical.contiguous(), v=b.v_logical.contiguous(),
                       cu_seqlens_q=b.cu_seqlens_q, cu_seqlens_kv=cu_kv, sinks=b.sinks,
                       scale=b.scale, paged=b)


# --------------------------------------------------------------------------
# The five named workloads.  Shapes follow the attention of gpt-oss-20b
# (64 q heads, 8 KV heads, head_dim 64) and Qwen3-235B (64 q heads, 4 KV
# heads, head_dim 128); weights are never involved.
# --------------------------------------------------------------------------


def tiny_fp32(seed: int = 0, keep_logical: bool = False):
    """fp32, 1 seq, 4/1 heads, d=64, scale 1/8: a 256-token causal prefill,
    then one decode step at 257 tokens, in a shuffled 17-page pool.

    Returns (prefill_batch, decode_batch, new_token) where the prefill pool
    holds NaN in the slot of token 256 and `new_token` = (page, slot, k, v)
    is what an append writes there before the decode step.
    """
    gen = torch.Generator().manual_seed(seed)
    full = build_batch(gen, "f32", [257], [257], 4, 1, 64, sink_mode="normal",
                       scale=0.125, spare_frac=0.0, keep_logical=True)
    # decode query drawn after everything else
    q_dec = torch.randn(1, 4, 64, generator=gen).to(torch.float32)
    page = int(full.block_table[0, 256 // PAGE_SIZE])
    slot = 256 % PAGE_SIZE
    new_k = full.k_cache[page, :, slot, :].clone()
    new_v = full.v_cache[page, :, slot, :].clone()
    pre_k = full.k_cache.clone()
    pre_v = full.v_cache.clone()
    pre_k[page, :, slot, :] = float("nan")
    pre_v[page, :, slot, :] = float("nan")
    prefill = replace(full, seq_lens=torch.tensor([256], dtype=torch.int32),
                      cu_seqlens_q=torch.tensor([0, 256], dtype=torch.int32),
                      q=full.q[:256].contiguous(), k_cache=pre_k, v_cache=pre_v,
                      meta={"name": "tiny_fp32_prefill"})
    decode = replace(full, cu_seqlens_q=torch.tensor([0, 1], dtype=torch.int32), q=q_dec,
                     meta={"name": "tiny_fp32_decode"})
    if not keep_logical:
        prefill = replace(prefill, k_logical=None, v_logical=None, kv_offsets=None)
        decode = replace(decode, k_logical=None, v_logical=None, kv_offsets=None)
    else:
        prefill = replace(prefill, k_logical=full.k_logical[:256],
                          v_logical=full.v_logical[:256],
                          kv_offsets=torch.tensor([0, 256], dtype=torch.int64))
    return prefill, decode, (page, slot, new_k, new_v)


def gptoss_decode(seed: int = 0, keep_logical: bool = False) -> PagedBatch:
    """bf16 decode: 64 seqs x 1 token, 64/8 heads, d=64, L ~ U[1024, 8192]."""
    gen = torch.Generator().manual_seed(seed)
    L = _draw_lengths(gen, 64, 1024, 8192)
    b = build_batch(gen, "bf16", L, torch.ones(64, dtype=torch.int32), 64, 8, 64,
                    sink_mode="normal", keep_logical=keep_logical)
    b.meta["name"] = "gptoss_decode"
    return b


def gptoss_prefill(seed: int = 0, keep_logical: bool = False) -> PagedBatch:
    """bf16 causal prefill: 8 seqs x 4096 tokens (varlen offsets), 64/8, d=64."""
    gen = torch.Generator().manual_seed(seed)
    L = torch.full((8,), 4096, dtype=torch.int32)
    b = build_batch(gen, "bf16", L, L, 64, 8, 64, sink_mode="normal",
                    keep_logical=keep_logical)
    b.meta["name"] = "gptoss_prefill"
    return b


def qwen_decode(seed: int = 0, keep_logical: bool = False, sink_mode: str = "neginf") -> PagedBatch:
    """bf16 decode: 128 seqs x 1 token, 64/4 heads, d=128, L ~ U[4096, 32768],
    sinks = -inf (sink_mode "none" passes sinks=None instead)."""
    gen = torch.Generator().manual_seed(seed)
    L = _draw_lengths(gen, 128, 4096, 32768)
    b = build_batch(gen, "bf16", L, torch.ones(128, dtype=torch.int32), 64, 4, 128,
                    sink_mode=sink_mode, keep_logical=keep_logical)
    b.meta["name"] = "qwen_decode"
    return b


def qwen_prefill(seed: int = 0, keep_logical: bool = False) -> PagedBatch:
    """bf16 causal prefill in the Qwen decode's head shape: 4 seqs x 4096
    tokens, 64/4 heads, d=128, sinks = -inf."""
    gen = torch.Generator().manual_seed(seed)
    L = torch.full((4,), 4096, dtype=torch.int32)
    b = build_batch(gen, "bf16", L, L, 64, 4, 128, sink_mode="neginf",
                    keep_logical=keep_logical)
    b.meta["name"] = "qwen_prefill"
    return b


def mixed(seed: int = 0, keep_logical: bool = False):
    """bf16, 64/8, d=64, sinks ~ N(0, 2): 32 decode seqs (L ~ U[2048, 16384])
    and 2 prefill chunks of 2048 tokens over 8192-token cached prefixes, all in
    one pool and one page table.

    Returns (full, decode_part, prefill_part); the parts share the pool.
    """
    gen = torch.Generator().manual_seed(seed)
    L_dec = _draw_lengths(gen, 32, 2048, 16384)
    L = torch.cat([L_dec, torch.full((2,), 8192 + 2048, dtype=torch.int32)])
    Lq = torch.cat([torch.ones(32, dtype=torch.int32), torch.full((2,), 2048, dtype=torch.int32)])
    full = build_batch(gen, "bf16", L, Lq, 64, 8, 64, sink_mode="normal", sink_std=2.0,
                       keep_logical=keep_logical)
    full.meta["name"] = "mixed"
    dec = full.rows(0, 32)
    dec.meta = {"name": "mixed_decode"}
    pre = full.rows(32, 34)
    pre.meta = {"name": "mixed_prefill"}
    return full, dec, pre


def small_batch(seed: int, dtype: str, seq_lens, q_lens, num_q_heads: int, num_kv_heads: int,
                head_dim: int, **kw) -> PagedBatch:
    """A batch of arbitrary small shape for tests (same recipe, own seed)."""
    gen = torch.Generator().manual_seed(seed)
    return build_batch(gen, dtype, seq_lens, q_lens, num_q_heads, num_kv_heads, head_dim, **kw)
