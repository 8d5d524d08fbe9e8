"""Grouped-query attention over a paged (HND) KV cache with per-head sinks.

Thin ctypes binding of the C ABI in include/attn_sinks.h (libattn_sinks.so,
built for gfx950 by ``python -m gqa_paged_attention_amd.build``).  The
functions below only marshal torch tensors into pointers and sizes; every
step of the computation runs in the library's HIP kernels.  PyTorch supplies
device memory and the current stream.  There is no CPU fallback: if the
library is missing, calling any entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # imported first so the library binds to the HIP runtime torch loaded

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libattn_sinks.so")

ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1
_DTYPE_CODE = {torch.float32: ATTN_DTYPE_F32, torch.bfloat16: ATTN_DTYPE_BF16}
PAGE_SIZE = 16

_lib = None


class AttnSinksError(RuntimeError):
    """A nonzero status from the library (nothing was enqueued unless ATTN_ERR_HIP)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"attn_sinks status {status}: {message}")
        self.status = status


def library():
    """Load libattn_sinks.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m gqa_paged_attention_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    I, P, F, Z = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    lib.attn_sinks_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.attn_sinks_decode_workspace_bytes.restype = Z
    lib.attn_sinks_decode.argtypes = [I] * 9 + [P] * 6 + [F, P, P, Z, P]
    lib.attn_sinks_decode.restype = I
    lib.attn_sinks_decode_partials.argtypes = [I] * 9 + [P] * 5 + [F, P, Z, P]
    lib.attn_sinks_decode_partials.restype = I
    lib.attn_sinks_decode_merge.argtypes = [I] * 6 + [P, P, P, Z, P, P]
    lib.attn_sinks_decode_merge.restype = I
    lib.attn_sinks_prefill.argtypes = [I] * 11 + [P] * 7 + [F, P, P]
    lib.attn_sinks_prefill.restype = I
    lib.attn_sinks_decode_window.argtypes = [I] * 9 + [P] * 6 + [F, I, P, P, Z, P]
    lib.attn_sinks_decode_window.restype = I
    lib.attn_sinks_decode_noalloc.argtypes = [I] * 9 + [P] * 6 + [F, I, P, P]
    lib.attn_sinks_decode_noalloc.restype = I
    lib.attn_sinks_prefill_window.argtypes = [I] * 11 + [P] * 7 + [F, I, P, P]
    lib.attn_sinks_prefill_window.restype = I
    lib.attn_sinks_append_kv.argtypes = [I] * 9 + [P] * 7 + [P]
    lib.attn_sinks_append_kv.restype = I
    lib.attn_sinks_rope_append.argtypes = [I] * 10 + [P] * 4 + [F, F, I, F, F] + [P] * 6
    lib.attn_sinks_rope_append.restype = I
    lib.attn_sinks_decode_append.argtypes = [I] * 9 + [P] * 8 + [F, I, P, P, Z, P]
    lib.attn_sinks_decode_append.restype = I
    lib.attn_sinks_prefill_append.argtypes = [I] * 11 + [P] * 9 + [F, I, P, P]
    lib.attn_sinks_prefill_append.restype = I
    lib.attn_sinks_decode_multi_workspace_bytes.argtypes = [I] * 6
    lib.attn_sinks_decode_multi_workspace_bytes.restype = Z
    lib.attn_sinks_decode_multi.argtypes = [I] * 11 + [P] * 7 + [F, P, P, Z, P]
    lib.attn_sinks_decode_multi.restype = I
    lib.attn_sinks_ragged.argtypes = [I] * 10 + [P] * 6 + [F, P, P, P]
    lib.attn_sinks_mixed.argtypes = [I] * 13 + [P] * 7 + [F, P, P, Z, P]
    lib.attn_sinks_mixed.restype = I
    lib.attn_sinks_ragged.restype = I
    lib.attn_sinks_status_string.argtypes = [I]
    lib.attn_sinks_status_string.restype = ctypes.c_char_p
    lib.attn_sinks_version.argtypes = []
    lib.attn_sinks_version.restype = I
    lib.attn_sinks_set_debug.argtypes = [I, I]
    lib.attn_sinks_set_debug.restype = I
    _lib = lib
    return lib


def attn_sinks_status_string(status: int) -> str:
    return library().attn_sinks_status_string(int(status)).decode()


def attn_sinks_version() -> int:
    return int(library().attn_sinks_version())


ATTN_DEBUG_PREFILL_ONE_HEAD = 0
ATTN_DEBUG_PREFILL_WAIT_ALL = 1
ATTN_DEBUG_PREFILL_WINDOW_STREAMED = 2


def attn_sinks_set_debug(setting: int, value: int) -> int:
    """Set a debug setting for the launches that follow; returns the previous
    value (-1: unknown setting).  Every setting gives the same results."""
    return int(library().attn_sinks_set_debug(int(setting), int(value)))


def attn_sinks_decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                      head_dim: int, max_seq_len: int) -> int:
    return int(library().attn_sinks_decode_workspace_bytes(
        int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim), int(max_seq_len)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _check_dense(name: str, t: Optional[torch.Tensor], dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _raise(status: int):
    if status != 0:
        raise AttnSinksError(status, attn_sinks_status_string(status))


def attn_sinks_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_table: torch.Tensor, seq_lens: torch.Tensor,
                      sinks: Optional[torch.Tensor], scale: float, out: torch.Tensor,
                      workspace: Optional[torch.Tensor], max_seq_len: int, stream=None) -> None:
    """Enqueue attn_sinks_decode on `stream` (default: torch's current stream).

    q [B][Hq][d], k_cache/v_cache [num_pages][Hkv][16][d], block_table
    [B][max_pages] int32, seq_lens [B] int32, sinks [Hq] fp32 or None, out like
    q, workspace a byte (uint8) tensor of at least
    attn_sinks_decode_workspace_bytes(...) bytes.
    """
    _decode(None, q, k_cache, v_cache, block_table, seq_lens, sinks, scale, out, workspace,
            max_seq_len, stream)


def attn_sinks_decode_window(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             block_table: torch.Tensor, seq_lens: torch.Tensor,
                             sinks: Optional[torch.Tensor], scale: float, window: int,
                             out: torch.Tensor, workspace: Optional[torch.Tensor],
                             max_seq_len: int, stream=None) -> None:
    """Enqueue attn_sinks_decode_window: as attn_sinks_decode, each query
    seeing only its sequence's last `window` keys (0: all of them)."""
    _decode(int(window), q, k_cache, v_cache, block_table, seq_lens, sinks, scale, out,
            workspace, max_seq_len, stream)


def attn_sinks_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_table: torch.Tensor, seq_lens: torch.Tensor,
                              sinks: Optional[torch.Tensor], scale: float, window: int,
                              out: torch.Tensor, max_seq_len: int, stream=None) -> None:
    """Enqueue attn_sinks_decode_noalloc: attn_sinks_decode_window with the
    partial results in the library's fixed per-GPU scratch (no workspace)."""
    _decode(int(window), q, k_cache, v_cache, block_table, seq_lens, sinks, scale, out, None,
            max_seq_len, stream, noalloc=True)


def _decode(window, q, k_cache, v_cache, block_table, seq_lens, sinks, scale, out, workspace,
            max_seq_len, stream, noalloc=False):
    dt = _DTYPE_CODE.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out)):
        _check_dense(name, t, q.dtype)
    _check_dense("block_table", block_table, torch.int32)
    _check_dense("seq_lens", seq_lens, torch.int32)
    _check_dense("sinks", sinks, torch.float32)
    _check_dense("workspace", workspace)
    B, Hq, d = q.shape
    num_pages, Hkv, P, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != (B, Hq, d):
        raise ValueError("q / k_cache / v_cache / out shapes disagree")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("block_table / seq_lens do not match the batch")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (dt, B, Hq, Hkv, d, P, num_pages, block_table.shape[1], int(max_seq_len),
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(sinks),
            ctypes.c_float(scale))
    if noalloc:
        _raise(library().attn_sinks_decode_noalloc(*head, window, _ptr(out),
                                                   _stream_handle(stream)))
        return
    tail = (_ptr(out), _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream_handle(stream))
    if window is None:
        status = library().attn_sinks_decode(*head, *tail)
    else:
        status = library().attn_sinks_decode_window(*head, window, *tail)
    _raise(status)


def attn_sinks_mixed(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     block_table: torch.Tensor, seq_lens: torch.Tensor,
                     cu_seqlens_q: torch.Tensor, sinks: Optional[torch.Tensor], scale: float,
                     out: torch.Tensor, num_decode_seqs: int, decode_max_seq_len: int,
                     max_q_len: int, max_seq_len: int, workspace: Optional[torch.Tensor],
                     stream=None) -> None:
    """Enqueue attn_sinks_mixed: sequences [0, num_decode_seqs) are
    single-token decodes in rows 0 .. num_decode_seqs - 1 of q [total_q][Hq][d],
    the rest prefill chunks by cu_seqlens_q [B+1]; workspace as for
    attn_sinks_decode over the decode sequences."""
    dt = _DTYPE_CODE.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out)):
        _check_dense(name, t, q.dtype)
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens),
                    ("cu_seqlens_q", cu_seqlens_q)):
        _check_dense(name, t, torch.int32)
    _check_dense("sinks", sinks, torch.float32)
    _check_dense("workspace", workspace)
    total_q, Hq, d = q.shape
    num_pages, Hkv, P, d2 = k_cache.shape
    B = seq_lens.numel()
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q / k_cache / v_cache / out shapes disagree")
    if block_table.dim() != 2 or block_table.shape[0] != B or cu_seqlens_q.numel() != B + 1:
        raise ValueError("block_table / cu_seqlens_q do not match the batch")
    nd = int(num_decode_seqs)
    if not 0 <= nd <= B:
        raise ValueError("num_decode_seqs out of range")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _raise(library().attn_sinks_mixed(
        dt, nd, B - nd, Hq, Hkv, d, P, num_pages, block_table.shape[1],
        int(decode_max_seq_len), total_q, int(max_q_len), int(max_seq_len), _ptr(q),
        _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(cu_seqlens_q),
        _ptr(sinks), ctypes.c_float(scale), _ptr(out), _ptr(workspace),
        ctypes.c_size_t(ws_bytes), _stream_handle(stream)))


def attn_sinks_decode_partials(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                               workspace: torch.Tensor, max_seq_len: int, stream=None) -> None:
    """Enqueue the split pass of decode (bf16): partial results into workspace."""
    dt = _DTYPE_CODE.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_dense(name, t, q.dtype)
    _check_dense("block_table", block_table, torch.int32)
    _check_dense("seq_lens", seq_lens, torch.int32)
    _check_dense("workspace", workspace)
    B, Hq, d = q.shape
    num_pages, Hkv, P, _ = k_cache.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    status = library().attn_sinks_decode_partials(
        dt, B, Hq, Hkv, d, P, num_pages, block_table.shape[1], int(max_seq_len),
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        ctypes.c_float(scale), _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream_handle(stream))
    _raise(status)


def attn_sinks_decode_merge(seq_lens: torch.Tensor, sinks: Optional[torch.Tensor],
                            workspace: torch.Tensor, out: torch.Tensor, num_kv_heads: int,
                            max_seq_len: int, stream=None) -> None:
    """Enqueue the merge pass of decode: splits + sink -> out [B][Hq][d]."""
    dt = _DTYPE_CODE.get(out.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {out.dtype}")
    _check_dense("out", out)
    _check_dense("seq_lens", seq_lens, torch.int32)
    _check_dense("sinks", sinks, torch.float32)
    _check_dense("workspace", workspace)
    B, Hq, d = out.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    status = library().attn_sinks_decode_merge(
        dt, B, Hq, int(num_kv_heads), d, int(max_seq_len), _ptr(seq_lens), _ptr(sinks),
        _ptr(workspace), ctypes.c_size_t(ws_bytes), _ptr(out), _stream_handle(stream))
    _raise(status)


def attn_sinks_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       block_table: torch.Tensor, seq_lens: torch.Tensor,
                       cu_seqlens_q: torch.Tensor, sinks: Optional[torch.Tensor], scale: float,
                       out: torch.Tensor, max_q_len: int, max_seq_len: int, stream=None) -> None:
    """Enqueue attn_sinks_prefill on `stream` (default: torch's current stream).

    q [total_q][Hq][d] ragged by cu_seqlens_q [B+1] int32; out like q.
    """
    _prefill(None, q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, sinks, scale, out,
             max_q_len, max_seq_len, stream)


def attn_sinks_prefill_window(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_table: torch.Tensor, seq_lens: torch.Tensor,
                              cu_seqlens_q: torch.Tensor, sinks: Optional[torch.Tensor],
                              scale: float, window: int, out: torch.Tensor, max_q_len: int,
                              max_seq_len: int, stream=None) -> None:
    """Enqueue attn_sinks_prefill_window: as attn_sinks_prefill, the row at
    position p seeing keys p - window + 1 .. p (window 0: all up to p)."""
    _prefill(int(window), q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, sinks,
             scale, out, max_q_len, max_seq_len, stream)


def _prefill(window, q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, sinks, scale,
             out, max_q_len, max_seq_len, stream):
    dt = _DTYPE_CODE.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out)):
        _check_dense(name, t, q.dtype)
    _check_dense("block_table", block_table, torch.int32)
    _check_dense("seq_lens", seq_lens, torch.int32)
    _check_dense("cu_seqlens_q", cu_seqlens_q, torch.int32)
    _check_dense("sinks", sinks, torch.float32)
    T, Hq, d = q.shape
    num_pages, Hkv, P, d2 = k_cache.shape
    B = seq_lens.numel()
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != (T, Hq, d):
        raise ValueError("q / k_cache / v_cache / out shapes disagree")
    if block_table.dim() != 2 or block_table.shape[0] != B or cu_seqlens_q.numel() != B + 1:
        raise ValueError("block_table / cu_seqlens_q do not match the batch")
    head = (dt, B, Hq, Hkv, d, P, num_pages, block_table.shape[1], T, int(max_q_len),
            int(max_seq_len), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(cu_seqlens_q), _ptr(sinks), ctypes.c_float(scale))
    tail = (_ptr(out), _stream_handle(stream))
    if window is None:
        status = library().attn_sinks_prefill(*head, *tail)
    else:
        status = library().attn_sinks_prefill_window(*head, window, *tail)
    _raise(status)


def attn_sinks_append_kv(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                         v_cache: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, cu_seqlens_new: Optional[torch.Tensor],
                         max_seq_len: int, stream=None) -> None:
    """Enqueue attn_sinks_append_kv: rows k_new / v_new [total_new][Hkv][d]
    into their page slots (the last n_b positions of each sequence, n_b from
    cu_seqlens_new [B+1] int32, or one token per sequence when None)."""
    dt = _DTYPE_CODE.get(k_cache.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {k_cache.dtype}")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _check_dense(name, t, k_cache.dtype)
    _check_dense("block_table", block_table, torch.int32)
    _check_dense("seq_lens", seq_lens, torch.int32)
    _check_dense("cu_seqlens_new", cu_seqlens_new, torch.int32)
    num_pages, Hkv, P, d = k_cache.shape
    T = k_new.shape[0]
    B = seq_lens.numel()
    if tuple(k_new.shape) != (T, Hkv, d) or tuple(v_new.shape) != (T, Hkv, d) or \
            tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_new / v_new / cache shapes disagree")
    status = library().attn_sinks_append_kv(
        dt, B, Hkv, d, P, num_pages, block_table.shape[1], int(max_seq_len), T, _ptr(k_new),
        _ptr(v_new), _ptr(block_table), _ptr(seq_lens), _ptr(cu_seqlens_new), _ptr(k_cache),
        _ptr(v_cache), _stream_handle(stream))
    _raise(status)


def attn_sinks_rope_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                           positions: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_table: torch.Tensor, seq_lens: torch.Tensor,
                           cu_seqlens_new: Optional[torch.Tensor], max_seq_len: int,
                           rope_base: float, rope_scale: float, orig_ctx: int = 4096,
                           beta_fast: float = 32.0, beta_slow: float = 1.0, stream=None) -> None:
    """Enqueue attn_sinks_rope_append: rotate q [total_new][Hq][d] in place and
    the new K rows into their cache slots (NeoX RoPE, YaRN scaling, rotary
    positions int32 [total_new]), append V; placement as attn_sinks_append_kv."""
    dt = _DTYPE_CODE.get(k_cache.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {k_cache.dtype}")
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _check_dense(name, t, k_cache.dtype)
    for name, t in (("positions", positions), ("block_table", block_table),
                    ("seq_lens", seq_lens), ("cu_seqlens_new", cu_seqlens_new)):
        _check_dense(name, t, torch.int32)
    num_pages, Hkv, P, d = k_cache.shape
    T = k_new.shape[0]
    Hq = q.shape[1]
    B = seq_lens.numel()
    if tuple(k_new.shape) != (T, Hkv, d) or tuple(v_new.shape) != (T, Hkv, d) or \
            tuple(q.shape) != (T, Hq, d) or positions.numel() != T or \
            tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q / k_new / v_new / positions / cache shapes disagree")
    status = library().attn_sinks_rope_append(
        dt, B, Hq, Hkv, d, P, num_pages, block_table.shape[1], int(max_seq_len), T, _ptr(q),
        _ptr(k_new), _ptr(v_new), _ptr(positions), float(rope_base), float(rope_scale),
        int(orig_ctx), float(beta_fast), float(beta_slow), _ptr(block_table), _ptr(seq_lens),
        _ptr(cu_seqlens_new), _ptr(k_cache), _ptr(v_cache), _stream_handle(stream))
    _raise(status)


def attn_sinks_decode_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, sinks,
                             scale: float, window: int, out, workspace, max_seq_len: int,
                             stream=None) -> None:
    """Enqueue attn_sinks_decode_append: append one token per sequence, then
    the (windowed) decode."""
    dt = _DTYPE_CODE.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache), ("out", out)):
        _check_dense(name, t, q.dtype)
    _check_dense("block_table", block_table, torch.int32)
    _check_dense("seq_lens", seq_lens, torch.int32)
    _check_dense("sinks", sinks, torch.float32)
    _check_dense("workspace", workspace)
    B, Hq, d = q.shape
    num_pages, Hkv, P, _ = k_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    status = library().attn_sinks_decode_append(
        dt, B, Hq, Hkv, d, P, num_pages, block_table.shape[1], int(max_seq_len), _ptr(q),
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(sinks), ctypes.c_float(scale), int(window), _ptr(out),
        _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream_handle(stream))
    _raise(status)


def attn_sinks_prefill_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                              cu_seqlens_q, sinks, scale: float, window: int, out,
                              max_q_len: int, max_seq_len: int, stream=None) -> None:
    """Enqueue attn_sinks_prefill_append: append the chunk's tokens, then the
    (windowed) causal prefill."""
    dt = _DTYPE_CODE.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache), ("out", out)):
        _check_dense(name, t, q.dtype)
    _check_dense("block_table", block_table, torch.int32)
    _check_dense("seq_lens", seq_lens, torch.int32)
    _check_dense("cu_seqlens_q", cu_seqlens_q, torch.int32)
    _check_dense("sinks", sinks, torch.float32)
    T, Hq, d = q.shape
    num_pages, Hkv, P, _ = k_cache.shape
    B = seq_lens.numel()
    status = library().attn_sinks_prefill_append(
        dt, B, Hq, Hkv, d, P, num_pages, block_table.shape[1], T, int(max_q_len),
        int(max_seq_len), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), _ptr(cu_seqlens_q), _ptr(sinks),
        ctypes.c_float(scale), int(window), _ptr(out), _stream_handle(stream))
    _raise(status)


def attn_sinks_decode_multi_workspace_bytes(num_seqs: int, num_q_heads: int,
                                            num_kv_heads: int, head_dim: int, max_seq_len: int,
                                            max_q_len: int) -> int:
    return int(library().attn_sinks_decode_multi_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, max_q_len))


def attn_sinks_decode_multi(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, sinks,
                            scale: float, out, workspace, max_q_len: int, max_seq_len: int,
                            stream=None) -> None:
    """Enqueue attn_sinks_decode_multi: a few new tokens per sequence (rows
    of q as cu_seqlens_q says); the result of attn_sinks_prefill, computed by
    the split decode passes with GQA-packed rows where the shape allows."""
    dt = _DTYPE_CODE.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out)):
        _check_dense(name, t, q.dtype)
    _check_dense("block_table", block_table, torch.int32)
    _check_dense("seq_lens", seq_lens, torch.int32)
    _check_dense("cu_seqlens_q", cu_seqlens_q, torch.int32)
    _check_dense("sinks", sinks, torch.float32)
    _check_dense("workspace", workspace)
    T, Hq, d = q.shape
    num_pages, Hkv, P, _ = k_cache.shape
    B = seq_lens.numel()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    status = library().attn_sinks_decode_multi(
        dt, B, Hq, Hkv, d, P, num_pages, block_table.shape[1], T, int(max_q_len),
        int(max_seq_len), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(cu_seqlens_q), _ptr(sinks), ctypes.c_float(scale), _ptr(out),
        _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream_handle(stream))
    _raise(status)


def attn_sinks_ragged(q, k, v, cu_seqlens_q, cu_seqlens_kv, sinks, scale: float, causal: bool,
                      out, lse, max_q_len: int, max_kv_len: int, stream=None) -> None:
    """Enqueue attn_sinks_ragged: contiguous K/V rows per sequence (no KV
    cache), optional causal mask, out [total_q][Hq][d] and, when `lse` is a
    tensor, the fp32 natural-log LSE [total_q][Hq]."""
    dt = _DTYPE_CODE.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_dense(name, t, q.dtype)
    _check_dense("cu_seqlens_q", cu_seqlens_q, torch.int32)
    _check_dense("cu_seqlens_kv", cu_seqlens_kv, torch.int32)
    _check_dense("sinks", sinks, torch.float32)
    _check_dense("lse", lse, torch.float32)
    T, Hq, d = q.shape
    Tk, Hkv, d2 = k.shape
    B = cu_seqlens_q.numel() - 1
    if d2 != d or tuple(v.shape) != tuple(k.shape) or tuple(out.shape) != (T, Hq, d):
        raise ValueError("q / k / v / out shapes disagree")
    if cu_seqlens_kv.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv differ in length")
    status = library().attn_sinks_ragged(
        dt, B, Hq, Hkv, d, T, Tk, int(max_q_len), int(max_kv_len), int(bool(causal)), _ptr(q),
        _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), _ptr(sinks),
        ctypes.c_float(scale), _ptr(out), _ptr(lse), _stream_handle(stream))
    _raise(status)


# ------------------------------------------------------------ conveniences

def decode_batch(batch, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None,
                 window: Optional[int] = None) -> torch.Tensor:
    """Run attn_sinks_decode (attn_sinks_decode_window when `window` is given)
    on a workloads.PagedBatch already on the GPU."""
    if out is None:
        out = torch.empty_like(batch.q)
    if workspace is None:
        nbytes = attn_sinks_decode_workspace_bytes(batch.num_seqs, batch.num_q_heads,
                                                   batch.num_kv_heads, batch.head_dim,
                                                   batch.max_seq_len)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=batch.q.device)
    args = (batch.q, batch.k_cache, batch.v_cache, batch.block_table, batch.seq_lens,
            batch.sinks, batch.scale)
    if window is None:
        attn_sinks_decode(*args, out, workspace, batch.max_seq_len, stream)
    else:
        attn_sinks_decode_window(*args, window, out, workspace, batch.max_seq_len, stream)
    return out


def prefill_batch(batch, out: Optional[torch.Tensor] = None, stream=None,
                  window: Optional[int] = None) -> torch.Tensor:
    """Run attn_sinks_prefill (attn_sinks_prefill_window when `window` is
    given) on a workloads.PagedBatch already on the GPU."""
    if out is None:
        out = torch.empty_like(batch.q)
    args = (batch.q, batch.k_cache, batch.v_cache, batch.block_table, batch.seq_lens,
            batch.cu_seqlens_q, batch.sinks, batch.scale)
    if window is None:
        attn_sinks_prefill(*args, out, batch.max_q_len, batch.max_seq_len, stream)
    else:
        attn_sinks_prefill_window(*args, window, out, batch.max_q_len, batch.max_seq_len, stream)
    return out
