"""The C-ABI library loads, exports what include/attn_sinks.h declares, and
rejects bad arguments on the host before enqueuing anything (CPU only: no
call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import gqa_paged_attention_amd as ga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_sinks.h")

# status codes as the header defines them
OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_ALIGN, ERR_HIP, ERR_SCRATCH = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_sinks_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ga.LIB_PATH):
        pytest.fail("libattn_sinks.so is not built (python -m gqa_paged_attention_amd.build)")
    return ga.library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"attn_sinks_decode", "attn_sinks_prefill",
                          "attn_sinks_decode_workspace_bytes", "attn_sinks_status_string"}
    for name in names:
        assert hasattr(lib, name), f"{name} declared but not exported"


def test_status_strings_and_version(lib):
    for code in range(8):
        s = ga.attn_sinks_status_string(code)
        assert isinstance(s, str) and s
    assert ga.attn_sinks_status_string(99) == "unknown status"
    assert ga.attn_sinks_version() >= 100


def _expected_ws(B, Hq, Hkv, d, max_len):
    """The layout the header documents: W workgroups per group of up to 4 KV
    heads (4-wave workgroups on 192 of the 256 CUs, smaller ones 4 waves per
    CU on all 256, capped by the unit count); slots = B + W; ml
    [slots][Hq][2] padded to a multiple of 4 floats, then acc [slots][Hq][d]."""
    per_wg = min(Hkv, 4)
    groups = -(-Hkv // per_wg)
    cus = 192 if per_wg >= 4 else 256
    w = max((cus * max(4, per_wg) // per_wg) // groups, 1)
    w = min(w, B * ((max_len + 31) // 32))
    if w == 0:
        return 0
    slots = B + w
    ml = (slots * Hq * 2 + 3) // 4 * 4
    return (ml + slots * Hq * d) * 4


def test_workspace_bytes(lib):
    for args in [(64, 64, 8, 64, 8192), (128, 64, 4, 128, 32768), (1, 4, 1, 64, 257),
                 (3, 8, 2, 128, 100), (32, 64, 8, 64, 16384)]:
        assert ga.attn_sinks_decode_workspace_bytes(*args) == _expected_ws(*args), args
    assert ga.attn_sinks_decode_workspace_bytes(64, 64, 8, 64, 0) == 0
    assert ga.attn_sinks_decode_workspace_bytes(64, 64, 8, 96, 8192) == 0   # head_dim
    assert ga.attn_sinks_decode_workspace_bytes(64, 64, 7, 64, 8192) == 0   # Hq % Hkv
    assert ga.attn_sinks_decode_workspace_bytes(64, 64, 2, 64, 8192) == 0   # group 32 > 16
    # monotone in the length bound
    a = ga.attn_sinks_decode_workspace_bytes(8, 16, 2, 128, 1000)
    b = ga.attn_sinks_decode_workspace_bytes(8, 16, 2, 128, 100000)
    assert 0 < a <= b


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced


def _decode(lib, **kw):
    args = dict(dtype=1, B=2, Hq=8, Hkv=2, d=64, P=16, pages=8, max_pages=4, max_len=64,
                q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, sinks=None, scale=0.125, out=FAKE,
                ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    return lib.attn_sinks_decode(
        args["dtype"], args["B"], args["Hq"], args["Hkv"], args["d"], args["P"], args["pages"],
        args["max_pages"], args["max_len"], args["q"], args["k"], args["v"], args["bt"],
        args["sl"], args["sinks"], ctypes.c_float(args["scale"]), args["out"], args["ws"],
        ctypes.c_size_t(args["ws_bytes"]), None)


def _prefill(lib, **kw):
    args = dict(dtype=1, B=2, Hq=8, Hkv=2, d=64, P=16, pages=8, max_pages=4, total_q=40,
                max_q=32, max_len=64, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, cu=FAKE,
                sinks=None, scale=0.125, out=FAKE)
    args.update(kw)
    return lib.attn_sinks_prefill(
        args["dtype"], args["B"], args["Hq"], args["Hkv"], args["d"], args["P"], args["pages"],
        args["max_pages"], args["total_q"], args["max_q"], args["max_len"], args["q"],
        args["k"], args["v"], args["bt"], args["sl"], args["cu"], args["sinks"],
        ctypes.c_float(args["scale"]), args["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), ERR_UNSUPPORTED),
    (dict(d=96), ERR_UNSUPPORTED),
    (dict(P=32), ERR_UNSUPPORTED),
    (dict(Hkv=3), ERR_SHAPE),
    (dict(Hq=64, Hkv=2), ERR_UNSUPPORTED),
    (dict(B=-1), ERR_SHAPE),
    (dict(max_len=65), ERR_SHAPE),           # > max_pages * 16
    (dict(scale=float("nan")), ERR_SHAPE),
    (dict(scale=float("inf")), ERR_SHAPE),
    (dict(q=None), ERR_NULL),
    (dict(out=None), ERR_NULL),
    (dict(bt=None), ERR_NULL),
    (dict(ws=None), ERR_NULL),
    (dict(ws_bytes=16), ERR_WORKSPACE),
    (dict(q=FAKE + 8), ERR_ALIGN),
    (dict(k=FAKE + 4), ERR_ALIGN),
    (dict(sl=FAKE + 2), ERR_ALIGN),
])
def test_decode_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), ERR_UNSUPPORTED),
    (dict(d=32), ERR_UNSUPPORTED),
    (dict(Hkv=5), ERR_SHAPE),
    (dict(max_q=65), ERR_SHAPE),             # > max_len
    (dict(max_q=41), ERR_SHAPE),             # > total_q
    (dict(total_q=-1), ERR_SHAPE),
    (dict(scale=float("nan")), ERR_SHAPE),
    (dict(cu=None), ERR_NULL),
    (dict(v=None), ERR_NULL),
    (dict(out=FAKE + 8), ERR_ALIGN),
    (dict(cu=FAKE + 1), ERR_ALIGN),
])
def test_prefill_rejects(lib, kw, code):
    assert _prefill(lib, **kw) == code


def test_empty_batches_enqueue_nothing(lib):
    # zero sequences / zero query rows return OK without touching the GPU
    assert _decode(lib, B=0) == OK
    assert _prefill(lib, B=0) == OK
    assert _prefill(lib, total_q=0, max_q=0) == OK


def test_binding_raises_on_status(lib):
    with pytest.raises(ga.AttnSinksError) as ei:
        ga._raise(ERR_SHAPE)
    assert ei.value.status == ERR_SHAPE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(ga, "_lib", None)
    monkeypatch.setattr(ga, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ga.library()


def _decode_window(lib, window, **kw):
    args = dict(dtype=1, B=2, Hq=8, Hkv=2, d=64, P=16, pages=8, max_pages=4, max_len=64,
                q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, sinks=None, scale=0.125, out=FAKE,
                ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    return lib.attn_sinks_decode_window(
        args["dtype"], args["B"], args["Hq"], args["Hkv"], args["d"], args["P"], args["pages"],
        args["max_pages"], args["max_len"], args["q"], args["k"], args["v"], args["bt"],
        args["sl"], args["sinks"], ctypes.c_float(args["scale"]), window, args["out"],
        args["ws"], ctypes.c_size_t(args["ws_bytes"]), None)


def _prefill_window(lib, window, **kw):
    args = dict(dtype=1, B=2, Hq=8, Hkv=2, d=64, P=16, pages=8, max_pages=4, total_q=40,
                max_q=32, max_len=64, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, cu=FAKE,
                sinks=None, scale=0.125, out=FAKE)
    args.update(kw)
    return lib.attn_sinks_prefill_window(
        args["dtype"], args["B"], args["Hq"], args["Hkv"], args["d"], args["P"], args["pages"],
        args["max_pages"], args["total_q"], args["max_q"], args["max_len"], args["q"],
        args["k"], args["v"], args["bt"], args["sl"], args["cu"], args["sinks"],
        ctypes.c_float(args["scale"]), window, args["out"], None)


@pytest.mark.parametrize("call", [_decode_window, _prefill_window], ids=["decode", "prefill"])
def test_window_entry_points_check_like_the_plain_ones(lib, call):
    assert call(lib, -1) == ERR_SHAPE
    assert call(lib, -1000) == ERR_SHAPE
    assert call(lib, 128, dtype=2) == ERR_UNSUPPORTED
    assert call(lib, 128, q=None) == ERR_NULL
    assert call(lib, 128, out=FAKE + 8) == ERR_ALIGN
    assert call(lib, 128, scale=float("nan")) == ERR_SHAPE
    assert call(lib, 0, B=0) == OK
    assert call(lib, 128, B=0) == OK


def _append(lib, **kw):
    args = dict(dtype=1, B=2, Hkv=2, d=64, P=16, pages=8, max_pages=4, max_len=64, T=5,
                k_new=FAKE, v_new=FAKE, bt=FAKE, sl=FAKE, cu=FAKE, kc=FAKE, vc=FAKE)
    args.update(kw)
    return lib.attn_sinks_append_kv(
        args["dtype"], args["B"], args["Hkv"], args["d"], args["P"], args["pages"],
        args["max_pages"], args["max_len"], args["T"], args["k_new"], args["v_new"], args["bt"],
        args["sl"], args["cu"], args["kc"], args["vc"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), ERR_UNSUPPORTED),
    (dict(d=80), ERR_UNSUPPORTED),
    (dict(P=8), ERR_UNSUPPORTED),
    (dict(T=-1), ERR_SHAPE),
    (dict(cu=None, T=5), ERR_SHAPE),          # one token per sequence needs T == B
    (dict(max_len=0), ERR_SHAPE),             # new tokens need a page
    (dict(max_len=65), ERR_SHAPE),
    (dict(k_new=None), ERR_NULL),
    (dict(vc=None), ERR_NULL),
    (dict(bt=None), ERR_NULL),
    (dict(v_new=FAKE + 8), ERR_ALIGN),
    (dict(kc=FAKE + 4), ERR_ALIGN),
    (dict(cu=FAKE + 2), ERR_ALIGN),
])
def test_append_rejects(lib, kw, code):
    assert _append(lib, **kw) == code


def _rope(lib, **kw):
    args = dict(dtype=1, B=2, Hq=8, Hkv=2, d=64, P=16, pages=8, max_pages=4, max_len=64, T=5,
                q=FAKE, k_new=FAKE, v_new=FAKE, pos=FAKE, base=10000.0, scale=32.0, orig=4096,
                bf=32.0, bs=1.0, bt=FAKE, sl=FAKE, cu=FAKE, kc=FAKE, vc=FAKE)
    args.update(kw)
    F = ctypes.c_float
    return lib.attn_sinks_rope_append(
        args["dtype"], args["B"], args["Hq"], args["Hkv"], args["d"], args["P"], args["pages"],
        args["max_pages"], args["max_len"], args["T"], args["q"], args["k_new"], args["v_new"],
        args["pos"], F(args["base"]), F(args["scale"]), args["orig"], F(args["bf"]),
        F(args["bs"]), args["bt"], args["sl"], args["cu"], args["kc"], args["vc"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), ERR_UNSUPPORTED),
    (dict(d=80), ERR_UNSUPPORTED),
    (dict(Hq=7), ERR_SHAPE),                  # Hq not a multiple of Hkv
    (dict(Hq=64), ERR_UNSUPPORTED),           # group of 32
    (dict(T=-1), ERR_SHAPE),
    (dict(base=0.0), ERR_SHAPE),
    (dict(base=float("inf")), ERR_SHAPE),
    (dict(scale=0.0), ERR_SHAPE),
    (dict(scale=float("nan")), ERR_SHAPE),
    (dict(orig=0), ERR_SHAPE),
    (dict(bf=1.0, bs=1.0), ERR_SHAPE),        # empty ramp with scale != 1
    (dict(bf=float("nan")), ERR_SHAPE),
    (dict(bs=0.0), ERR_SHAPE),                # no pair turns zero times
    (dict(bf=-1.0, bs=-2.0), ERR_SHAPE),
    (dict(base=1.0), ERR_SHAPE),              # ln(base) = 0
    (dict(q=None), ERR_NULL),
    (dict(pos=None), ERR_NULL),
    (dict(k_new=None), ERR_NULL),
    (dict(q=FAKE + 8), ERR_ALIGN),
    (dict(pos=FAKE + 2), ERR_ALIGN),
])
def test_rope_append_rejects(lib, kw, code):
    assert _rope(lib, **kw) == code


def test_rope_append_scale_one_needs_no_ramp(lib):
    # plain RoPE: the ramp bounds are not used, and nothing is launched for T = 0
    assert _rope(lib, scale=1.0, bf=1.0, bs=1.0, T=0) == OK
    assert _rope(lib, T=0) == OK


def test_append_empty_enqueues_nothing(lib):
    assert _append(lib, T=0) == OK
    assert _append(lib, B=0, T=0) == OK


def test_combined_calls_check_before_enqueueing(lib):
    # bad decode arguments: rejected before the append is launched
    rc = lib.attn_sinks_decode_append(1, 2, 8, 2, 64, 16, 8, 4, 64, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, None, ctypes.c_float(0.125), -1, FAKE,
                                      FAKE, ctypes.c_size_t(1 << 30), None)
    assert rc == ERR_SHAPE
    rc = lib.attn_sinks_decode_append(1, 2, 8, 2, 64, 16, 8, 4, 64, FAKE, None, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, None, ctypes.c_float(0.125), 0, FAKE,
                                      FAKE, ctypes.c_size_t(1 << 30), None)
    assert rc == ERR_NULL
    rc = lib.attn_sinks_prefill_append(1, 2, 8, 2, 64, 16, 8, 4, 40, 32, 64, FAKE, FAKE, FAKE,
                                       FAKE + 4, FAKE, FAKE, FAKE, FAKE, None,
                                       ctypes.c_float(0.125), 0, FAKE, None)
    assert rc == ERR_ALIGN
    rc = lib.attn_sinks_prefill_append(1, 2, 8, 2, 64, 16, 8, 4, 40, 41, 64, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                       ctypes.c_float(0.125), 0, FAKE, None)
    assert rc == ERR_SHAPE


def test_multi_workspace_bytes(lib):
    # packed shapes: the decode layout with max_q_len query rows per slot
    for B, Hq, Hkv, d, L, q in [(64, 64, 8, 64, 8192, 4), (3, 8, 2, 64, 100, 2),
                                (16, 16, 1, 128, 5000, 1), (5, 8, 8, 64, 300, 8)]:
        one = _expected_ws(B, Hq, Hkv, d, L)
        got = ga.attn_sinks_decode_multi_workspace_bytes(B, Hq, Hkv, d, L, q)
        assert got > 0 and got >= one * q * 0.99, (B, Hq, Hkv, d, L, q)
        if q == 1:
            assert got == one
    # shapes that run the prefill kernel need no workspace
    assert ga.attn_sinks_decode_multi_workspace_bytes(64, 64, 8, 64, 8192, 17) == 0  # 136 rows
    assert ga.attn_sinks_decode_multi_workspace_bytes(4, 64, 4, 128, 9000, 9) == 0   # 144 rows
    # up to 128 packed rows take the split passes, in layers
    assert ga.attn_sinks_decode_multi_workspace_bytes(64, 64, 8, 64, 8192, 9) > 0    # 72 rows
    assert ga.attn_sinks_decode_multi_workspace_bytes(4, 64, 4, 128, 9000, 8) > 0    # 128 rows
    assert ga.attn_sinks_decode_multi_workspace_bytes(4, 64, 8, 96, 9000, 2) == 0    # head_dim


def _multi(lib, **kw):
    args = dict(dtype=1, B=2, Hq=8, Hkv=2, d=64, P=16, pages=8, max_pages=4, total_q=6,
                max_q=4, max_len=64, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, cu=FAKE,
                sinks=None, scale=0.125, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    return lib.attn_sinks_decode_multi(
        args["dtype"], args["B"], args["Hq"], args["Hkv"], args["d"], args["P"], args["pages"],
        args["max_pages"], args["total_q"], args["max_q"], args["max_len"], args["q"],
        args["k"], args["v"], args["bt"], args["sl"], args["cu"], args["sinks"],
        ctypes.c_float(args["scale"]), args["out"], args["ws"],
        ctypes.c_size_t(args["ws_bytes"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), ERR_UNSUPPORTED),
    (dict(max_q=7), ERR_SHAPE),             # > total_q
    (dict(max_q=65, total_q=100), ERR_SHAPE),  # > max_len (prefill path)
    (dict(cu=None), ERR_NULL),
    (dict(ws=None), ERR_NULL),
    (dict(ws_bytes=64), ERR_WORKSPACE),
    (dict(cu=FAKE + 2), ERR_ALIGN),
    (dict(q=FAKE + 8), ERR_ALIGN),
    (dict(scale=float("nan")), ERR_SHAPE),
])
def test_multi_rejects(lib, kw, code):
    assert _multi(lib, **kw) == code


def test_multi_empty(lib):
    assert _multi(lib, B=0) == OK
    assert _multi(lib, total_q=0, max_q=0) == OK


def _ragged(lib, **kw):
    args = dict(dtype=1, B=2, Hq=8, Hkv=2, d=64, Tq=40, Tk=100, mq=32, mk=64, causal=1,
                q=FAKE, k=FAKE, v=FAKE, cq=FAKE, ck=FAKE, sinks=None, scale=0.125, out=FAKE,
                lse=None)
    args.update(kw)
    return lib.attn_sinks_ragged(
        args["dtype"], args["B"], args["Hq"], args["Hkv"], args["d"], args["Tq"], args["Tk"],
        args["mq"], args["mk"], args["causal"], args["q"], args["k"], args["v"], args["cq"],
        args["ck"], args["sinks"], ctypes.c_float(args["scale"]), args["out"], args["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), ERR_UNSUPPORTED),        # bf16 only
    (dict(dtype=9), ERR_UNSUPPORTED),
    (dict(d=256), ERR_UNSUPPORTED),
    (dict(Hkv=3), ERR_SHAPE),
    (dict(causal=2), ERR_SHAPE),
    (dict(mq=41), ERR_SHAPE),                # > total_q
    (dict(mk=101), ERR_SHAPE),               # > total_kv
    (dict(mq=40, mk=30), ERR_SHAPE),         # causal rows need Lq <= L
    (dict(mk=1 << 21, Tk=1 << 22, Hkv=8, Hq=8), ERR_SHAPE),   # 31-bit row offsets
    (dict(scale=float("nan")), ERR_SHAPE),
    (dict(ck=None), ERR_NULL),
    (dict(k=None), ERR_NULL),
    (dict(out=FAKE + 8), ERR_ALIGN),
    (dict(lse=FAKE + 2), ERR_ALIGN),
])
def test_ragged_rejects(lib, kw, code):
    assert _ragged(lib, **kw) == code


def test_ragged_noncausal_allows_more_rows_than_keys(lib):
    assert _ragged(lib, causal=0, mq=40, mk=30, B=0) == OK
    assert _ragged(lib, Tq=0, mq=0) == OK


def _noalloc(lib, **kw):
    args = dict(dtype=1, B=2, Hq=8, Hkv=2, d=64, P=16, pages=8, max_pages=4, max_len=64,
                q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, sinks=None, scale=0.125, window=0,
                out=FAKE)
    args.update(kw)
    return lib.attn_sinks_decode_noalloc(
        args["dtype"], args["B"], args["Hq"], args["Hkv"], args["d"], args["P"], args["pages"],
        args["max_pages"], args["max_len"], args["q"], args["k"], args["v"], args["bt"],
        args["sl"], args["sinks"], ctypes.c_float(args["scale"]), args["window"], args["out"],
        None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), ERR_UNSUPPORTED),
    (dict(d=96), ERR_UNSUPPORTED),
    (dict(Hkv=3), ERR_SHAPE),
    (dict(max_len=65), ERR_SHAPE),
    (dict(window=-1), ERR_SHAPE),
    (dict(scale=float("nan")), ERR_SHAPE),
    (dict(q=None), ERR_NULL),
    (dict(out=FAKE + 8), ERR_ALIGN),
    # more partial results than the fixed 32 MiB scratch holds
    (dict(B=2000, Hq=64, Hkv=8, pages=1, max_pages=512, max_len=8192), ERR_SCRATCH),
    (dict(B=0), OK),
])
def test_noalloc_rejects(lib, kw, code):
    assert _noalloc(lib, **kw) == code


def test_noalloc_limit_is_the_workspace_size(lib):
    # the call takes exactly the sizes whose decode workspace fits 32 MiB
    limit = 32 << 20
    assert ga.attn_sinks_decode_workspace_bytes(1800, 64, 8, 64, 8192) <= limit
    assert ga.attn_sinks_decode_workspace_bytes(700, 64, 4, 128, 32768) <= limit
    assert ga.attn_sinks_decode_workspace_bytes(2000, 64, 8, 64, 8192) > limit


def test_debug_settings(lib):
    # set returns the previous value; unknown settings give -1 and change nothing
    for s in (ga.ATTN_DEBUG_PREFILL_ONE_HEAD, ga.ATTN_DEBUG_PREFILL_WAIT_ALL,
              ga.ATTN_DEBUG_PREFILL_WINDOW_STREAMED):
        before = ga.attn_sinks_set_debug(s, 1)
        assert before in (0, 1)
        assert ga.attn_sinks_set_debug(s, 0) == 1
        assert ga.attn_sinks_set_debug(s, before) == 0
    assert ga.attn_sinks_set_debug(3, 1) == -1
    assert ga.attn_sinks_set_debug(-1, 1) == -1


def _mixed(lib, **kw):
    # 2 decode sequences (rows 0, 1) and 1 prefill chunk of 30 rows
    args = dict(dtype=1, nd=2, np=1, Hq=8, Hkv=2, d=64, P=16, pages=16, max_pages=4,
                dec_len=64, Tq=32, mq=30, max_len=64, q=FAKE, k=FAKE, v=FAKE, bt=FAKE,
                sl=FAKE, cu=FAKE, sinks=None, scale=0.125, out=FAKE, ws=FAKE,
                ws_bytes=1 << 20)
    args.update(kw)
    return lib.attn_sinks_mixed(
        args["dtype"], args["nd"], args["np"], args["Hq"], args["Hkv"], args["d"], args["P"],
        args["pages"], args["max_pages"], args["dec_len"], args["Tq"], args["mq"],
        args["max_len"], args["q"], args["k"], args["v"], args["bt"], args["sl"], args["cu"],
        args["sinks"], ctypes.c_float(args["scale"]), args["out"], args["ws"],
        ctypes.c_size_t(args["ws_bytes"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), ERR_UNSUPPORTED),
    (dict(nd=-1), ERR_SHAPE),
    (dict(np=-1), ERR_SHAPE),
    (dict(nd=40000, np=30000), ERR_SHAPE),
    (dict(Tq=1), ERR_SHAPE),              # fewer rows than decode sequences
    (dict(dec_len=65), ERR_SHAPE),        # beyond max_pages * 16
    (dict(mq=33), ERR_SHAPE),             # more chunk rows than rows
    (dict(scale=float("inf")), ERR_SHAPE),
    (dict(q=None), ERR_NULL),
    (dict(cu=None), ERR_NULL),
    (dict(ws=None), ERR_NULL),
    (dict(ws_bytes=16), ERR_WORKSPACE),
    (dict(out=FAKE + 4), ERR_ALIGN),
    (dict(cu=FAKE + 2), ERR_ALIGN),
])
def test_mixed_rejects(lib, kw, code):
    assert _mixed(lib, **kw) == code


def test_mixed_empty_parts_enqueue_nothing(lib):
    # nothing to compute in either part: checks pass, nothing is launched
    assert _mixed(lib, nd=0, np=0, Tq=0, mq=0, dec_len=0, max_len=0) == OK
    assert _mixed(lib, nd=0, np=1, Tq=0, mq=0) == OK
