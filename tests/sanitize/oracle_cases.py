"""Run the oracle's C function on small edge cases and save the outputs.

Run as a script by tests/test_sanitizers.py, once against the normal build
of oracle.c and once, under AddressSanitizer and UndefinedBehaviorSanitizer,
against an instrumented build.  Uses numpy and ctypes only (no torch), so the
sanitizer runtime preloaded into this process sees nothing but the oracle.

    python oracle_cases.py LIB OUT.npz
"""
import ctypes
import sys

import numpy as np

P = ctypes.c_void_p


def bf16_bits(x):
    u = np.asarray(x, np.float32).view(np.uint32)
    # round to nearest even
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def case(rng, dtype, lens, qlens, hq, hkv, d, sinks, window, causal, spare=3):
    B = len(lens)
    pages = [(L + 15) // 16 for L in lens]
    maxp = max(max(pages), 1)
    npages = sum(pages) + spare
    perm = rng.permutation(npages).astype(np.int32)
    bt = np.full((B, maxp), -1, np.int32)
    k = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[k:k + pages[b]]
        k += pages[b]
    kv = rng.standard_normal((2, npages, hkv, 16, d)).astype(np.float32)
    T = int(sum(qlens))
    q = rng.standard_normal((T, hq, d)).astype(np.float32)
    if dtype == 1:
        q, kv = bf16_bits(q), bf16_bits(kv)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    s = None if sinks is None else np.asarray(sinks, np.float32)
    rows_t = np.repeat(np.arange(T, dtype=np.int64), hq)
    rows_h = np.tile(np.arange(hq, dtype=np.int32), T)
    return dict(dtype=dtype, B=B, hq=hq, hkv=hkv, d=d, maxp=maxp, q=np.ascontiguousarray(q),
                k=np.ascontiguousarray(kv[0]), v=np.ascontiguousarray(kv[1]), bt=bt,
                sl=np.asarray(lens, np.int32), cu=cu, sinks=s, window=window, causal=causal,
                rt=rows_t, rh=rows_h)


def run(lib, c):
    n = c["rt"].size
    out = np.zeros((n, c["d"]), np.float64)
    lse = np.zeros(n, np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data_as(P)
    rc = lib.oracle_attention_rows(
        c["dtype"], c["B"], c["hq"], c["hkv"], c["d"], 16, c["maxp"], ptr(c["q"]), ptr(c["k"]),
        ptr(c["v"]), ptr(c["bt"]), ptr(c["sl"]), ptr(c["cu"]), ptr(c["sinks"]),
        ctypes.c_double(0.125), c["window"], c["causal"], ctypes.c_int64(n), ptr(c["rt"]),
        ptr(c["rh"]), ptr(out), ptr(lse), 2)
    assert rc == 0, rc
    return out, lse


def main(path, dest):
    lib = ctypes.CDLL(path)
    f = lib.oracle_attention_rows
    f.argtypes = [ctypes.c_int] * 7 + [P] * 6 + [P, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int64, P, P, P, P, ctypes.c_int]
    f.restype = ctypes.c_int
    rng = np.random.default_rng(5)
    cases = [
        case(rng, 0, [37, 1, 64], [5, 1, 64], 8, 2, 16, rng.standard_normal(8), 0, 1),
        case(rng, 1, [130, 17], [1, 17], 4, 4, 64, None, 0, 1),
        case(rng, 1, [0, 40], [0, 3], 6, 3, 32, [-np.inf] * 6, 0, 1),      # an empty sequence
        case(rng, 0, [100, 33], [20, 33], 4, 1, 8, [50.0] * 4, 7, 1),      # window, big sink
        case(rng, 1, [12, 29], [30, 5], 2, 1, 16, rng.standard_normal(2), 0, 0),  # unmasked
    ]
    res = {}
    for i, c in enumerate(cases):
        out, lse = run(lib, c)
        res[f"out{i}"], res[f"lse{i}"] = out, lse
    np.savez(dest, **res)
    print(f"{len(cases)} cases ok", flush=True)


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
