"""Pins of the RoPE / YaRN oracle (oracle/rope.py), and planted mistakes.

"GPT OSS" model notes, sections 3 and 4.1: Q and K are rotated with
NeoX-style RoPE under YaRN scaling (original context 4096, beta_fast 32,
beta_slow 1) before K is appended to the cache.  The pins check the oracle
against what the mathematics fixes rather than against a retyped copy of it:

* with scale 1 the rotation is complex multiplication of the NeoX pairs
  (x_i + i x_{i+d/2}) by exp(i p theta_i), theta_i = base^(-2i/d);
* position 0 is the identity (times YaRN's factor on q and k);
* each pair keeps its norm, times 0.1 ln(s) + 1;
* the dot product of a rotated q and k depends only on their position gap;
* YaRN keeps the frequency of pairs that turn more than beta_fast times in
  the original context, divides by s those that turn fewer than beta_slow
  times, and blends monotonically in between; the rotation applies exactly
  those frequencies;
* inside the blend, the frequencies of a hand-worked case
  (tests/golden/yarn_ramp.json) and a blend weight that is affine in the
  pair index (its second differences vanish);
* the fused append writes V as the plain append does and K rotated.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import rope as R
from gqa_paged_attention_amd import workloads as wl

BASE, ORIG, BF, BS = 10000.0, 4096, 32.0, 1.0


def _x(seed, T, H, d):
    return np.random.default_rng(seed).standard_normal((T, H, d))


def pin_complex_form(impl):
    d, T, H = 16, 7, 3
    x = _x(1, T, H, d)
    pos = np.array([0, 1, 2, 17, 4095, 65536, 131071], dtype=np.int64)
    got = impl.rope(x, pos, impl.yarn_frequencies(d, BASE, 1.0, ORIG, BF, BS),
                    impl.yarn_mscale(1.0))
    h = d // 2
    theta = np.power(BASE, -np.arange(h) * 2.0 / d)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    want = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def pin_identity_at_zero(impl):
    d, s = 64, 32.0
    x = _x(2, 4, 5, d)
    got = impl.rope(x, np.zeros(4, np.int64), impl.yarn_frequencies(d, BASE, s, ORIG, BF, BS),
                    impl.yarn_mscale(s))
    np.testing.assert_allclose(got, x * (0.1 * math.log(s) + 1.0), rtol=1e-13, atol=0)


def pin_norms(impl):
    d, s = 64, 32.0
    x = _x(3, 6, 2, d)
    pos = np.array([1, 9, 100, 5000, 70000, 131071])
    y = impl.rope(x, pos, impl.yarn_frequencies(d, BASE, s, ORIG, BF, BS), impl.yarn_mscale(s))
    h = d // 2
    nx = np.hypot(x[..., :h], x[..., h:])
    ny = np.hypot(y[..., :h], y[..., h:])
    np.testing.assert_allclose(ny, nx * (0.1 * math.log(s) + 1.0), rtol=1e-12)


def pin_relative_position(impl):
    d, s = 64, 32.0
    f = impl.yarn_frequencies(d, BASE, s, ORIG, BF, BS)
    ms = impl.yarn_mscale(s)
    q, k = _x(4, 1, 1, d), _x(5, 1, 1, d)
    for p, n in [(10, 3), (5000, 4999), (100000, 2)]:
        dots = []
        for shift in (0, 1, 777, 20000):
            qa = impl.rope(q, [p + shift], f, ms)
            ka = impl.rope(k, [n + shift], f, ms)
            dots.append(float((qa * ka).sum()))
        np.testing.assert_allclose(dots, dots[0], rtol=1e-9, atol=1e-9)


def pin_yarn_regions(impl):
    d, s = 64, 32.0
    f = impl.yarn_frequencies(d, BASE, s, ORIG, BF, BS)
    theta = np.power(BASE, -np.arange(d // 2) * 2.0 / d)
    turns = ORIG * theta / (2 * math.pi)  # rotations within the original context
    fast, slow = turns > BF, turns < BS
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    np.testing.assert_allclose(f[fast], theta[fast], rtol=1e-14)
    np.testing.assert_allclose(f[slow], theta[slow] / s, rtol=1e-14)
    ratio = f / theta
    mid = ~fast & ~slow
    assert np.all((ratio[mid] > 1 / s) & (ratio[mid] < 1)), ratio[mid]
    assert np.all(np.diff(ratio) <= 1e-15), "the blend must fall from fast to slow pairs"
    # the rotation turns basis vector e_i by exactly f_i at position 1
    ms = impl.yarn_mscale(s)
    for i in (0, 5, 12, 20, 31):
        e = np.zeros((1, 1, d))
        e[0, 0, i] = 1.0
        y = impl.rope(e, [1], f, ms)[0, 0] / ms
        assert math.isclose(math.atan2(y[i + d // 2], y[i]), f[i], rel_tol=1e-12)


def pin_fused_append(impl):
    full = wl.small_batch(41, "bf16", [40, 5, 17], [7, 5, 1], 8, 2, 64, sink_mode="normal")
    before, k_new, v_new = wl.split_new_tokens(full)
    q = full.q
    pos = torch.tensor([3, 100, 7, 8, 9, 4095, 0, 1, 2, 131071, 12, 13, 16], dtype=torch.int32)
    q_rot, k_rot, kc, vc = impl.rope_append(before, q, k_new, v_new, pos, BASE, 32.0, ORIG, BF,
                                            BS)
    f = impl.yarn_frequencies(64, BASE, 32.0, ORIG, BF, BS)
    ms = impl.yarn_mscale(32.0)
    np.testing.assert_allclose(q_rot, impl.rope(q, pos, f, ms), rtol=0, atol=0)
    kc2, vc2 = oracle.append_kv(before, torch.from_numpy(impl.rope(k_new, pos, f, ms)).to(
        torch.bfloat16), v_new)
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    _, vplain = oracle.append_kv(before, k_new, v_new)
    assert torch.equal(vc.view(torch.int16), vplain.view(torch.int16))


GOLDEN_YARN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "yarn_ramp.json")


def pin_yarn_golden(impl):
    g = json.load(open(GOLDEN_YARN))
    p = g["params"]
    f = impl.yarn_frequencies(p["head_dim"], p["base"], p["scale"], p["orig_ctx"],
                              p["beta_fast"], p["beta_slow"])
    for i, want in g["frequencies"].items():
        assert math.isclose(f[int(i)], want, rel_tol=g["tolerance_rel"]), (i, f[int(i)], want)


def pin_yarn_ramp_affine(impl):
    # the blend weight w_i = (1 - f_i / theta_i) / (1 - 1/s) of the pairs
    # strictly inside the blend is affine in i, at several bases and heads
    for d, base, s, ctx in ((64, BASE, 32.0, ORIG), (128, 500000.0, 8.0, 8192),
                            (64, 150000.0, 32.0, ORIG)):
        f = impl.yarn_frequencies(d, base, s, ctx, BF, BS)
        theta = np.power(base, -np.arange(d // 2) * 2.0 / d)
        w = (1.0 - f / theta) / (1.0 - 1.0 / s)
        inner = np.nonzero((w > 1e-12) & (w < 1 - 1e-12))[0]
        assert len(inner) >= 4, (d, base, inner)
        assert np.all(np.diff(inner) == 1)
        np.testing.assert_allclose(np.diff(w[inner], 2), 0.0, atol=1e-12)


PINS = [pin_complex_form, pin_identity_at_zero, pin_norms, pin_relative_position,
        pin_yarn_regions, pin_yarn_golden, pin_yarn_ramp_affine, pin_fused_append]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_rope_oracle_pin(pin):
    pin(R)


def test_scale_one_is_plain_rope():
    f = R.yarn_frequencies(128, 500000.0, 1.0, ORIG, BF, BS)
    np.testing.assert_allclose(f, np.power(500000.0, -np.arange(64) * 2.0 / 128), rtol=1e-15)
    assert R.yarn_mscale(1.0) == 1.0


MUTANTS = {
    "GPT-J pairing": ("x1, x2 = x[..., :half], x[..., half:]",
                      "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    "rotation turned the other way": ("x1 * c - x2 * s, x1 * s + x2 * c",
                                      "x1 * c + x2 * s, x2 * c - x1 * s"),
    "ramp reversed": ("(1.0 - ramp) * theta + ramp * theta / scale",
                      "ramp * theta + (1.0 - ramp) * theta / scale"),
    "ramp bounds swapped": ("(np.arange(half, dtype=np.float64) - lo) / (hi - lo)",
                            "(np.arange(half, dtype=np.float64) - hi) / (lo - hi)"),
    "ramp linear in the pair's turns, not its index": (
        "np.clip((np.arange(half, dtype=np.float64) - lo) / (hi - lo), 0.0, 1.0)",
        "1.0 - np.clip((orig_ctx * theta / (2.0 * math.pi) - beta_slow) / "
        "(beta_fast - beta_slow), 0.0, 1.0)"),
    "correction bounds rounded outward to whole pairs": (
        "ramp = np.clip((np.arange(half, dtype=np.float64) - lo)",
        "lo, hi = math.floor(lo), math.ceil(hi)\n"
        "    ramp = np.clip((np.arange(half, dtype=np.float64) - lo)"),
    "correction index without the factor d/2": (
        "return (head_dim / 2.0) * math.log(", "return math.log("),
    "YaRN factor dropped": ("axis=-1) * mscale", "axis=-1)"),
    "frequency exponent halved": ("base ** (-2.0 * i / head_dim)", "base ** (-1.0 * i / head_dim)"),
    "positions off by one": ("ang = pos[:, None] * freqs[None, :]",
                             "ang = (pos[:, None] + 1) * freqs[None, :]"),
    "slow pairs not interpolated": ("ramp * theta / scale", "ramp * theta"),
}


def _mutant(old, new):
    src = open(R.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle.rope_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "rope_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_rope_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin rejects the mutant '{name}'"
