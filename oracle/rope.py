"""fp64 rotary position embedding with YaRN scaling, NeoX pairing.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only tests/, the
smoke check and the benchmark's CPU-baseline leg may import it.

What it computes ("GPT OSS" model notes, sections 3 and 4.1: Q and K are
rotated with NeoX-style RoPE under YaRN scaling before K is appended to the
cache, with original context 4096, frequency scale 1/RopeScale, beta_fast 32
and beta_slow 1; section 11: the positions come as an explicit array).  The
notes give the form and those parameters, not the formula, so the formula is
the published one:

* RoPE (Su et al., RoFormer): pair i of a head of dimension d (i < d/2) has
  frequency theta_i = base^(-2 i / d); a token at position p turns the pair
  by the angle p * theta_i.  NeoX pairing: element i pairs with element
  i + d/2 (not with 2i+1).
* YaRN (Peng et al., "YaRN: Efficient Context Window Extension of Large
  Language Models", "NTK-by-parts" interpolation and attention scaling),
  in the form that takes beta_fast and beta_slow as arguments, as the notes'
  RoPEEx call does: a pair that turns `beta` times within the original
  context L0 (L0 theta_i / (2 pi) = beta) sits at the fractional pair index
      c(beta) = (d/2) ln(L0 / (2 pi beta)) / ln(base);
  pairs below lo = c(beta_fast) turn more often and keep theta_i, pairs
  above hi = c(beta_slow) are interpolated to theta_i / s, and in between
  the blend is linear in the pair index:
      ramp_i = clamp((i - lo) / (hi - lo), 0, 1),
      f_i = (1 - ramp_i) theta_i + ramp_i theta_i / s.
  The bounds are used as they are, not rounded to whole pairs.  Both q and
  k are multiplied by sqrt(1/t) = 0.1 ln(s) + 1 (1 when s <= 1), so the
  logits carry the paper's temperature.  s = 1 gives plain RoPE.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def correction_index(head_dim: int, base: float, orig_ctx: float, turns: float) -> float:
    """Fractional pair index whose pair turns `turns` times within orig_ctx."""
    return (head_dim / 2.0) * math.log(orig_ctx / (2.0 * math.pi * turns)) / math.log(base)


def yarn_frequencies(head_dim: int, base: float, scale: float, orig_ctx: int,
                     beta_fast: float, beta_slow: float) -> np.ndarray:
    """Per-pair angular frequencies [head_dim / 2] in fp64."""
    half = head_dim // 2
    theta = np.array([base ** (-2.0 * i / head_dim) for i in range(half)], dtype=np.float64)
    if scale == 1.0:
        return theta
    lo = correction_index(head_dim, base, orig_ctx, beta_fast)
    hi = correction_index(head_dim, base, orig_ctx, beta_slow)
    ramp = np.clip((np.arange(half, dtype=np.float64) - lo) / (hi - lo), 0.0, 1.0)
    return (1.0 - ramp) * theta + ramp * theta / scale


def yarn_mscale(scale: float) -> float:
    """The factor on q and k (the square root of YaRN's 1/t)."""
    return 1.0 if scale <= 1.0 else 0.1 * math.log(scale) + 1.0


def rope(x, positions, freqs: np.ndarray, mscale: float) -> np.ndarray:
    """Rotate x [T][H][d] (any real dtype, taken to fp64) at positions [T]."""
    x = np.asarray(x.double() if isinstance(x, torch.Tensor) else x, dtype=np.float64)
    pos = np.asarray(positions.tolist() if isinstance(positions, torch.Tensor) else positions,
                     dtype=np.float64)
    half = x.shape[-1] // 2
    ang = pos[:, None] * freqs[None, :]           # [T][half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1) * mscale


def rope_append(batch, q, k_new, v_new, positions, base: float, scale: float, orig_ctx: int,
                beta_fast: float, beta_slow: float):
    """The fused step: q and the new K rotated (fp64), then the rotated K --
    rounded to the cache dtype -- and V appended as ``append_kv`` does.
    Returns (q_rot fp64 [T][Hq][d], k_rot fp64 [T][Hkv][d], k_cache, v_cache)."""
    from . import append_kv
    freqs = yarn_frequencies(batch.head_dim, base, scale, orig_ctx, beta_fast, beta_slow)
    ms = yarn_mscale(scale)
    q_rot = rope(q, positions, freqs, ms)
    k_rot = rope(k_new, positions, freqs, ms)
    k_cache, v_cache = append_kv(batch, torch.from_numpy(k_rot).to(batch.k_cache.dtype), v_new)
    return q_rot, k_rot, k_cache, v_cache
