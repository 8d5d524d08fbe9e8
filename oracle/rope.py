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
  Language Models", "NTK-by-parts" interpolation and attention scaling):
  with scale s (= RopeScale), original context L0 and the pair's wavelength
  lambda_i = 2 pi / theta_i, let r_i = L0 / lambda_i and
      gamma(r) = 0 if r < beta_slow,  1 if r > beta_fast,
                 (r - beta_slow) / (beta_fast - beta_slow) otherwise;
  the pair's frequency becomes (1 - gamma) theta_i / s + gamma theta_i
  (slow pairs are interpolated by s, fast pairs kept), and both q and k are
  multiplied by sqrt(1/t) = 0.1 ln(s) + 1 (1 when s <= 1), so the logits
  carry the paper's temperature.  s = 1 gives plain RoPE.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def yarn_frequencies(head_dim: int, base: float, scale: float, orig_ctx: int,
                     beta_fast: float, beta_slow: float) -> np.ndarray:
    """Per-pair angular frequencies [head_dim / 2] in fp64."""
    half = head_dim // 2
    theta = np.array([base ** (-2.0 * i / head_dim) for i in range(half)], dtype=np.float64)
    if scale == 1.0:
        return theta
    r = orig_ctx * theta / (2.0 * math.pi)  # rotations of the pair within L0
    gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return (1.0 - gamma) * theta / scale + gamma * theta


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
