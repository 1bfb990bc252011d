"""Partial rotary position embedding (test infrastructure only).

RoPE acts on only the last 64 dimensions of queries and compressed entries,
and RoPE at position -i is applied to the attention output so the result
carries relative positions ([P5] "Two ways to shrink attention, interleaved").

Readings where the pages are silent:
  * pairs are adjacent dims (D-R+2i, D-R+2i+1), i = 0..R/2-1;
  * frequencies theta_i = base^(-2i/R) with base 10000, no long-context
    rescaling (the pages mention none);
  * a pair (x0, x1) at position p becomes
        (x0 cos(p theta_i) - x1 sin(p theta_i),  x0 sin(p theta_i) + x1 cos(p theta_i)).
All angles are formed in float64 from the exact integer position.
"""

import numpy as np


def inv_freq(R, base):
    """theta_i = base^(-2i/R), i = 0..R/2-1, float64."""
    i = np.arange(R // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / R)


def rope(x, pos, R, base):
    """Rotate the last R dims of x [..., D] by position `pos`.

    `pos` is a scalar or an array broadcastable to x.shape[:-1]; negative
    positions rotate backwards (used for the output's inverse rotation)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    pos = np.asarray(pos, dtype=np.float64)[..., None]
    ang = pos * inv_freq(R, base)                 # [..., R/2]
    c, s = np.cos(ang), np.sin(ang)
    y = x.copy()
    x0 = x[..., D - R::2]
    x1 = x[..., D - R + 1::2]
    y[..., D - R::2] = x0 * c - x1 * s
    y[..., D - R + 1::2] = x0 * s + x1 * c
    return y
