"""Rotary position embedding applied before the TurboQuant rotation (fp64).

[TurboESM] "2. Metodologia", part A (pipeline invariant to RoPE): RoPE
R_{theta,i} is applied to keys and queries first and the orthogonal rotation
Pi after it; since Pi^T Pi = I, the rotated inner product equals
q^T R_i^T R_j k, so positional information survives the rotation.

Reading (the pages give no RoPE convention): interleaved pairs
(2i, 2i + 1), theta_i = base^(-2i / d), angle = position * theta_i.
"""

import numpy as np


def rope_interleaved(x, positions, base=10000.0):
    """Rotate each pair (x[..., 2i], x[..., 2i+1]) of every row by
    positions * base^(-2i/d).  x: (..., n, d); positions: (n,)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even dimension")
    pos = np.asarray(positions, dtype=np.float64)
    i = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / d)
    ang = pos[:, None] * theta[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out
