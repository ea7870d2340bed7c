"""Six synthetic statistical regimes for the codec's statistical validation.

"Riepilogo Tecnico: Ablazione, Inferenza Statistica e Validazione",
"Metodologia": controlled regimes that isolate one structural assumption
each (distribution shape, K/V subspace alignment, eigenvalue decay).  The
pages name the axes, not the constructions; these are this project's:

  isotropic         K, V, q i.i.d. N(0, 1)
  heavy_tailed      K, V, q i.i.d. Student-t(3) / sqrt(3)
  shared_subspace   K = Z_K A^T + 0.05 E, V = Z_V A^T + 0.05 E: one rank-8
                    basis A (orthonormal columns) for K and V
  split_subspace    as above with independent rank-8 bases for K and V
  fast_decay        Gaussian rows with covariance eigenvalues i^-2 in a
                    random orthonormal basis (K and V share the basis)
  slow_decay        the same with eigenvalues i^-0.5

Queries follow the key distribution (scores carry the keys' structure).
Every regime is scaled to unit average energy per coordinate.
Each draw returns K, V [n, d] and q [n_q, d] as fp16 (the GPU's input type;
the oracle reads the same rounded values).  The codec's own draws (D, S)
come from `codec_draws` with a generator of the caller's choice: the
statistical tests draw them from PCG64 on the oracle side and from MT19937
on the GPU side.

This module only draws random arrays; it holds none of the codec's
arithmetic.
"""

import numpy as np

REGIMES = ("isotropic", "heavy_tailed", "shared_subspace", "split_subspace", "fast_decay",
           "slow_decay")


def _basis(rng, d, r):
    q, _ = np.linalg.qr(rng.standard_normal((d, r)))
    return q


def draw(regime, rng, n=512, d=128, n_q=4, rank=8, noise=0.05):
    """One draw of (K, V, q) for `regime` from generator `rng`."""
    if regime == "isotropic":
        k, v, q = (rng.standard_normal((m, d)) for m in (n, n, n_q))
    elif regime == "heavy_tailed":
        # Student-t(3) has variance 3
        k, v, q = (rng.standard_t(3, (m, d)) / np.sqrt(3.0) for m in (n, n, n_q))
    elif regime in ("shared_subspace", "split_subspace"):
        a = _basis(rng, d, rank)
        b = a if regime == "shared_subspace" else _basis(rng, d, rank)
        k = rng.standard_normal((n, rank)) @ a.T + noise * rng.standard_normal((n, d))
        v = rng.standard_normal((n, rank)) @ b.T + noise * rng.standard_normal((n, d))
        q = rng.standard_normal((n_q, rank)) @ a.T + noise * rng.standard_normal((n_q, d))
        # unit average energy per coordinate, like the other regimes
        scale = 1.0 / np.sqrt(rank / d + noise ** 2)
        k, v, q = k * scale, v * scale, q * scale
    elif regime in ("fast_decay", "slow_decay"):
        alpha = 2.0 if regime == "fast_decay" else 0.5
        u = _basis(rng, d, d)
        sd = np.arange(1, d + 1, dtype=np.float64) ** (-alpha / 2.0)
        k, v, q = ((rng.standard_normal((m, d)) * sd) @ u.T for m in (n, n, n_q))
        # unit average energy per coordinate, like the other regimes
        scale = np.sqrt(d / np.sum(sd ** 2))
        k, v, q = k * scale, v * scale, q * scale
    else:
        raise ValueError("unknown regime %r" % regime)
    return tuple(np.asarray(x, dtype=np.float16) for x in (k, v, q))
