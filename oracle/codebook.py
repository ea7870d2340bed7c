"""Coordinate density and the scalar Lloyd-Max codebook (fp64, offline).

[TurboQuant-es] "La mecánica geométrica de TurboQuant": after a random
rotation each coordinate of a unit vector follows a concentrated Beta law, and
the codec uses, per bit width b, the scalar quantizer that minimises the MSE
cost C(f_X, b), solved once offline and stored.  [FibQuant] "2.1 La Sorgente
Canonica" gives the same law as the k = 1 case of the spherical-Beta source.
[TurboQuant-pl] "Magia losowej rotacji" restates both points.

The density of one coordinate of a uniform point on the sphere S^{d-1} is

    f_d(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - x^2)^((d-3)/2),
    x in [-1, 1].

Reading of the cost as printed: its outer cells use the undefined c_0 and
c_{2^b+1}; here the outer cells extend to the ends of the support, -1 and +1,
where the density vanishes (it is zero outside).

Integrals are taken with the oracle's own composite Gauss-Legendre rule (the
node/weight routine of numpy is the only library primitive used).
"""

import math

import numpy as np

_GL_NODES = 24
_GL_PANELS = 96


def beta_coord_pdf(x, d):
    """f_d(x) for x in [-1, 1] (zero outside).  [TurboQuant-es] "La mecánica
    geométrica de TurboQuant" (Beta law of a rotated coordinate)."""
    x = np.asarray(x, dtype=np.float64)
    if d < 2:
        raise ValueError("d must be >= 2")
    log_c = math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0)
    alpha = (d - 3) / 2.0
    inside = np.abs(x) < 1.0
    out = np.zeros_like(x)
    xi = x[inside]
    out[inside] = np.exp(log_c + alpha * np.log1p(-xi * xi))
    if alpha == 0.0:  # d = 3: uniform density, endpoints included
        out[np.abs(x) == 1.0] = math.exp(log_c)
    return out


def cell_moments(edges, d):
    """For each cell [edges[k], edges[k+1]]: the integrals of f_d, x f_d and
    x^2 f_d (zeroth, first and second moments)."""
    edges = np.asarray(edges, dtype=np.float64)
    xg, wg = np.polynomial.legendre.leggauss(_GL_NODES)
    frac = np.linspace(0.0, 1.0, _GL_PANELS + 1)
    lo = edges[:-1, None] + (edges[1:] - edges[:-1])[:, None] * frac[None, :-1]
    hi = edges[:-1, None] + (edges[1:] - edges[:-1])[:, None] * frac[None, 1:]
    half = 0.5 * (hi - lo)
    mid = 0.5 * (hi + lo)
    nodes = mid[:, :, None] + half[:, :, None] * xg[None, None, :]
    f = beta_coord_pdf(nodes, d) * (half[:, :, None] * wg[None, None, :])
    m0 = f.sum(axis=(1, 2))
    m1 = (nodes * f).sum(axis=(1, 2))
    m2 = (nodes * nodes * f).sum(axis=(1, 2))
    return m0, m1, m2


def _thresholds(c):
    """Decision thresholds of a nearest-centroid quantizer: the midpoints of
    neighbouring centroids (the cell limits of C(f_X, b))."""
    return 0.5 * (c[:-1] + c[1:])


def lloyd_max(d, bits, tol=1e-15, max_iter=200000):
    """Lloyd-Max iteration for f_d at `bits` bits.

    [TurboQuant-es] "La mecánica geométrica de TurboQuant": minimise
    C(f_X, b) over sorted centroids in [-1, 1].  The two optimality
    conditions are iterated alternately: thresholds at the midpoints of
    neighbouring centroids, then each centroid at the conditional mean of its
    cell.  Stops when no centroid moves by more than `tol`.

    Returns (centroids, thresholds, iterations), fp64, centroids ascending.
    """
    if bits < 1:
        raise ValueError("bits must be >= 1")
    n = 1 << bits
    sigma = 1.0 / math.sqrt(d)
    span = min(0.9, 2.5 * sigma)
    c = np.linspace(-span, span, n)
    for it in range(1, max_iter + 1):
        t = _thresholds(c)
        edges = np.concatenate(([-1.0], t, [1.0]))
        m0, m1, _ = cell_moments(edges, d)
        c_new = m1 / m0
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step <= tol:
            # f_d is even, so the optimum is symmetric (c_k = -c_{N-1-k});
            # symmetrising removes the rounding noise, which puts the middle
            # threshold exactly at 0.
            c = 0.5 * (c - c[::-1])
            return c, _thresholds(c), it
    raise RuntimeError("Lloyd-Max did not converge (d=%d, bits=%d)" % (d, bits))


_CACHE = {}


def codebook(d, bits):
    """Cached (centroids, thresholds) of `lloyd_max`: the codebook is solved
    once per (d, bit width) and then reused ([TurboQuant-es] "La mecánica
    geométrica de TurboQuant")."""
    key = (int(d), int(bits))
    if key not in _CACHE:
        c, t, _ = lloyd_max(d, bits)
        _CACHE[key] = (c, t)
    c, t = _CACHE[key]
    return c.copy(), t.copy()


def distortion(d, centroids):
    """Normalised MSE distortion D = d * E[(X - Q(X))^2], X ~ f_d, for the
    nearest-centroid quantizer with these centroids (cells split at the
    midpoints, outer cells to the support ends)."""
    c = np.asarray(centroids, dtype=np.float64)
    edges = np.concatenate(([-1.0], _thresholds(c), [1.0]))
    m0, m1, m2 = cell_moments(edges, d)
    return float(d * np.sum(m2 - 2.0 * c * m1 + c * c * m0))
