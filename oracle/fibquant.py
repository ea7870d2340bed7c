"""FibQuant at k = 2: a fixed-rate vector code for 2-coordinate blocks of the
rotated unit vector (fp64, offline codebook; encode / decode).

[FibQuant] "2.1 La Sorgente Canonica": after normalisation and rotation,
any block of k consecutive coordinates follows one spherical-Beta density
on the unit k-ball, whatever the input.  For k = 2 (the first two
coordinates of a uniform point on S^{d-1}):

    f_{d,2}(y) = (d - 2) / (2 pi) * (1 - |y|^2)^((d - 4) / 2),  |y| < 1,

so |y|^2 ~ Beta(1, (d - 2) / 2).

[FibQuant] "2.2 Costruzione del Codice", N codewords (rate
b = log2(N) / 2 bits per coordinate, "2.3"):
1. Radii by Bennett-Gersho companding: the point density proportional to
   f^(k/(k+2)) = f^(1/2) for k = 2.  Its mass inside radius r is
   1 - (1 - r^2)^(d/4), so codeword n (n = 0..N-1) sits at the radius
   where that mass is t_n = (n + 1/2) / N:  r_n^2 = 1 - (1 - t_n)^(4/d),
   a quantile of Beta(1, d/4) (the closed form the page mentions).
2. Directions on the planar Fibonacci spiral (golden-angle quantizer):
   theta_n = phase + n * g, g = pi (3 - sqrt 5).
3. Lloyd refinement, multi-restart: the source is assigned to its nearest
   codeword and each codeword moves to the centroid of its cell; the
   spiral is restarted at several phases and the lowest-MSE code is kept.

[FibQuant] "2.3 Codifica e Decodifica": encode = norm, rotate the unit
vector, split it into d/2 blocks, nearest codeword per block; decode =
look the codewords up, concatenate, rotate back, rescale by the norm.  The
block codes are packed like the scalar codes (one LSB-first stream of
log2(N)-bit fields, fixed rate, fixed address).

Readings where the page is silent:
* The rotation is the codec's randomized Walsh-Hadamard Pi (the same
  normalise-rotate interface as the scalar codec); blocks are coordinates
  (2j, 2j + 1).
* Lloyd runs on a fixed equal-probability polar quadrature of f_{d,2}:
  R = 128 rings at the Beta(1, (d-2)/2) quantiles (i + 1/2) / R of |y|^2,
  A = 256 angles 2 pi (j + 1/2) / A, all points of equal weight.
* LLOYD_ITERS = 40 iterations per restart; restarts at phases
  {0, 1/2} * g; a later restart replaces the kept code only when its MSE is
  lower by more than a relative RESTART_MARGIN = 1e-9 (at small N the
  restarts reach rotations of one code whose MSEs differ only by rounding);
  a codeword whose cell is empty stays where it is; ties in the nearest
  search go to the lower index.
"""

import math

import numpy as np

from .codec import pack_codes, unpack_codes
from .rotation import rotate, rotate_inverse

GOLDEN_ANGLE = math.pi * (3.0 - math.sqrt(5.0))
QUAD_RINGS = 128
QUAD_ANGLES = 256
LLOYD_ITERS = 40
RESTART_PHASES = (0.0, 0.5)
RESTART_MARGIN = 1e-9


def block_pdf(y, d):
    """f_{d,2}(y) for points y (..., 2) ([FibQuant] 2.1)."""
    y = np.asarray(y, dtype=np.float64)
    r2 = np.sum(y * y, axis=-1)
    out = np.zeros(r2.shape)
    inside = r2 < 1.0
    out[inside] = (d - 2) / (2.0 * math.pi) * (1.0 - r2[inside]) ** ((d - 4) / 2.0)
    return out


def spiral_init(d, n_codes, phase=0.0):
    """Companded radii on the golden-angle spiral (steps 1 and 2)."""
    n = np.arange(n_codes, dtype=np.float64)
    t = (n + 0.5) / n_codes
    r = np.sqrt(1.0 - (1.0 - t) ** (4.0 / d))
    th = phase * GOLDEN_ANGLE + n * GOLDEN_ANGLE
    return np.stack([r * np.cos(th), r * np.sin(th)], axis=1)


def quadrature(d):
    """Equal-weight points of the source: rings at equal-probability |y|^2."""
    q = (np.arange(QUAD_RINGS, dtype=np.float64) + 0.5) / QUAD_RINGS
    r = np.sqrt(1.0 - (1.0 - q) ** (2.0 / (d - 2)))
    th = 2.0 * math.pi * (np.arange(QUAD_ANGLES, dtype=np.float64) + 0.5) / QUAD_ANGLES
    return np.stack([np.outer(r, np.cos(th)).ravel(), np.outer(r, np.sin(th)).ravel()], axis=1)


def nearest(y, code):
    """Index of the nearest codeword for each row of y (ties: lower index)."""
    y = np.asarray(y, dtype=np.float64)
    d2 = np.sum((y[:, None, :] - code[None, :, :]) ** 2, axis=-1)
    return np.argmin(d2, axis=1)


def block_mse(y, code):
    """Mean of |y - nearest codeword|^2 over the rows of y."""
    a = nearest(y, code)
    return float(np.mean(np.sum((y - code[a]) ** 2, axis=-1)))


def lloyd(code, pts, iters=LLOYD_ITERS):
    """Lloyd iterations on equal-weight points (step 3)."""
    code = np.array(code, dtype=np.float64)
    for _ in range(iters):
        a = nearest(pts, code)
        for n in range(code.shape[0]):
            cell = pts[a == n]
            if len(cell):
                code[n] = cell.mean(axis=0)
    return code


def fibquant_codebook(d, n_codes):
    """The N x 2 codebook for dimension d: the best of the restarts."""
    if n_codes < 2 or n_codes & (n_codes - 1):
        raise ValueError("n_codes must be a power of two >= 2")
    pts = quadrature(d)
    best, best_mse = None, math.inf
    for ph in RESTART_PHASES:
        c = lloyd(spiral_init(d, n_codes, ph), pts)
        m = block_mse(pts, c)
        if m < best_mse * (1.0 - RESTART_MARGIN):
            best, best_mse = c, m
    return best


def code_bits(n_codes):
    return int(round(math.log2(n_codes)))


def encode_vq(x, signs, code):
    """nu = |x|, z = Pi x / nu, idx_j = nearest codeword of (z_2j, z_2j+1)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        nu = np.sqrt(np.sum(x * x, axis=1))
    # the zero row, and a row with an inf or NaN element (which keeps its
    # non-finite norm), take z = 0
    live = np.all(np.isfinite(x), axis=1) & (nu > 0)
    u = np.zeros_like(x)
    u[live] = x[live] / nu[live, None]
    z = rotate(u, signs)
    n, d = z.shape
    idx = nearest(z.reshape(-1, 2), code).reshape(n, d // 2)
    return idx, nu, z


def decode_vq(idx, nu, signs, code):
    """x_hat = nu * Pi^T (concatenated codewords)."""
    idx = np.asarray(idx)
    n, nb = idx.shape
    w = code[idx].reshape(n, 2 * nb)
    return np.asarray(nu, dtype=np.float64)[:, None] * rotate_inverse(w, signs)


def pack_vq(idx, n_codes):
    return pack_codes(idx, code_bits(n_codes))


def unpack_vq(packed, d, n_codes):
    return unpack_codes(packed, d // 2, code_bits(n_codes))
