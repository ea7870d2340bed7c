"""The shared random rotation Pi (fp64).

[Ablation] "Configurazione Sperimentale": the TurboQuant family rotates with
a randomized Walsh-Hadamard transform (a random sign flip D, then the
Hadamard transform), which spreads each token's energy evenly over the
coordinates.  [FibQuant] "1. Enunciato del Problema" and "2.1 La Sorgente
Canonica" describe the same slot as a shared Haar rotation; [TurboQuant-es]
"La mecánica geométrica de TurboQuant" as a random rotation Pi.

Readings used here:
* Pi u = H_d (D * u) / sqrt(d): the sign flip first, then the Hadamard
  matrix in natural (Sylvester) order, scaled to be orthogonal; the inverse
  is Pi^T w = D * (H_d^T w) / sqrt(d).
* One D per codec instance, shared by every vector it encodes.
* d = 1536 is not a power of two; there H = H_12 (x) H_128 (Kronecker
  product), with H_12 from Paley's first construction at q = 11.  Index
  i = 128 a + c (a the 128-chunk, c inside it): the order-128 transform runs
  inside each chunk, then the order-12 transform mixes the chunks.
* The Haar variant (QR of a Gaussian matrix) serves the statistical pins,
  whose closed forms hold exactly only under a Haar rotation.
"""

import numpy as np


def hadamard_sylvester(d):
    """Sylvester-ordered Hadamard matrix, H[i, j] = (-1)^popcount(i & j)."""
    if d < 1 or d & (d - 1):
        raise ValueError("Sylvester order must be a power of two")
    i = np.arange(d, dtype=np.int64)
    parity = np.zeros((d, d), dtype=np.int64)
    a = i[:, None] & i[None, :]
    while np.any(a):
        parity ^= a & 1
        a = a >> 1
    return np.where(parity == 1, -1.0, 1.0)


def paley_hadamard_12():
    """Hadamard matrix of order 12 by Paley's first construction, q = 11.

    chi is the quadratic character mod 11, Q[i, j] = chi(j - i) the
    Jacobsthal matrix (antisymmetric since 11 = 3 mod 4), and
    H = I + [[0, 1^T], [-1, Q]]."""
    q = 11
    residues = {(x * x) % q for x in range(1, q)}
    chi = np.array([0] + [1 if a in residues else -1 for a in range(1, q)],
                   dtype=np.int64)
    idx = np.arange(q)
    jac = chi[(idx[None, :] - idx[:, None]) % q]
    s = np.zeros((q + 1, q + 1), dtype=np.int64)
    s[0, 1:] = 1
    s[1:, 0] = -1
    s[1:, 1:] = jac
    return (np.eye(q + 1, dtype=np.int64) + s).astype(np.float64)


def hadamard_matrix(d):
    """H_d: Sylvester order for powers of two, H_12 (x) H_{d/12} when d is 12
    times a power of two (d = 1536 gives H_12 (x) H_128)."""
    if d & (d - 1) == 0:
        return hadamard_sylvester(d)
    if d % 12 == 0 and (d // 12) & (d // 12 - 1) == 0:
        return np.kron(paley_hadamard_12(), hadamard_sylvester(d // 12))
    raise ValueError("no Hadamard order for d=%d" % d)


_H_CACHE = {}


def _h(d):
    if d not in _H_CACHE:
        _H_CACHE[d] = hadamard_matrix(d)
    return _H_CACHE[d]


def _sign_vector(signs, d):
    s = np.asarray(signs)
    if s.shape != (d,):
        raise ValueError("sign vector must have d entries")
    if s.dtype == np.bool_:
        return np.where(s, -1.0, 1.0)  # True marks a flipped coordinate
    s = s.astype(np.float64)
    if not np.all(np.abs(s) == 1.0):
        raise ValueError("sign vector entries must be +1 or -1")
    return s


def rotate(u, signs):
    """Pi u for each row of u: z = H_d (D * u) / sqrt(d)."""
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    dvec = _sign_vector(signs, d)
    return (u * dvec) @ _h(d).T / np.sqrt(d)


def rotate_inverse(w, signs):
    """Pi^T w for each row of w: D * (H_d^T w) / sqrt(d)."""
    w = np.asarray(w, dtype=np.float64)
    d = w.shape[-1]
    dvec = _sign_vector(signs, d)
    return (w @ _h(d)) * dvec / np.sqrt(d)


def haar_rotation(d, rng):
    """A Haar-distributed orthogonal matrix: QR of an i.i.d. Gaussian matrix
    with the column signs of Q fixed by the signs of diag(R)."""
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]
