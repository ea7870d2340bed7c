"""TurboQuant encode / decode / inner-product estimate (fp64).

Follows:
* [FibQuant] "1. Enunciato del Problema" and "2.3 Codifica e Decodifica":
  the normalize-rotate-quantize interface (store the norm, rotate the unit
  vector with the shared rotation, quantize each rotated coordinate with the
  scalar table; decode looks the centroids up, rotates back and rescales by
  the norm), with every vector's code at a fixed address.
* [TurboQuant-es] "La mecánica geométrica de TurboQuant" (the scalar
  Lloyd-Max table) and "Eliminación del sesgo interno del producto"
  (TurboQuant_prod: the mse quantizer at b-1 bits, then a 1-bit quantized
  Johnson-Lindenstrauss sketch of the residual, for an unbiased inner-product
  estimate).  [TurboQuant-pl] "Błąd średniokwadratowy to pułapka" restates
  the two stages.

Readings where the pages are silent:
* The residual lives in the rotated, unit-normalised domain:
  r = Pi(x / |x|) - c[idx].  Its norm gamma = |r| is stored per vector in
  addition to the norm nu = |x| (the unbiased estimate needs it).
* The QJL matrix S is m x d with i.i.d. N(0, 1) entries and m = d; the sign
  bit of row i is 1 when (S r)_i >= 0, else 0 (sign(0) = +1).
* The estimate of <q, x> reads
      nu * ( <Pi q, c[idx]> + sqrt(pi/2)/m * gamma * <S Pi q, 2 sigma - 1> ),
  since E[sign(<g, r>) <g, y>] = sqrt(2/pi) <r, y> / |r| for g ~ N(0, I).
* A code is the number of thresholds at or below the coordinate,
  idx = #{k : z >= t_k} (a value on a threshold goes to the upper cell).
* The zero vector encodes as u = 0: idx = #{k : 0 >= t_k}, r = -c[idx],
  and its estimate is 0 because nu = 0.  A row with an inf or NaN element
  gets the same codes and keeps its non-finite norm.
* Packing: a row's codes form one LSB-first bit stream, code i in stream
  bits [i b, (i+1) b), stream bit k = bit (k mod 8) of byte k // 8; a row
  occupies exactly d b / 8 bytes, row j at byte j d b / 8 (fixed rate, fixed
  address).  Sign bits use the same LSB-first order, m / 8 bytes per row.
"""

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .rotation import rotate, rotate_inverse


def qjl_factor(m):
    """sqrt(pi/2) / m, the scale that makes the 1-bit sketch unbiased."""
    return math.sqrt(math.pi / 2.0) / m


@dataclass
class EncodedMSE:
    idx: np.ndarray      # (n, d) integer codes
    norm: np.ndarray     # (n,) nu = |x|
    z: Optional[np.ndarray] = None   # (n, d) rotated unit vectors, for band checks


@dataclass
class EncodedProd:
    idx: np.ndarray      # (n, d) integer codes at b - 1 bits
    sign: np.ndarray     # (n, m) 0/1 sign bits of S r
    norm: np.ndarray     # (n,) nu
    rnorm: np.ndarray    # (n,) gamma = |r|
    z: Optional[np.ndarray] = None   # (n, d)
    p: Optional[np.ndarray] = None   # (n, m) S r, for band checks


def _as_rows(x):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("expected an (n, d) array")
    return x


def _normalize_rotate(x, signs):
    """nu = |x| and z = Pi (x / nu), with u = 0 for the zero vector.

    A row holding an inf or NaN has no unit vector; the pages define no code
    for it.  Here it also takes u = 0 (the zero vector's codes) and keeps its
    non-finite norm: inf when its largest element is infinite, NaN when an
    element is NaN (the sum of squares computed as written)."""
    with np.errstate(over="ignore", invalid="ignore"):
        nu = np.sqrt(np.sum(x * x, axis=1))
    live = np.all(np.isfinite(x), axis=1) & (nu > 0)
    u = np.zeros_like(x)
    u[live] = x[live] / nu[live, None]
    return nu, rotate(u, signs)


def _quantize(z, thresholds):
    t = np.asarray(thresholds, dtype=np.float64)
    return np.sum(z[..., None] >= t, axis=-1).astype(np.int64)


def encode_mse(x, signs, thresholds, keep_z=True):
    """TurboQuant_mse encode of each row of x (n, d)."""
    x = _as_rows(x)
    nu, z = _normalize_rotate(x, signs)
    idx = _quantize(z, thresholds)
    return EncodedMSE(idx=idx, norm=nu, z=z if keep_z else None)


def qjl_projection(r, S):
    """p = S r for each row r: p_i = sum_k S[i, k] r_k."""
    return np.asarray(r, dtype=np.float64) @ np.asarray(S, dtype=np.float64).T


def encode_prod(x, signs, centroids, thresholds, S, keep_z=True):
    """TurboQuant_prod encode: the mse codes at the given (b - 1)-bit table,
    then the residual norm and the QJL sign bits of the residual."""
    x = _as_rows(x)
    c = np.asarray(centroids, dtype=np.float64)
    nu, z = _normalize_rotate(x, signs)
    idx = _quantize(z, thresholds)
    r = z - c[idx]
    gamma = np.sqrt(np.sum(r * r, axis=1))
    p = qjl_projection(r, S)
    sign = (p >= 0.0).astype(np.uint8)
    return EncodedProd(idx=idx, sign=sign, norm=nu, rnorm=gamma,
                       z=z if keep_z else None, p=p if keep_z else None)


def residual_from_codes(z, idx, centroids):
    """r = z - c[idx]: used to re-derive the sign bits from a given set of
    codes (the conditional QJL check)."""
    c = np.asarray(centroids, dtype=np.float64)
    return np.asarray(z, dtype=np.float64) - c[np.asarray(idx)]


def decode_mse(idx, norm, signs, centroids):
    """x_hat = nu * Pi^T c[idx]  ([FibQuant] "2.3 Codifica e Decodifica")."""
    c = np.asarray(centroids, dtype=np.float64)
    return np.asarray(norm, dtype=np.float64)[:, None] * rotate_inverse(c[np.asarray(idx)], signs)


def decode_prod(idx, sign, norm, rnorm, signs, centroids, S):
    """x_hat = nu * Pi^T (c[idx] + sqrt(pi/2)/m * gamma * S^T (2 sigma - 1))."""
    c = np.asarray(centroids, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    m = S.shape[0]
    pm = 2.0 * np.asarray(sign, dtype=np.float64) - 1.0
    w = c[np.asarray(idx)] + qjl_factor(m) * np.asarray(rnorm, dtype=np.float64)[:, None] * (pm @ S)
    return np.asarray(norm, dtype=np.float64)[:, None] * rotate_inverse(w, signs)


def estimate_ip(q, idx, norm, signs, centroids, sign=None, rnorm=None, S=None):
    """Code-domain estimate of <q_a, x_j> for every query row a and code row j.

    mse: nu_j <Pi q_a, c[idx_j]>.  prod (sign, rnorm, S given): adds
    nu_j sqrt(pi/2)/m gamma_j <S Pi q_a, 2 sigma_j - 1>  ([TurboQuant-es]
    "Eliminación del sesgo interno del producto", the unbiased estimator).
    Returns an (n_q, n) fp64 array."""
    q = _as_rows(q)
    c = np.asarray(centroids, dtype=np.float64)
    qr = rotate(q, signs)
    nu = np.asarray(norm, dtype=np.float64)
    est = qr @ c[np.asarray(idx)].T
    if sign is not None:
        S = np.asarray(S, dtype=np.float64)
        m = S.shape[0]
        sq = qr @ S.T
        pm = 2.0 * np.asarray(sign, dtype=np.float64) - 1.0
        est = est + qjl_factor(m) * (sq @ pm.T) * np.asarray(rnorm, dtype=np.float64)[None, :]
    return est * nu[None, :]


def pack_codes(idx, bits):
    """Pack (n, d) codes of `bits` bits into (n, d * bits / 8) bytes, one
    LSB-first bit stream per row."""
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    if (d * bits) % 8:
        raise ValueError("d * bits must be a whole number of bytes")
    if np.any(idx < 0) or np.any(idx >= (1 << bits)):
        raise ValueError("code out of range")
    stream = ((idx[:, :, None] >> np.arange(bits)[None, None, :]) & 1).reshape(n, d * bits)
    return np.packbits(stream.astype(np.uint8), axis=1, bitorder="little")


def unpack_codes(packed, d, bits):
    """Inverse of `pack_codes`."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    stream = np.unpackbits(packed, axis=1, bitorder="little")[:, :d * bits]
    stream = stream.reshape(n, d, bits).astype(np.int64)
    return np.sum(stream << np.arange(bits)[None, None, :], axis=2)


def pack_bits(bits01):
    """Pack (n, m) 0/1 values into (n, m / 8) bytes, LSB first."""
    b = np.asarray(bits01, dtype=np.uint8)
    if b.shape[1] % 8:
        raise ValueError("m must be a multiple of 8")
    return np.packbits(b, axis=1, bitorder="little")


def unpack_bits(packed, m):
    """Inverse of `pack_bits`."""
    return np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=1,
                         bitorder="little")[:, :m]
