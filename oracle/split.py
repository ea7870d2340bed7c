"""Outlier-channel split: rates between whole bits (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[TurboQuant-es] "Desempeño teórico y empírico": for rates between whole bits the
outlier channels of a vector get more bits (e.g. 3) and the other channels
fewer (e.g. 2), for effective rates such as 2.5 or 3.5 bits per channel.
[TurboQuant-pl] "Co to oznacza w praktyce?" reports the 3.5-bit point as
quality-neutral on a long-context retrieval test.

Readings where the pages are silent:
* The split is two codec instances over a channel partition: the outlier
  channels form one vector, the others a second, and each is coded on its
  own (its own norm, rotation, table and, for keys, S and gamma).  An inner
  product splits over the partition: <q, x> = <q_O, x_O> + <q_R, x_R>, so the
  key estimate is the sum of the two halves' estimates; attention softmaxes
  that sum.
* The outlier set of a KV head: the d_hi channels of largest mean square
  over a calibration sample of that head's vectors, ties to the lower
  channel index.  The channel order used by the codec puts the outlier
  channels first, each group in ascending channel order
  (`outlier_permutation`); a deployment applies it once to the projection
  weights that produce K, V and q, so a permuted row is coded positionally:
  channels [0, d_hi) with `hi`, the rest with `lo`.
* Effective rate: (d_hi b_hi + d_lo b_lo) / d bits per channel, where b is
  a half's total bits per coordinate (prod: b - 1 table bits + 1 QJL bit);
  the 2.5 and 3.5 points are d_hi = d / 2 with (b_hi, b_lo) = (3, 2) and
  (4, 3).  The two norms (and two gammas for keys) are stored in fp32 like
  the single codec's.
"""

import numpy as np

from .codec import (decode_mse, decode_prod, encode_mse, encode_prod,
                    estimate_ip)


def outlier_permutation(calib, d_hi):
    """Channel order with the d_hi largest-mean-square channels of `calib`
    (n x d) first, each group ascending; ties go to the lower channel."""
    calib = np.asarray(calib, dtype=np.float64)
    ms = np.mean(calib * calib, axis=0)
    order = np.lexsort((np.arange(ms.size), -ms))     # by -ms, then by index
    top = np.sort(order[:d_hi])
    rest = np.sort(order[d_hi:])
    return np.concatenate([top, rest])


def effective_rate(d_hi, b_hi, d_lo, b_lo):
    return (d_hi * b_hi + d_lo * b_lo) / float(d_hi + d_lo)


def _halves(x, d_hi):
    x = np.asarray(x, dtype=np.float64)
    return x[:, :d_hi], x[:, d_hi:]


def encode_split_mse(x, d_hi, hi, lo):
    """hi / lo: dicts with "signs" and "thresholds" of each half's codec.
    Returns the two EncodedMSE."""
    a, b = _halves(x, d_hi)
    return (encode_mse(a, hi["signs"], hi["thresholds"]),
            encode_mse(b, lo["signs"], lo["thresholds"]))


def encode_split_prod(x, d_hi, hi, lo):
    """hi / lo: dicts with "signs", "centroids", "thresholds" and "S".
    Returns the two EncodedProd."""
    a, b = _halves(x, d_hi)
    return (encode_prod(a, hi["signs"], hi["centroids"], hi["thresholds"], hi["S"]),
            encode_prod(b, lo["signs"], lo["centroids"], lo["thresholds"], lo["S"]))


def decode_split(enc, hi, lo):
    """Concatenated decodes of the two halves (mse or prod by the type of
    the encoded halves)."""
    out = []
    for e, c in zip(enc, (hi, lo)):
        if hasattr(e, "sign"):
            out.append(decode_prod(e.idx, e.sign, e.norm, e.rnorm, c["signs"], c["centroids"],
                                   c["S"]))
        else:
            out.append(decode_mse(e.idx, e.norm, c["signs"], c["centroids"]))
    return np.concatenate(out, axis=1)


def estimate_split(q, enc, d_hi, hi, lo):
    """Estimated inner products of the rows of q with the encoded rows: the
    sum of the halves' estimates, q (n_q x d) -> (n_q x n)."""
    q = np.asarray(q, dtype=np.float64)
    parts = []
    for e, c, qq in zip(enc, (hi, lo), (q[:, :d_hi], q[:, d_hi:])):
        if hasattr(e, "sign"):
            parts.append(estimate_ip(qq, e.idx, e.norm, c["signs"], c["centroids"], sign=e.sign,
                                     rnorm=e.rnorm, S=c["S"]))
        else:
            parts.append(estimate_ip(qq, e.idx, e.norm, c["signs"], c["centroids"]))
    return parts[0] + parts[1]


def attention_split(q, kenc, venc, d_hi, khi, klo, vhi, vlo, scale=None):
    """softmax(scale * estimate_split(q, K)) @ decode_split(V), q: n_q x d."""
    q = np.asarray(q, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    s = scale * estimate_split(q, kenc, d_hi, khi, klo)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ decode_split(venc, vhi, vlo)
