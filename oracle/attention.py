"""Attention straight from TurboQuant codes (fp64, naive).

[TurboESM] "2. Metodologia", part E (fused kernel): one pass unpacks the
codes, applies the residual correction, undoes the rotation and computes
attention with an online softmax, with no dequantized intermediate.
[FibQuant] "5. Significato e Affermazioni": the fixed-address layout is what
lets decompression fuse into attention kernels.

The oracle does the same arithmetic in the plainest order: for query head h
with KV head g = h // G (G = Hq / Hkv), the score of token j is the
code-domain estimate of <q_h, k_{g,j}> times the scale, the weights are the
max-subtracted softmax over all ctx tokens (no causal mask), and the output
is the weighted sum of the decoded values nu_j Pi^T c_V[idx_j].
"""

import math

import numpy as np

from .codec import estimate_ip, decode_mse, decode_prod


def _softmax_rows(s):
    s = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(s)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_from_codes(q, k_codes, v_codes, k_book, v_book, scale=None,
                         return_scores=False):
    """q: (B, Hq, nq, d).  k_codes: dict idx (B, Hkv, ctx, d), sign
    (B, Hkv, ctx, m), norm, rnorm (B, Hkv, ctx).  v_codes: dict idx, norm.
    k_book: dict signs (d,), centroids, S (m, d); v_book: dict signs,
    centroids.  Returns out (B, Hq, nq, d) [and scores (B, Hq, nq, ctx)]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, nq, d = q.shape
    Hkv = k_codes["idx"].shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ctx = k_codes["idx"].shape[2]
    out = np.zeros((B, Hq, nq, d))
    scores = np.zeros((B, Hq, nq, ctx)) if return_scores else None
    for b in range(B):
        for g in range(Hkv):
            vhat = decode_mse(v_codes["idx"][b, g], v_codes["norm"][b, g],
                              v_book["signs"], v_book["centroids"])
            for h in range(g * G, (g + 1) * G):
                s = estimate_ip(q[b, h], k_codes["idx"][b, g], k_codes["norm"][b, g],
                                k_book["signs"], k_book["centroids"],
                                sign=k_codes["sign"][b, g], rnorm=k_codes["rnorm"][b, g],
                                S=k_book["S"]) * scale
                if return_scores:
                    scores[b, h] = s
                out[b, h] = _softmax_rows(s) @ vhat
    if return_scores:
        return out, scores
    return out


def attention_materialized(q, k_codes, v_codes, k_book, v_book, scale=None):
    """Two-pass form: decode K and V to vectors, then plain softmax attention.
    Mathematically identical to `attention_from_codes`."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, nq, d = q.shape
    Hkv = k_codes["idx"].shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, nq, d))
    for b in range(B):
        for g in range(Hkv):
            khat = decode_prod(k_codes["idx"][b, g], k_codes["sign"][b, g],
                               k_codes["norm"][b, g], k_codes["rnorm"][b, g],
                               k_book["signs"], k_book["centroids"], k_book["S"])
            vhat = decode_mse(v_codes["idx"][b, g], v_codes["norm"][b, g],
                              v_book["signs"], v_book["centroids"])
            for h in range(g * G, (g + 1) * G):
                out[b, h] = _softmax_rows(q[b, h] @ khat.T * scale) @ vhat
    return out
