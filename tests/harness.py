"""Statistical validation harness (test infrastructure).

"Riepilogo Tecnico: Ablazione, Inferenza Statistica e Validazione",
"Configurazione Sperimentale" and "Validazione Statistica e Disuguaglianza
di Jensen":
* metrics: relMSE (mean over rows of |x - x_hat|^2 / |x|^2), the direction
  error through cosine similarity, and the 2-D metric d^2 combining them;
  relMSE_K and relMSE_V isolate the two caches, the attention output's
  relMSE / cosine / d^2 the end result;
* the oracle and the GPU library run with different random number
  generators for the codec's own draws (D and S): PCG64 on the oracle side,
  MT19937 on the GPU side; a two-sample Kolmogorov-Smirnov test on the
  per-seed metric distributions separates a systematic difference from
  seed-to-seed variance.

Readings where the page is silent:
* d^2 = relMSE^2 + (1 - cos)^2: the squared distance of the point
  (relMSE, 1 - cos) from the error-free point (0, 0).
* The two schemes at a budget of b bits per coordinate: TQ-KV = mse keys
  and values at b bits; TQ-QKV = prod keys (b - 1 bit table + 1-bit QJL)
  and mse values at b bits.  Two more at 2.5 bits: FQ = FibQuant k = 2 at
  N = 32 for keys and values; SPLIT = the outlier-channel split, 3 bits on
  the 64 channels of largest mean square (measured on the tensor itself)
  and 2 on the rest, prod keys and mse values (both sides order the
  channels with their own implementation of the rule, and the decoded
  channels are put back in the original order).
* The reference attention is plain softmax attention in fp64 on the
  unquantized K, V (scale 1 / sqrt(d)); the codec's attention output is the
  same attention on the decoded vectors (equal to attention from codes, a
  pinned identity of the oracle).
"""

import math

import numpy as np
from scipy import stats as sstats

import oracle
import synth
from synth import regimes

SCHEMES = ("TQ-KV", "TQ-QKV")
SCHEMES_25 = ("FQ", "SPLIT")          # 2.5 bits per coordinate


def rel_mse(x, xh):
    x = np.asarray(x, dtype=np.float64)
    xh = np.asarray(xh, dtype=np.float64)
    return float(np.mean(np.sum((x - xh) ** 2, axis=-1) / np.sum(x * x, axis=-1)))


def cosine(x, xh):
    x = np.asarray(x, dtype=np.float64)
    xh = np.asarray(xh, dtype=np.float64)
    return float(np.mean(np.sum(x * xh, axis=-1) /
                         (np.linalg.norm(x, axis=-1) * np.linalg.norm(xh, axis=-1))))


def d2(rel, cos):
    return rel * rel + (1.0 - cos) ** 2


def attention(q, k, v):
    """softmax(q k^T / sqrt(d)) v in fp64."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    s = q @ k.T / math.sqrt(q.shape[-1])
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return (p / p.sum(axis=-1, keepdims=True)) @ v


def codec_rng(family, seed):
    """Generator of the codec's own draws: "pcg64" (oracle) or "mt19937" (GPU)."""
    bitgen = {"pcg64": np.random.PCG64, "mt19937": np.random.MT19937}[family]
    return np.random.Generator(bitgen(np.random.SeedSequence(90000 + seed)))


def data(regime, seed, n=512, d=128, n_q=4):
    """The seed's K, V, q (identical for both sides)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(70000 + seed)))
    return regimes.draw(regime, rng, n=n, d=d, n_q=n_q)


def draws_for(scheme, rng, d):
    """The codec's own draws: (K, V) sign flips and S; for SPLIT one pair
    per 64-channel half ((K hi, K lo), (V hi, V lo))."""
    if scheme == "SPLIT":
        kd = (synth.codec_draws(rng, d // 2, m=d // 2), synth.codec_draws(rng, d // 2, m=d // 2))
        vd = (synth.codec_draws(rng, d // 2), synth.codec_draws(rng, d // 2))
        return kd, vd
    kd = synth.codec_draws(rng, d, m=d if scheme == "TQ-QKV" else 0)
    vd = synth.codec_draws(rng, d)
    return kd, vd


_FQ_BOOK = {}


def fq_book(d, n_codes=32):
    if (d, n_codes) not in _FQ_BOOK:
        _FQ_BOOK[(d, n_codes)] = oracle.fibquant_codebook(d, n_codes)
    return _FQ_BOOK[(d, n_codes)]


def split_half(draws, bits, prod):
    if prod:
        c, t = oracle.codebook(draws.flip.size, bits - 1)
        return {"signs": draws.flip, "centroids": c, "thresholds": t,
                "S": draws.S.astype(np.float64)}
    c, t = oracle.codebook(draws.flip.size, bits)
    return {"signs": draws.flip, "centroids": c, "thresholds": t}


def _split_decoded(x, draws, prod):
    perm = oracle.outlier_permutation(x, x.shape[1] // 2)
    hi, lo = split_half(draws[0], 3, prod), split_half(draws[1], 2, prod)
    xp = x[:, perm]
    enc = (oracle.encode_split_prod if prod else oracle.encode_split_mse)(xp, x.shape[1] // 2, hi, lo)
    out = np.empty_like(xp)
    out[:, perm] = oracle.decode_split(enc, hi, lo)
    return out


def metrics(k, v, q, kh, vh):
    o = attention(q, k, v)
    oh = attention(q, kh, vh)
    ro, co = rel_mse(o, oh), cosine(o, oh)
    return {"relmse_k": rel_mse(k, kh), "relmse_v": rel_mse(v, vh), "relmse_o": ro,
            "cos_o": co, "d2_o": d2(ro, co)}


def oracle_decoded(scheme, bits, k, v, kd, vd, qjl_factor_scale=1.0):
    """Oracle encode + decode of K and V.  `qjl_factor_scale` != 1 plants a
    wrong QJL constant (used only to show the KS test's power)."""
    d = k.shape[-1]
    k64, v64 = k.astype(np.float64), v.astype(np.float64)
    if scheme == "FQ":
        code = fq_book(d)
        ik, nk, _ = oracle.encode_vq(k64, kd.flip, code)
        iv, nv, _ = oracle.encode_vq(v64, vd.flip, code)
        return oracle.decode_vq(ik, nk, kd.flip, code), oracle.decode_vq(iv, nv, vd.flip, code)
    if scheme == "SPLIT":
        return _split_decoded(k64, kd, True), _split_decoded(v64, vd, False)
    if scheme == "TQ-QKV":
        c, t = oracle.codebook(d, bits - 1)
        S = kd.S.astype(np.float64)
        e = oracle.encode_prod(k64, kd.flip, c, t, S)
        kh = oracle.decode_prod(e.idx, e.sign, e.norm, e.rnorm * qjl_factor_scale, kd.flip, c, S)
    else:
        c, t = oracle.codebook(d, bits)
        e = oracle.encode_mse(k64, kd.flip, t)
        kh = oracle.decode_mse(e.idx, e.norm, kd.flip, c)
    cv, tv = oracle.codebook(d, bits)
    ev = oracle.encode_mse(v64, vd.flip, tv)
    vh = oracle.decode_mse(ev.idx, ev.norm, vd.flip, cv)
    return kh, vh


def oracle_run(regime, scheme, bits, seeds, family="pcg64", qjl_factor_scale=1.0):
    """Per-seed metrics of the oracle; returns {metric: array over seeds}."""
    out = {}
    for s in seeds:
        k, v, q = data(regime, s)
        kd, vd = draws_for(scheme, codec_rng(family, s), k.shape[-1])
        kh, vh = oracle_decoded(scheme, bits, k, v, kd, vd, qjl_factor_scale)
        for name, val in metrics(k, v, q, kh, vh).items():
            out.setdefault(name, []).append(val)
    return {name: np.array(vals) for name, vals in out.items()}


def ks_p(a, b):
    return float(sstats.ks_2samp(a, b).pvalue)
