"""Pins of the outlier-channel split (oracle/split.py): the page's rate
points, the selection rule on a hand-made example, the error of each half
against the scalar codec's closed-form distortion (exact in expectation for
isotropic Gaussian halves under any fixed orthogonal rotation), the
unbiasedness of the summed key estimate over draws of S, and the identities
that tie the estimate and the attention to the materialized decode.

[TurboQuant-es] "Desempeño teórico y empírico"; [TurboQuant-pl] "Co to
oznacza w praktyce?".
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import split as SP

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def page_figures():
    out = {}
    with open(os.path.join(GOLDEN, "page_figures.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()[:2]
                out[k] = float(v)
    return out


def half(d, bits, mode, rng):
    """One half's codec parameters: mse at `bits`, prod at `bits` total
    (bits - 1 table bits + the QJL bit, S Gaussian d x d)."""
    signs = rng.integers(0, 2, d).astype(bool)
    if mode == "prod":
        c, t = oracle.codebook(d, bits - 1)
        return {"signs": signs, "centroids": c, "thresholds": t,
                "S": rng.standard_normal((d, d))}
    c, t = oracle.codebook(d, bits)
    return {"signs": signs, "centroids": c, "thresholds": t}


def test_page_rate_points():
    fig = page_figures()
    assert SP.effective_rate(64, 3, 64, 2) == fig["split_rate_3_2"]
    assert SP.effective_rate(64, 4, 64, 3) == fig["split_rate_4_3"]
    # the same rates from other partitions of other widths
    assert SP.effective_rate(32, 3, 32, 2) == 2.5 and SP.effective_rate(32, 4, 96, 2) == 2.5


def test_outlier_permutation_hand_example():
    """Channel scales 1, 5, 5, 0.1, 3, 3: the three largest are 1 and 2 (tied)
    and then 4 (tied with 5, the lower index wins)."""
    scale = np.array([1.0, 5.0, 5.0, 0.1, 3.0, 3.0])
    calib = np.ones((10, 1)) * scale[None, :] * np.array([[1], [-1]] * 5)
    assert SP.outlier_permutation(calib, 3).tolist() == [1, 2, 4, 0, 3, 5]
    assert SP.outlier_permutation(calib, 0).tolist() == list(range(6))
    perm = SP.outlier_permutation(np.random.default_rng(0).standard_normal((50, 16)), 5)
    assert sorted(perm.tolist()) == list(range(16))


def test_outlier_permutation_finds_planted_channels():
    rng = np.random.default_rng(3)
    x = rng.standard_t(3, (4096, 128))
    planted = np.array([7, 40, 77, 120])
    x[:, planted] *= 20.0
    perm = SP.outlier_permutation(x, 64)
    assert set(planted.tolist()) <= set(perm[:64].tolist())
    assert np.all(np.diff(perm[:64]) > 0) and np.all(np.diff(perm[64:]) > 0)


@pytest.mark.parametrize("b_hi,b_lo", [(3, 2), (4, 3)])
def test_each_half_error_is_its_distortion(b_hi, b_lo):
    """mse halves: |x - x_hat|^2 is the sum of the halves' errors (disjoint
    channels), and for isotropic Gaussian halves E|x_h - x_hat_h|^2 / |x_h|^2
    is the scalar table's normalized distortion D(b) at d = 64, whatever the
    halves' scales (10:1 here)."""
    rng = np.random.default_rng(b_hi)
    n, d = 20000, 128
    x = rng.standard_normal((n, d))
    x[:, :64] *= 10.0
    hi, lo = half(64, b_hi, "mse", rng), half(64, b_lo, "mse", rng)
    enc = SP.encode_split_mse(x, 64, hi, lo)
    xh = SP.decode_split(enc, hi, lo)
    err_hi = np.sum((x[:, :64] - xh[:, :64]) ** 2, axis=1)
    err_lo = np.sum((x[:, 64:] - xh[:, 64:]) ** 2, axis=1)
    assert np.allclose(np.sum((x - xh) ** 2, axis=1), err_hi + err_lo, rtol=1e-12)
    for err, part, bits in ((err_hi, x[:, :64], b_hi), (err_lo, x[:, 64:], b_lo)):
        rel = err / np.sum(part * part, axis=1)
        want = oracle.distortion(64, oracle.codebook(64, bits)[0])
        assert abs(rel.mean() - want) <= 4.0 * rel.std() / math.sqrt(n), (bits, rel.mean(), want)


def test_split_prod_estimate_is_unbiased():
    """E over the draws of S_hi and S_lo of the summed estimate is <q, x>
    (each half's QJL term is unbiased for its residual)."""
    rng = np.random.default_rng(11)
    d_hi = d_lo = 16
    x = rng.standard_normal((3, d_hi + d_lo)) * np.array([4.0] * d_hi + [1.0] * d_lo)
    q = rng.standard_normal((2, d_hi + d_lo))
    hi, lo = half(d_hi, 3, "prod", rng), half(d_lo, 2, "prod", rng)
    trials = 4000
    ests = np.empty((trials, 2, 3))
    for t in range(trials):
        hi["S"] = rng.standard_normal((d_hi, d_hi))
        lo["S"] = rng.standard_normal((d_lo, d_lo))
        enc = SP.encode_split_prod(x, d_hi, hi, lo)
        ests[t] = SP.estimate_split(q, enc, d_hi, hi, lo)
    mean, se = ests.mean(axis=0), ests.std(axis=0) / math.sqrt(trials)
    z = (mean - q @ x.T) / se
    assert np.all(np.abs(z) < 4.5), z
    # a dropped QJL term on one half biases the estimate
    enc = SP.encode_split_prod(x, d_hi, hi, lo)
    only_tables = SP.estimate_split(q, (oracle.EncodedMSE(enc[0].idx, enc[0].norm), enc[1]), d_hi, hi, lo)
    assert not np.allclose(only_tables, SP.estimate_split(q, enc, d_hi, hi, lo))


def test_estimate_and_attention_equal_the_materialized_forms():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 128)) * rng.uniform(0.1, 10, (40, 1))
    v = rng.standard_normal((40, 128))
    q = rng.standard_normal((3, 128))
    khi, klo = half(64, 4, "prod", rng), half(64, 3, "prod", rng)
    vhi, vlo = half(64, 4, "mse", rng), half(64, 3, "mse", rng)
    kenc = SP.encode_split_prod(x, 64, khi, klo)
    venc = SP.encode_split_mse(v, 64, vhi, vlo)
    kh, vh = SP.decode_split(kenc, khi, klo), SP.decode_split(venc, vhi, vlo)
    est = SP.estimate_split(q, kenc, 64, khi, klo)
    assert np.allclose(est, q @ kh.T, rtol=1e-12, atol=1e-12)
    s = q @ kh.T / math.sqrt(128)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    want = (p / p.sum(axis=1, keepdims=True)) @ vh
    got = SP.attention_split(q, kenc, venc, 64, khi, klo, vhi, vlo)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_calibrated_split_beats_uniform_low_rate_on_outlier_channels():
    """Keys with four channels scaled x20: the split at 2.5 bits with the
    outliers in the 3-bit half has a lower error than a uniform 2-bit codec,
    and than the same split with the outliers forced into the 2-bit half."""
    rng = np.random.default_rng(8)
    x = rng.standard_t(3, (4096, 128))
    x[:, [3, 50, 90, 111]] *= 20.0
    hi, lo = half(64, 3, "mse", rng), half(64, 2, "mse", rng)

    def rel(xx, xh):
        return float(np.mean(np.sum((xx - xh) ** 2, axis=1) / np.sum(xx * xx, axis=1)))

    perm = SP.outlier_permutation(x[:1024], 64)
    xp = x[:, perm]
    good = rel(xp, SP.decode_split(SP.encode_split_mse(xp, 64, hi, lo), hi, lo))
    xr = x[:, np.concatenate([perm[64:], perm[:64]])]
    bad = rel(xr, SP.decode_split(SP.encode_split_mse(xr, 64, hi, lo), hi, lo))
    c2, t2 = oracle.codebook(128, 2)
    flip = rng.integers(0, 2, 128).astype(bool)
    e = oracle.encode_mse(x, flip, t2)
    uniform2 = rel(x, oracle.decode_mse(e.idx, e.norm, flip, c2))
    assert good < 0.6 * uniform2 and good < 0.6 * bad, (good, bad, uniform2)
