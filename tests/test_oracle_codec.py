"""Pins of the oracle's encode / decode / estimate.

* packing: a hand-worked byte example and round trips;
* quantizer: brute-force nearest centroid;
* mse distortion: Monte Carlo against the codebook's own D(b) integral;
* mse inner-product bias (1 - D(b)) under a Haar rotation, and its 2/pi
  high-dimension limit printed on [TurboQuant-es] "Eliminación del sesgo
  interno del producto";
* TurboQuant_prod unbiasedness over many QJL matrices, with the closed-form
  per-seed variance ([TurboQuant-es] same section; [TurboQuant-pl] "Błąd
  średniokwadratowy to pułapka");
* brute-force sign bits and the zero vector.
"""

import math
import os

import numpy as np
import pytest
from scipy import special

from oracle import (codebook, distortion, encode_mse, encode_prod, decode_mse,
                    decode_prod, estimate_ip, pack_codes, unpack_codes,
                    pack_bits, unpack_bits, haar_rotation, rotate)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pack_example():
    vals = {}
    with open(os.path.join(GOLDEN, "pack_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            vals[k] = [int(a) for a in v]
    return vals


def test_pack_golden_example():
    ex = _pack_example()
    bits = ex["bits"][0]
    codes = np.array([ex["codes"]])
    assert pack_codes(codes, bits).tolist() == [ex["bytes"]]
    assert unpack_codes(np.array([ex["bytes"]], dtype=np.uint8), 8, bits).tolist() == [ex["codes"]]
    sb = np.array([ex["signbits"]])
    assert pack_bits(sb).tolist() == [ex["signbytes"]]
    assert unpack_bits(np.array([ex["signbytes"]], dtype=np.uint8), 16).tolist() == [ex["signbits"]]


@pytest.mark.parametrize("d,bits", [(64, 1), (64, 2), (128, 3), (128, 4), (1536, 1), (1536, 3)])
def test_pack_round_trip(d, bits):
    rng = np.random.default_rng(bits * d)
    idx = rng.integers(0, 1 << bits, size=(7, d))
    packed = pack_codes(idx, bits)
    assert packed.shape == (7, d * bits // 8)
    assert np.array_equal(unpack_codes(packed, d, bits), idx)
    # code i sits at stream bits [i b, (i+1) b) (explicit bit reads)
    for i in (0, 1, d // 2 + 1, d - 1):
        v = 0
        for t in range(bits):
            k = i * bits + t
            v |= ((int(packed[3, k // 8]) >> (k % 8)) & 1) << t
        assert v == idx[3, i]


@pytest.mark.parametrize("d,bits", [(64, 2), (128, 3), (128, 4)])
def test_quantizer_is_nearest_centroid(d, bits):
    c, t = codebook(d, bits)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((400, d))
    enc = encode_mse(x, np.ones(d), t)
    near = np.argmin(np.abs(enc.z[..., None] - c[None, None, :]), axis=-1)
    assert np.array_equal(enc.idx, near)
    assert np.allclose(enc.norm, np.linalg.norm(x, axis=1), rtol=1e-15)


@pytest.mark.parametrize("d,bits", [(64, 2), (128, 3)])
def test_mse_matches_codebook_distortion(d, bits):
    # For x uniform on the sphere, Pi x is uniform for any fixed rotation,
    # so E|x - x_hat|^2 / |x|^2 equals the codebook's D(b).
    c, t = codebook(d, bits)
    rng = np.random.default_rng(5)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    x = rng.standard_normal((20000, d)) * 3.0
    enc = encode_mse(x, signs, t)
    xh = decode_mse(enc.idx, enc.norm, signs, c)
    rel = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    dist = distortion(d, c)
    se = rel.std() / math.sqrt(len(rel))
    assert abs(rel.mean() - dist) < 4 * se


def _abs_mean(d):
    return math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)


@pytest.mark.parametrize("bits", [1, 2])
def test_mse_inner_product_bias_under_haar(bits):
    """E_Pi <y, x_hat_mse> = (1 - D(b)) <y, x> for a Haar rotation; at b = 1
    the factor is d (E|X|)^2, which tends to 2/pi."""
    d = 32
    c, t = codebook(d, bits)
    rng = np.random.default_rng(100 + bits)
    x = rng.standard_normal(d)
    x /= np.linalg.norm(x)
    y = 0.6 * x + 0.8 * np.linalg.qr(np.stack([x, rng.standard_normal(d)], 1))[0][:, 1]
    ones = np.ones(d)
    vals = []
    for _ in range(12000):
        q = haar_rotation(d, rng)
        enc = encode_mse((q @ x)[None], ones, t)
        vals.append(float(decode_mse(enc.idx, enc.norm, ones, c)[0] @ (q @ y)))
    vals = np.array(vals)
    expect = (1 - distortion(d, c)) * float(x @ y)
    assert abs(vals.mean() - expect) < 4 * vals.std() / math.sqrt(len(vals))
    if bits == 1:
        assert 1 - distortion(d, c) == pytest.approx(d * _abs_mean(d) ** 2, abs=1e-12)


def test_one_bit_bias_tends_to_two_over_pi():
    page = 2 / math.pi    # [TurboQuant-es] "Eliminación del sesgo interno del producto"
    vals = [1 - distortion(d, codebook(d, 1)[0]) for d in (64, 128, 1536)]
    assert vals[0] > vals[1] > vals[2] > page
    assert vals[2] - page < 3e-4
    assert vals[1] == pytest.approx(0.63911, abs=2e-5)


def _qjl_trial(d, bits, n_seeds, seed):
    c, t = codebook(d, bits - 1)
    rng = np.random.default_rng(seed)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    x = rng.standard_normal((1, d)) * 2.5
    q = rng.standard_normal((1, d))
    ests = np.empty(n_seeds)
    for s in range(n_seeds):
        S = rng.standard_normal((d, d))
        enc = encode_prod(x, signs, c, t, S)
        ests[s] = estimate_ip(q, enc.idx, enc.norm, signs, c, sign=enc.sign,
                              rnorm=enc.rnorm, S=S)[0, 0]
    # the residual does not depend on S
    r = enc.z - c[enc.idx]
    qr = rotate(q, signs)[0]
    nu, gamma = enc.norm[0], enc.rnorm[0]
    var = nu ** 2 / d * (math.pi / 2 * gamma ** 2 * qr @ qr - (r[0] @ qr) ** 2)
    return ests, float(q[0] @ x[0]), var


@pytest.mark.parametrize("d,bits,seed", [(16, 3, 1), (16, 2, 2), (16, 4, 3)])
def test_prod_unbiased_and_variance(d, bits, seed):
    ests, truth, var = _qjl_trial(d, bits, 20000, seed)
    zscore = (ests.mean() - truth) / math.sqrt(var / len(ests))
    assert abs(zscore) < 4
    assert 0.93 < ests.var() / var < 1.07


def test_prod_unbiased_d128():
    ests, truth, var = _qjl_trial(128, 3, 2000, 9)
    assert abs((ests.mean() - truth) / math.sqrt(var / len(ests))) < 4
    assert 0.85 < ests.var() / var < 1.15


def test_zscores_over_pairs_look_standard():
    zs = []
    for seed in range(20):
        ests, truth, var = _qjl_trial(8, 3, 1500, 1000 + seed)
        zs.append((ests.mean() - truth) / math.sqrt(var / len(ests)))
    zs = np.array(zs)
    assert abs(zs.mean()) < 4 / math.sqrt(len(zs))
    assert 0.4 < zs.std() < 1.6


def test_sign_bits_brute_force():
    d = 8
    c, t = codebook(d, 2)
    rng = np.random.default_rng(4)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    S = rng.standard_normal((d, d))
    x = rng.standard_normal((3, d))
    enc = encode_prod(x, signs, c, t, S)
    for n in range(3):
        r = [enc.z[n, k] - c[enc.idx[n, k]] for k in range(d)]
        assert enc.rnorm[n] == pytest.approx(math.sqrt(sum(v * v for v in r)), rel=1e-14)
        for i in range(d):
            p = 0.0
            for k in range(d):
                p += S[i, k] * r[k]
            assert enc.sign[n, i] == (1 if p >= 0 else 0)


def test_estimate_equals_inner_product_with_decoded():
    d = 64
    c, t = codebook(d, 2)
    rng = np.random.default_rng(8)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    S = rng.standard_normal((d, d))
    x = rng.standard_normal((50, d))
    q = rng.standard_normal((6, d))
    enc = encode_prod(x, signs, c, t, S)
    est = estimate_ip(q, enc.idx, enc.norm, signs, c, sign=enc.sign, rnorm=enc.rnorm, S=S)
    xh = decode_prod(enc.idx, enc.sign, enc.norm, enc.rnorm, signs, c, S)
    assert np.allclose(est, q @ xh.T, atol=1e-12)
    encm = encode_mse(x, signs, t)
    estm = estimate_ip(q, encm.idx, encm.norm, signs, c)
    assert np.allclose(estm, q @ decode_mse(encm.idx, encm.norm, signs, c).T, atol=1e-12)


def test_zero_vector():
    d = 128
    c, t = codebook(d, 3)
    S = np.random.default_rng(0).standard_normal((d, d))
    enc = encode_prod(np.zeros((1, d)), np.ones(d), c, t, S)
    assert enc.norm[0] == 0.0
    assert np.all(enc.idx == np.sum(0.0 >= t))
    assert enc.rnorm[0] == pytest.approx(np.linalg.norm(c[np.sum(0.0 >= t)] * np.ones(d)))
    q = np.ones((1, d))
    assert estimate_ip(q, enc.idx, enc.norm, np.ones(d), c, sign=enc.sign,
                       rnorm=enc.rnorm, S=S)[0, 0] == 0.0


def test_residual_from_codes_brute_force_and_cell_bounds():
    """The conditional QJL check re-derives r = z - c[idx] from given codes.
    Pinned three ways: element by element in plain Python on hand-edited
    codes; each residual of the oracle's own codes lies inside its cell
    (t_{k-1} - c_k <= r <= t_k - c_k, outer cells to -1 and +1); and, on the
    oracle's own codes, |r| equals the stored gamma and the sign bits of
    S r equal the stored ones.  A flipped sign, a shifted table index or a
    transposed operand fails one of these."""
    from oracle.codec import residual_from_codes
    d = 16
    c, t = codebook(d, 2)
    rng = np.random.default_rng(21)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    S = rng.standard_normal((d, d))
    x = rng.standard_normal((5, d))
    enc = encode_prod(x, signs, c, t, S)
    edited = enc.idx.copy()
    edited[0, 3] = (edited[0, 3] + 1) % 4
    edited[2, :] = 3 - edited[2, :]
    edited[4, 7] = 0
    r = residual_from_codes(enc.z, edited, c)
    for n in range(5):
        for k in range(d):
            assert r[n, k] == enc.z[n, k] - c[edited[n, k]]
    lo = np.concatenate([[-1.0], t])
    hi = np.concatenate([t, [1.0]])
    r0 = residual_from_codes(enc.z, enc.idx, c)
    assert np.all(r0 >= lo[enc.idx] - c[enc.idx] - 1e-15)
    assert np.all(r0 <= hi[enc.idx] - c[enc.idx] + 1e-15)
    assert np.allclose(np.sqrt(np.sum(r0 * r0, axis=1)), enc.rnorm, rtol=1e-14, atol=0)
    p = np.array([[sum(S[i, k] * r0[n, k] for k in range(d)) for i in range(d)] for n in range(5)])
    assert np.array_equal((p >= 0).astype(np.uint8), enc.sign)


def test_non_finite_rows_take_the_zero_vector_codes():
    """A row holding inf or NaN gets the zero vector's codes (idx, sign
    bits, gamma) and keeps its non-finite norm: inf for an infinite element,
    NaN when a NaN is present.  Other rows are unaffected."""
    d = 32
    c, t = codebook(d, 3)
    rng = np.random.default_rng(5)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    S = rng.standard_normal((d, d))
    x = rng.standard_normal((6, d))
    x[1, 4] = np.inf
    x[2, 0] = -np.inf
    x[3, 9] = np.nan
    x[4, 1], x[4, 2] = np.inf, np.nan
    x[5] = 0.0
    enc = encode_prod(x, signs, c, t, S)
    mse = encode_mse(x, signs, t)
    zero = encode_prod(np.zeros((1, d)), signs, c, t, S)
    for n in (1, 2, 3, 4, 5):
        assert np.array_equal(enc.idx[n], zero.idx[0]) and np.array_equal(mse.idx[n], zero.idx[0])
        assert np.array_equal(enc.sign[n], zero.sign[0])
        assert enc.rnorm[n] == zero.rnorm[0]
    assert np.isposinf(enc.norm[1]) and np.isposinf(enc.norm[2])
    assert np.isnan(enc.norm[3]) and np.isnan(enc.norm[4]) and enc.norm[5] == 0.0
    assert np.array_equal(mse.norm[1:3], enc.norm[1:3])
    alone = encode_prod(x[:1], signs, c, t, S)
    assert np.array_equal(alone.idx, enc.idx[:1]) and alone.norm[0] == enc.norm[0]
