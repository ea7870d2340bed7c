"""The statistical validation harness on the CPU: its metrics against closed
forms, the lognormal identity behind the Jensen effect, and the KS
methodology on the oracle itself (two RNG families agree; a planted wrong
constant is separated).  "Riepilogo Tecnico: Ablazione, Inferenza
Statistica e Validazione", "Configurazione Sperimentale" and "Validazione
Statistica e Disuguaglianza di Jensen"."""

import math

import numpy as np
import pytest

import harness as H


def test_metrics_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 16))
    assert H.rel_mse(x, x) == 0.0
    assert H.rel_mse(x, 2 * x) == pytest.approx(1.0, abs=1e-15)
    assert H.rel_mse(x, 0 * x) == pytest.approx(1.0, abs=1e-15)
    assert H.cosine(x, 3 * x) == pytest.approx(1.0, abs=1e-15)
    assert H.cosine(x, -x) == pytest.approx(-1.0, abs=1e-15)
    y = np.zeros((1, 4))
    y[0, 0] = 1.0
    z = np.zeros((1, 4))
    z[0, 1] = 1.0
    assert H.cosine(y, z) == 0.0
    assert H.d2(0.0, 1.0) == 0.0
    assert H.d2(0.3, 0.6) == pytest.approx(0.09 + 0.16, abs=1e-15)


def test_attention_reference_special_cases():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((7, 8))
    q = rng.standard_normal((3, 8))
    same = np.tile(rng.standard_normal((1, 8)), (7, 1))
    # identical keys: uniform weights, the mean of V
    assert np.allclose(H.attention(q, same, v), np.tile(v.mean(axis=0), (3, 1)), atol=1e-14)
    # one key far ahead of the others: its value
    k = rng.standard_normal((7, 8)) * 1e-3
    k[4] = q[0] * 1e4
    assert np.allclose(H.attention(q[:1], k, v)[0], v[4], atol=1e-12)


@pytest.mark.parametrize("sigma", [0.3, 0.8])
def test_lognormal_identity(sigma):
    """E[exp(s + eps)] = exp(s) exp(sigma^2 / 2) for eps ~ N(0, sigma^2): the
    convexity that turns zero-mean score noise into a biased softmax."""
    rng = np.random.default_rng(2)
    s = 1.7
    e = rng.standard_normal(400000) * sigma
    samples = np.exp(s + e)
    se = samples.std() / math.sqrt(len(samples))
    assert abs(samples.mean() - math.exp(s + sigma * sigma / 2)) < 4 * se
    # the softmax denominator over many tokens carries the same factor
    sj = rng.standard_normal(2000)
    ratio = np.exp(sj[None, :] + rng.standard_normal((200, 2000)) * sigma).sum(axis=1) / np.exp(sj).sum()
    assert ratio.mean() == pytest.approx(math.exp(sigma * sigma / 2), rel=0.01)


SEEDS = range(32)


@pytest.mark.parametrize("regime", ["isotropic", "heavy_tailed"])
@pytest.mark.parametrize("scheme", H.SCHEMES)
def test_ks_two_rng_families_agree_on_the_oracle(regime, scheme):
    """The same codec with its draws from PCG64 or MT19937: the per-seed
    metric distributions are not separated (only seed variance differs)."""
    a = H.oracle_run(regime, scheme, 3, SEEDS, "pcg64")
    b = H.oracle_run(regime, scheme, 3, SEEDS, "mt19937")
    for name in a:
        assert H.ks_p(a[name], b[name]) > 1e-3, name


@pytest.mark.parametrize("scheme", H.SCHEMES_25)
def test_ks_two_rng_families_agree_at_two_and_a_half_bits(scheme):
    """The same for FibQuant at N = 32 and the 3 / 2 outlier split, whose
    errors sit between the whole-codec 2- and 3-bit ones."""
    a = H.oracle_run("heavy_tailed", scheme, 3, SEEDS, "pcg64")
    b = H.oracle_run("heavy_tailed", scheme, 3, SEEDS, "mt19937")
    for name in a:
        assert H.ks_p(a[name], b[name]) > 1e-3, name
    lo = H.oracle_run("heavy_tailed", "TQ-KV", 2, range(8), "pcg64")
    hi = H.oracle_run("heavy_tailed", "TQ-KV", 3, range(8), "pcg64")
    assert hi["relmse_v"].mean() < a["relmse_v"].mean() < lo["relmse_v"].mean()


def test_ks_separates_a_planted_wrong_qjl_constant():
    """A plausible mistake planted in a copy of the oracle -- the QJL scale
    sqrt(pi/2)/m off by 25% -- is separated from the correct codec."""
    a = H.oracle_run("isotropic", "TQ-QKV", 3, SEEDS, "pcg64")
    b = H.oracle_run("isotropic", "TQ-QKV", 3, SEEDS, "mt19937", qjl_factor_scale=1.25)
    assert H.ks_p(a["relmse_k"], b["relmse_k"]) < 1e-6


@pytest.mark.parametrize("regime", ["isotropic", "heavy_tailed"])
def test_qjl_on_keys_widens_the_attention_error_spread(regime):
    """The Jensen signature: the 1-bit QJL correction on the keys adds
    zero-mean score noise, which softmax turns into a much wider spread of
    the attention-output error across seeds than the mse-only keys at the
    same bit budget."""
    kv = H.oracle_run(regime, "TQ-KV", 3, SEEDS, "pcg64")
    qkv = H.oracle_run(regime, "TQ-QKV", 3, SEEDS, "pcg64")
    assert qkv["relmse_o"].std() > 3 * kv["relmse_o"].std()
    assert qkv["relmse_o"].mean() > kv["relmse_o"].mean()
