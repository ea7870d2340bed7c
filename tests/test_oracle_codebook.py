"""Pins of the oracle's coordinate density and Lloyd-Max codebook.

Each check uses something the oracle itself does not: scipy quadrature, the
incomplete-beta CDF, closed-form antiderivatives, the textbook uniform and
Gaussian reductions, and the figures printed on the pages.
"""

import math
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import beta_coord_pdf, codebook, distortion, lloyd_max

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_figure(key):
    with open(os.path.join(GOLDEN, "page_figures.txt")) as f:
        for line in f:
            if line.startswith(key + " "):
                return float(line.split()[1])
    raise KeyError(key)


def _max_table():
    rows = {}
    with open(os.path.join(GOLDEN, "max1960_gaussian_levels.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = line.split()
            rows[int(v[0])] = (float(v[1]), np.array([float(a) for a in v[2:]]))
    return rows


def _abs_mean(d):
    # E|X| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)), evaluated with scipy
    return special.gamma(d / 2) / (math.sqrt(math.pi) * special.gamma((d + 1) / 2)) \
        if d < 300 else math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)


def _cdf(t, d):
    # X^2 ~ Beta(1/2, (d-1)/2) for a coordinate of a uniform point on S^{d-1}
    return 0.5 + 0.5 * np.sign(t) * special.betainc(0.5, (d - 1) / 2.0, np.asarray(t) ** 2)


def _first_moment(a, b, d):
    # closed form of int_a^b x f_d(x) dx: -C (1-x^2)^{alpha+1} / (2(alpha+1))
    alpha = (d - 3) / 2.0
    logc = special.gammaln(d / 2) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2)
    F = lambda x: -math.exp(logc) * (1 - x * x) ** (alpha + 1) / (2 * (alpha + 1))
    return F(b) - F(a)


@pytest.mark.parametrize("d", [3, 8, 64, 128, 1536])
def test_density_normalised_and_moments(d):
    f = lambda x: float(beta_coord_pdf(np.array([x]), d)[0])
    pts = [-3 / math.sqrt(d), 0.0, 3 / math.sqrt(d)] if d > 9 else None
    mass = integrate.quad(f, -1, 1, points=pts, limit=200)[0]
    var = integrate.quad(lambda x: x * x * f(x), -1, 1, points=pts, limit=200)[0]
    absm = integrate.quad(lambda x: abs(x) * f(x), -1, 1, points=pts, limit=200)[0]
    assert abs(mass - 1) < 1e-10
    assert abs(var - 1.0 / d) < 1e-10 / d          # Var X = 1/d exactly
    assert abs(absm - _abs_mean(d)) < 1e-10


def test_abs_mean_values():
    # closed-form E|X| at the dimensions of the workloads
    assert _abs_mean(128) == pytest.approx(0.0706616, abs=1e-7)
    assert _abs_mean(64) == pytest.approx(0.1001259, abs=1e-7)
    assert _abs_mean(1536) == pytest.approx(0.0203618, abs=1e-7)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_d3_is_uniform_quantizer(bits):
    # d = 3: f is uniform on [-1, 1], so Lloyd-Max is the uniform quantizer
    n = 1 << bits
    c, t = codebook(3, bits)
    expect = -1 + (2 * np.arange(n) + 1) / n
    assert np.max(np.abs(c - expect)) < 1e-12
    assert np.max(np.abs(t - (-1 + 2 * np.arange(1, n) / n))) < 1e-12


@pytest.mark.parametrize("d,bits", [(64, 2), (64, 3), (128, 2), (128, 3), (128, 4),
                                    (1536, 1), (1536, 2)])
def test_optimality_conditions(d, bits):
    c, t = codebook(d, bits)
    n = 1 << bits
    assert np.all(np.diff(c) > 0)
    # midpoint condition (exact) and symmetry of the log-concave even density
    assert np.array_equal(t, 0.5 * (c[:-1] + c[1:]))
    assert np.max(np.abs(c + c[::-1])) < 1e-14
    # centroid condition with closed-form numerator and incomplete-beta mass
    edges = np.concatenate(([-1.0], t, [1.0]))
    for k in range(n):
        mass = _cdf(edges[k + 1], d) - _cdf(edges[k], d)
        mean = _first_moment(edges[k], edges[k + 1], d) / mass
        assert abs(mean - c[k]) < 1e-12, (k, mean, c[k])


@pytest.mark.parametrize("d", [64, 128, 1536])
def test_one_bit_is_plus_minus_abs_mean(d):
    c, t = codebook(d, 1)
    assert np.allclose(c, [-_abs_mean(d), _abs_mean(d)], rtol=0, atol=1e-13)
    assert t[0] == 0.0
    # distortion of the 1-bit table: d (E X^2 - (E|X|)^2) = 1 - d (E|X|)^2
    assert distortion(d, c) == pytest.approx(1 - d * _abs_mean(d) ** 2, abs=1e-12)


def _gauss_lloyd_max(n, iters=20000):
    """Independent Lloyd-Max for N(0, 1) with closed-form Gaussian cell moments."""
    c = np.linspace(-2, 2, n)
    for _ in range(iters):
        e = np.concatenate(([-np.inf], 0.5 * (c[1:] + c[:-1]), [np.inf]))
        mass = stats.norm.cdf(e[1:]) - stats.norm.cdf(e[:-1])
        c_new = (stats.norm.pdf(e[:-1]) - stats.norm.pdf(e[1:])) / mass
        if np.max(np.abs(c_new - c)) < 1e-14:
            return c_new
        c = c_new
    return c


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_large_d_tends_to_gaussian_lloyd_max(bits):
    n = 1 << bits
    g = _gauss_lloyd_max(n)
    mse_tab, lv_tab = _max_table()[n]
    # the independent Gaussian solution reproduces the textbook table
    assert np.allclose(g[n // 2:], lv_tab, atol=1.5e-3)
    errs = []
    for d in (128, 1536, 16384):
        c, _, _ = lloyd_max(d, bits)
        errs.append(np.max(np.abs(math.sqrt(d) * c - g)))
    # O(1/d) approach to the limit
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 6.0 / 16384 * g[-1]


def test_distortion_against_page_ratios():
    """[TurboQuant-es] "Desempeño teórico y empírico": distortion within a
    factor of about 2.7 of the 4^-b lower bound at every bit width, about
    1.45 at b = 1."""
    r_all = _page_figure("distortion_ratio_all_b")
    r_b1 = _page_figure("distortion_ratio_b1")
    panter_dite = math.pi * math.sqrt(3) / 2          # high-rate Gaussian limit, 2.7207
    for d in (64, 128, 1536):
        ratios = [distortion(d, codebook(d, b)[0]) * 4 ** b for b in (1, 2, 3, 4)]
        assert all(np.diff(ratios) > 0)
        assert ratios[-1] < panter_dite
        assert abs(panter_dite - r_all) < 0.03
        assert ratios[0] == pytest.approx(r_b1, abs=0.02)
    # b = 1 Gaussian limit 4 (1 - 2/pi) = 1.4535
    assert distortion(1536, codebook(1536, 1)[0]) * 4 == pytest.approx(4 * (1 - 2 / math.pi), abs=2e-3)


@pytest.mark.parametrize("d,bits", [(128, 3), (64, 2)])
def test_codebook_is_local_minimum(d, bits):
    c, _ = codebook(d, bits)
    base = distortion(d, c)
    rng = np.random.default_rng(7)
    for _ in range(20):
        pert = c + rng.normal(scale=1e-3 / math.sqrt(d), size=c.shape)
        assert distortion(d, np.sort(pert)) >= base - 1e-15
