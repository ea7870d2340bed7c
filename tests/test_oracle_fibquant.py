"""Pins of the FibQuant k = 2 oracle (oracle/fibquant.py) against things it
does not compute itself: the exact law of two coordinates of a uniform
point on the sphere (sampled independently through a chi-square), scipy's
Beta quantiles and numerical integration, the golden angle's other closed
form, a k-d tree for the nearest search, the scalar Lloyd-Max codec (pinned
on its own) for the rate comparison, and algebraic identities of the codec.

"FibQuant", "2.1 La Sorgente Canonica", "2.2 Costruzione del Codice",
"2.3 Codifica e Decodifica", "3.2 Vantaggio Vettoriale rispetto alla
Specializzazione Scalare".
"""

import functools
import math

import numpy as np
import pytest
from scipy import integrate, spatial
from scipy import stats as sstats

import oracle
from oracle import fibquant as F


@functools.lru_cache(maxsize=None)
def book(d, n):
    return F.fibquant_codebook(d, n)


def source_sample(d, n, seed):
    """First two coordinates of uniform points on S^{d-1}: g / sqrt(|g|^2 + c)
    with g ~ N(0, I_2) and c ~ chi^2_{d-2} independent."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((n, 2))
    c = rng.chisquare(d - 2, n)
    return g / np.sqrt(np.sum(g * g, axis=1) + c)[:, None]


def radial_mass(f, r, d):
    """Mass of a radial density f on the disk inside radius r."""
    return integrate.quad(lambda s: 2.0 * math.pi * s * f(s), 0.0, r, epsabs=1e-13, epsrel=1e-11)[0]


def pdf_r(d):
    return lambda s: float(F.block_pdf(np.array([[s, 0.0]]), d)[0])


@pytest.mark.parametrize("d", [6, 16, 64, 128])
def test_block_pdf_is_a_density_on_the_disk(d):
    assert radial_mass(pdf_r(d), 1.0, d) == pytest.approx(1.0, abs=1e-9)
    # zero outside the disk, circularly symmetric
    assert F.block_pdf(np.array([[0.8, 0.7], [1.0, 0.0]]), d).tolist() == [0.0, 0.0]
    th = np.linspace(0, 2 * math.pi, 7)
    v = F.block_pdf(0.3 * np.stack([np.cos(th), np.sin(th)], 1), d)
    assert np.allclose(v, v[0], rtol=1e-14)


@pytest.mark.parametrize("d", [16, 128])
def test_block_pdf_is_the_law_of_two_sphere_coordinates(d):
    """The radial CDF integrated from block_pdf matches the empirical CDF of
    |y|^2 for sphere samples, and the closed form of Beta(1, (d-2)/2)."""
    y = source_sample(d, 200000, 11 + d)
    s2 = np.sum(y * y, axis=1)
    for q in (0.1, 0.3, 0.5, 0.7, 0.9, 0.99):
        s = sstats.beta.ppf(q, 1.0, (d - 2) / 2.0)
        mass = radial_mass(pdf_r(d), math.sqrt(s), d)
        assert mass == pytest.approx(q, abs=1e-8)
        emp = float(np.mean(s2 <= s))
        assert abs(emp - mass) <= 5.0 * math.sqrt(q * (1 - q) / len(s2)), (q, emp, mass)


@pytest.mark.parametrize("d", [16, 64, 128])
def test_quadrature_rings_are_beta_quantiles(d):
    pts = F.quadrature(d)
    assert pts.shape == (F.QUAD_RINGS * F.QUAD_ANGLES, 2)
    r2 = np.sum(pts * pts, axis=1).reshape(F.QUAD_RINGS, F.QUAD_ANGLES)
    want = sstats.beta.ppf((np.arange(F.QUAD_RINGS) + 0.5) / F.QUAD_RINGS, 1.0, (d - 2) / 2.0)
    assert np.allclose(r2, want[:, None], rtol=1e-12, atol=1e-15)
    # E|y|^2 = 2/d for two coordinates of a unit vector; the midpoint rule on
    # the quantile scale falls short by the tail beyond the last ring (the
    # quantile function is steep near 1), below 1/(2R) relative
    assert 0.0 <= 1.0 - np.mean(r2) * d / 2.0 <= 0.5 / F.QUAD_RINGS
    # angles: equally spaced, half a step off the axis
    ang = np.mod(np.arctan2(pts[:F.QUAD_ANGLES, 1], pts[:F.QUAD_ANGLES, 0]), 2 * math.pi)
    assert np.allclose(ang, 2 * math.pi * (np.arange(F.QUAD_ANGLES) + 0.5) / F.QUAD_ANGLES)


@pytest.mark.parametrize("d,n", [(16, 8), (64, 32), (128, 16), (128, 256)])
def test_spiral_radii_follow_companding(d, n):
    """Bennett-Gersho point density ~ f^(1/2) for k = 2: the companded radius
    r_n holds mass (n + 1/2)/N of f^(1/2) (integrated from block_pdf) and is
    the Beta(1, d/4) quantile of r^2."""
    c = F.spiral_init(d, n)
    r = np.hypot(c[:, 0], c[:, 1])
    t = (np.arange(n) + 0.5) / n
    assert np.allclose(r * r, sstats.beta.ppf(t, 1.0, d / 4.0), rtol=1e-10, atol=1e-15)
    f = pdf_r(d)
    g = lambda s: math.sqrt(f(s))
    total = radial_mass(g, 1.0, d)
    for i in (0, n // 3, n - 1):
        assert radial_mass(g, r[i], d) / total == pytest.approx(t[i], abs=1e-8)


def test_spiral_angles_step_by_the_golden_angle():
    phi = (1.0 + math.sqrt(5.0)) / 2.0
    g = 2.0 * math.pi / (phi * phi)       # 2 pi (1 - 1/phi)
    assert F.GOLDEN_ANGLE == pytest.approx(g, rel=1e-15)
    for phase in (0.0, 0.5):
        c = F.spiral_init(64, 32, phase)
        ang = np.arctan2(c[:, 1], c[:, 0])
        step = np.mod(np.diff(ang), 2 * math.pi)
        assert np.allclose(step, g, atol=1e-12)
        assert np.mod(ang[0] - phase * g + math.pi, 2 * math.pi) - math.pi == pytest.approx(0.0, abs=1e-12)


def test_nearest_matches_kd_tree():
    rng = np.random.default_rng(5)
    code = rng.uniform(-1, 1, (37, 2))
    y = rng.uniform(-1.2, 1.2, (5000, 2))
    _, want = spatial.cKDTree(code).query(y)
    assert np.array_equal(F.nearest(y, code), want)
    # ties go to the lower index
    code2 = np.array([[1.0, 0.0], [-1.0, 0.0], [1.0, 0.0]])
    assert F.nearest(np.array([[0.0, 0.0], [2.0, 0.0]]), code2).tolist() == [0, 0]


def test_lloyd_step_brute_force():
    """One Lloyd step on a tiny point set: every codeword moves to the mean of
    the points the k-d tree assigns to it; a codeword with no points stays."""
    rng = np.random.default_rng(8)
    pts = rng.uniform(-1, 1, (60, 2))
    code = np.vstack([rng.uniform(-1, 1, (5, 2)), [[9.0, 9.0]]])
    _, a = spatial.cKDTree(code).query(pts)
    want = code.copy()
    for n in range(len(code)):
        members = [p for p, k in zip(pts.tolist(), a.tolist()) if k == n]
        if members:
            want[n] = [sum(p[0] for p in members) / len(members), sum(p[1] for p in members) / len(members)]
    got = F.lloyd(code, pts, iters=1)
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    assert got[5].tolist() == [9.0, 9.0]


@pytest.mark.parametrize("d,n", [(64, 16), (128, 32)])
def test_lloyd_lowers_the_error_monotonically(d, n):
    pts = F.quadrature(d)
    c = F.spiral_init(d, n)
    prev = F.block_mse(pts, c)
    for _ in range(8):
        c = F.lloyd(c, pts, iters=1)
        m = F.block_mse(pts, c)
        assert m <= prev * (1 + 1e-12)
        prev = m


@pytest.mark.parametrize("d", [64, 128])
def test_two_codewords_are_the_one_bit_scalar_quantizer(d):
    """N = 2: the optimal code is antipodal at the half-plane centroid, which
    is the 1-bit Lloyd-Max centroid E|y_1| of one coordinate."""
    c = book(d, 2)
    c1, _ = oracle.codebook(d, 1)
    r = np.hypot(c[:, 0], c[:, 1])
    assert np.allclose(c[0], -c[1], atol=1e-12)
    assert np.allclose(r, c1[1], rtol=2e-3)


@pytest.mark.parametrize("d", [64, 128])
def test_four_codewords_are_the_product_square(d):
    """N = 4 (b = 1): Lloyd reaches a square at radius sqrt(2) c_1, a rotation
    of the 1-bit product code, so its error equals the scalar 1-bit one."""
    c = book(d, 4)
    c1, _ = oracle.codebook(d, 1)
    r = np.hypot(c[:, 0], c[:, 1])
    assert np.allclose(r, math.sqrt(2.0) * c1[1], rtol=2e-3)
    ang = np.sort(np.mod(np.arctan2(c[:, 1], c[:, 0]), 2 * math.pi))
    assert np.allclose(np.diff(ang), math.pi / 2, atol=1e-6)


@pytest.mark.parametrize("d", [64, 128])
def test_vector_code_beats_scalar_at_equal_rate(d):
    """The k = 2 code against the scalar Lloyd-Max table at the same rate,
    error per coordinate on an independent sphere sample: strictly lower at
    b = 2 and 3 (N = 16, 64), equal within sampling error at b = 1 (N = 4)."""
    y = source_sample(d, 200000, 100 + d)
    for bits, n in ((1, 4), (2, 16), (3, 64)):
        vq = d * F.block_mse(y, book(d, n)) / 2.0        # d E(y_i - q_i)^2
        c, _ = oracle.codebook(d, bits)
        sq = oracle.distortion(d, c)
        if bits == 1:
            assert vq == pytest.approx(sq, rel=5e-3)
        else:
            assert vq < 0.97 * sq, (bits, vq, sq)


@pytest.mark.parametrize("d,n", [(64, 16), (128, 32)])
def test_quadrature_error_matches_the_source(d, n):
    """The code's error measured on the quadrature agrees with its error on an
    independent sphere sample: the code is fitted to the quadrature points,
    which makes the quadrature figure optimistic by up to a few percent."""
    c = book(d, n)
    y = source_sample(d, 400000, 7 * d + n)
    e = np.sum((y - c[F.nearest(y, c)]) ** 2, axis=1)
    m_q = F.block_mse(F.quadrature(d), c)
    assert abs(np.mean(e) - m_q) <= 4.0 * np.std(e) / math.sqrt(len(e)) + 3e-2 * m_q


def signs_for(d, seed):
    return np.random.default_rng(seed).integers(0, 2, d).astype(bool)


@pytest.mark.parametrize("d,n", [(64, 8), (128, 32)])
def test_round_trip_error_is_the_block_error(d, n):
    """|x - decode(encode(x))|^2 = nu^2 sum_j |z_j - c[idx_j]|^2 (Pi is
    orthogonal), and for isotropic rows its mean over rows is (d/2) times the
    code's block error on the source (the quadrature figure, optimistic by up
    to a few percent)."""
    rng = np.random.default_rng(d + n)
    x = rng.standard_normal((4000, d)) * rng.uniform(0.1, 10.0, (4000, 1))
    sg = signs_for(d, 3)
    c = book(d, n)
    idx, nu, z = F.encode_vq(x, sg, c)
    xh = F.decode_vq(idx, nu, sg, c)
    lhs = np.sum((x - xh) ** 2, axis=1)
    rhs = nu ** 2 * np.sum((z.reshape(len(x), -1, 2) - c[idx]) ** 2, axis=(1, 2))
    assert np.allclose(lhs, rhs, rtol=1e-9)
    rel = lhs / nu ** 2
    want = d / 2.0 * F.block_mse(F.quadrature(d), c)
    assert abs(rel.mean() - want) <= 4.0 * rel.std() / math.sqrt(len(rel)) + 3e-2 * want


def test_codeword_frequencies_are_the_cell_masses():
    """On isotropic rows the blocks of Pi x / nu follow the canonical source,
    so codeword n is used with the mass of its cell."""
    d, n = 64, 8
    rng = np.random.default_rng(21)
    x = rng.standard_normal((20000, d))
    c = book(d, n)
    idx, _, _ = F.encode_vq(x, signs_for(d, 4), c)
    counts = np.bincount(idx.ravel(), minlength=n)
    mass = np.bincount(F.nearest(F.quadrature(d), c), minlength=n) / (F.QUAD_RINGS * F.QUAD_ANGLES)
    chi = sstats.chisquare(counts, mass * counts.sum())
    assert chi.pvalue > 1e-4, (counts, mass)


def test_zero_row_and_scale_invariance():
    """The zero row encodes as z = 0 (the codeword nearest the origin) and
    decodes to 0; scaling a row by alpha > 0 keeps its codes and scales nu."""
    d, n = 64, 16
    c = book(d, n)
    sg = signs_for(d, 9)
    idx, nu, z = F.encode_vq(np.zeros((1, d)), sg, c)
    assert nu[0] == 0 and np.all(z == 0)
    assert np.all(idx == np.argmin(np.sum(c * c, axis=1)))
    assert np.all(F.decode_vq(idx, nu, sg, c) == 0)
    x = np.random.default_rng(2).standard_normal((200, d))
    i1, n1, _ = F.encode_vq(x, sg, c)
    i2, n2, _ = F.encode_vq(4.0 * x, sg, c)      # a power of two: exact
    assert np.array_equal(i1, i2) and np.array_equal(4.0 * n1, n2)


@pytest.mark.parametrize("d,n", [(64, 2), (64, 8), (64, 32), (128, 128), (128, 256)])
def test_pack_round_trip_fixed_rate(d, n):
    rng = np.random.default_rng(n)
    idx = rng.integers(0, n, (9, d // 2))
    p = F.pack_vq(idx, n)
    assert p.shape == (9, d // 2 * int(math.log2(n)) // 8)
    assert np.array_equal(F.unpack_vq(p, d, n), idx)


def test_restart_keeps_the_first_on_rounding_ties():
    """At N = 2 the two restarts reach rotations of one code; the first
    (phase 0) is kept, so its first codeword is on the phase-0 side."""
    d = 64
    pts = F.quadrature(d)
    a = F.lloyd(F.spiral_init(d, 2, 0.0), pts)
    assert np.allclose(book(d, 2), a, atol=0)


def test_non_finite_row_codes_like_the_zero_row():
    """A row holding inf or NaN takes z = 0 (the zero row's codes) and
    keeps its non-finite norm."""
    d = 64
    code = F.fibquant_codebook(d, 16)
    rng = np.random.default_rng(6)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    x = rng.standard_normal((4, d))
    x[1, 5] = np.inf
    x[2, 0] = np.nan
    x[3] = 0.0
    idx, nu, z = F.encode_vq(x, signs, code)
    assert np.all(z[1:] == 0.0)
    assert np.array_equal(idx[1], idx[3]) and np.array_equal(idx[2], idx[3])
    assert np.isposinf(nu[1]) and np.isnan(nu[2]) and nu[3] == 0.0
    assert np.all(np.isfinite(z[0])) and nu[0] > 0
