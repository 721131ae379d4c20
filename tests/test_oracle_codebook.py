"""Pins for the oracle's coordinate density and Lloyd-Max codebook.

Every check compares the oracle with something other than itself: a second
quadrature (scipy.integrate.quad), a closed form, the uniform special case,
an independent Gaussian Lloyd-Max, or values printed on the pages
("Eternal mathematics of TurboQuant": Lemma on coordinates, Step 2, Theorem 1).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle as O

HERE = os.path.dirname(__file__)
PAGE = json.load(open(os.path.join(HERE, "golden", "page_tables.json")))


@pytest.mark.parametrize("d", [3, 4, 8, 64, 128, 256])
def test_density_normalized_and_second_moment(d):
    f = lambda x: float(O.coord_density(d, x))
    pts = [-4.0 / math.sqrt(d), 0.0, 4.0 / math.sqrt(d)] if d > 16 else None
    total = integrate.quad(f, -1, 1, points=pts, epsabs=1e-14, epsrel=1e-13, limit=400)[0]
    m2 = integrate.quad(lambda x: x * x * f(x), -1, 1, points=pts, epsabs=1e-14, epsrel=1e-13, limit=400)[0]
    assert abs(total - 1.0) < 1e-10
    # a coordinate of a unit vector has E[x^2] = 1/d
    assert abs(m2 - 1.0 / d) < 1e-10 / d


def test_density_d3_is_uniform():
    xs = np.linspace(-0.99, 0.99, 7)
    assert np.allclose(O.coord_density(3, xs), 0.5, rtol=0, atol=1e-15)


def test_density_matches_sphere_sampling():
    # histogram of a coordinate of uniform points on S^{d-1} (normalized Gaussians)
    d = 16
    g = np.random.Generator(np.random.PCG64(7)).standard_normal((400000, d))
    x = g[:, 0] / np.linalg.norm(g, axis=1)
    edges = np.linspace(-0.8, 0.8, 17)
    hist, _ = np.histogram(x, bins=edges)
    mass = O.cell_mass(d, edges[:-1], edges[1:])
    expect = mass * x.size
    assert np.all(np.abs(hist - expect) < 5 * np.sqrt(expect) + 5)


@pytest.mark.parametrize("d", [8, 64, 128])
def test_cell_mass_and_moment_vs_quadrature(d):
    a, b = -0.05, 0.13
    f = lambda x: float(O.coord_density(d, x))
    m0 = integrate.quad(f, a, b, epsabs=1e-15, epsrel=1e-13)[0]
    m1 = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-15, epsrel=1e-13)[0]
    assert abs(float(O.cell_mass(d, a, b)) - m0) < 1e-13
    assert abs(float(O.cell_first_moment(d, a, b)) - m1) < 1e-13


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_uniform_special_case_d3(bits):
    # d = 3: f_X is uniform on [-1, 1], Lloyd-Max is the uniform quantizer with
    # centroids -1 + (2i+1)/K and distortion d * Delta^2 / 12 = 4^-b.
    c, cost, _ = O.lloyd_max(3, bits)
    K = 1 << bits
    expect = -1.0 + (2.0 * np.arange(K) + 1.0) / K
    assert np.allclose(c, expect, rtol=0, atol=1e-14)
    assert abs(3 * cost - 4.0 ** (-bits)) < 1e-14


@pytest.mark.parametrize("d", [8, 64, 128, 256, 1000])
def test_one_bit_closed_form(d):
    # b = 1: centroids are +- E|X| = +- Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)), D = 1 - d c^2
    c, cost, _ = O.lloyd_max(d, 1)
    cf = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c[1] - cf) < 1e-14 and abs(c[0] + cf) < 1e-14
    assert abs(d * cost - (1.0 - d * cf * cf)) < 1e-12


def test_gaussian_limit_centroids_match_page():
    # the page prints the large-d centroids: b=1 +-sqrt(2/(pi d)); b=2 +-0.453/sqrt(d), +-1.51/sqrt(d)
    d = 16384
    c1, _, _ = O.lloyd_max(d, 1)
    assert abs(math.sqrt(d) * c1[1] - PAGE["gaussian_limit_centroids_sqrt_d"]["1"][0]) < 1e-4
    c2, _, _ = O.lloyd_max(d, 2)
    lo, hi = PAGE["gaussian_limit_centroids_sqrt_d"]["2"]
    assert abs(math.sqrt(d) * c2[2] - lo) < 0.0006
    assert abs(math.sqrt(d) * c2[3] - hi) < 0.006


def _gaussian_lloyd_max(bits, iters=20000):
    """Independent Lloyd-Max for N(0,1): truncated-normal means via the pdf/cdf."""
    K = 1 << bits
    c = stats.norm.ppf((np.arange(K) + 0.5) / K)
    for _ in range(iters):
        t = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        mass = stats.norm.cdf(t[1:]) - stats.norm.cdf(t[:-1])
        c_new = (stats.norm.pdf(t[:-1]) - stats.norm.pdf(t[1:])) / mass
        if np.max(np.abs(c_new - c)) < 1e-14:
            c = c_new
            break
        c = c_new
    return c


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_large_d_approaches_gaussian_lloyd_max(bits):
    d = 8192
    c, _, _ = O.lloyd_max(d, bits)
    g = _gaussian_lloyd_max(bits)
    # f_X -> N(0, 1/d) with O(1/d) corrections
    assert np.allclose(math.sqrt(d) * c, g, rtol=2e-3, atol=2e-3)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_conditions_by_second_quadrature(d, bits):
    c, cost, _ = O.lloyd_max(d, bits)
    K = 1 << bits
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([-1.0], t, [1.0]))
    f = lambda x: float(O.coord_density(d, x))
    total_cost = 0.0
    s = 1.0 / math.sqrt(d)
    for i in range(K):
        a, b = edges[i], edges[i + 1]
        pts = [p for p in (-6 * s, 0.0, 6 * s) if a < p < b]
        m0 = integrate.quad(f, a, b, points=pts or None, epsabs=1e-16, epsrel=1e-13, limit=400)[0]
        m1 = integrate.quad(lambda x: x * f(x), a, b, points=pts or None, epsabs=1e-16, epsrel=1e-13, limit=400)[0]
        assert abs(m1 / m0 - c[i]) <= 1e-11 * max(abs(c[i]), s)       # centroid = conditional mean
        total_cost += integrate.quad(lambda x: (x - c[i]) ** 2 * f(x), a, b, points=pts or None,
                                     epsabs=1e-17, epsrel=1e-12, limit=400)[0]
    assert np.allclose(c, -c[::-1], rtol=0, atol=1e-14)                 # symmetric codebook
    cb = O.codebook(d, bits)
    assert np.array_equal(cb, -cb[::-1])                                 # exactly, once stored as fp32
    assert np.all(np.diff(c) > 0)
    assert abs(total_cost - cost) < 1e-11 * cost                        # the stated cost C(f_X, b)


def test_theorem1_table_and_bounds():
    # Theorem 1 table on the page, rounded; exact values stay within +-15 percent.
    for d in (64, 128, 256):
        for b in (1, 2, 3, 4):
            _, cost, _ = O.lloyd_max(d, b)
            D = d * cost
            printed = PAGE["d_mse"][str(b)]
            assert abs(D - printed) <= 0.15 * printed, (d, b, D, printed)
            # Shannon lower bound 4^-b (1 - O(1/d)) and the upper bound sqrt(3)*pi/2 * 4^-b
            assert D >= 4.0 ** (-b) * (1 - 2.0 / d)
            assert D <= (math.sqrt(3) * math.pi / 2) * 4.0 ** (-b)
            # "within about 2.7x of the theoretical minimum"
            assert D / 4.0 ** (-b) < 2.73


def test_panter_dite_constant_reading():
    # (1/12) (int f^{1/3})^3 * d -> sqrt(3) pi / 2 (the theorem constant, printed garbled)
    d = 4096
    s = 1 / math.sqrt(d)
    val = integrate.quad(lambda x: float(O.coord_density(d, x)) ** (1 / 3), -60 * s, 60 * s,
                         points=[0.0], limit=400, epsrel=1e-12)[0]
    pd = d * val ** 3 / 12.0
    assert abs(pd - math.sqrt(3) * math.pi / 2) < 2e-3


@pytest.mark.parametrize("d", [64, 128, 256])
def test_codebook_is_float32_rounding(d):
    for b in (1, 2, 3, 4):
        c64, _, _ = O.lloyd_max(d, b)
        cb = O.codebook(d, b)
        assert np.array_equal(cb, c64.astype(np.float32).astype(np.float64))
    assert np.array_equal(O.codebook(d, 0), [0.0])
