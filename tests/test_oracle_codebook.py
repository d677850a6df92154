"""Pins for the oracle's coordinate law and Lloyd-Max codebook.

Each check ties the oracle to something other than itself: closed forms
(d = 3 uniform law, b = 1 centroids, E[U^2] = 1/d), an independent numerical
integrator (scipy quad), a textbook table (Max 1960 Gaussian quantizer) and
the figures printed on the pages (tests/golden/page_figures.json).
"""
import json
import math
import os

import numpy as np
import pytest
import mpmath
from scipy.integrate import quad

import oracle
from oracle.codebook import distortion

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _quad(f, a, b):
    return quad(f, a, b, epsabs=0, epsrel=1e-13, limit=400)[0]


@pytest.mark.parametrize("d", [3, 8, 128, 1536])
def test_density_normalised_and_second_moment(d):
    # a point uniform on S^{d-1} has E[u_j^2] = 1/d (the d squares sum to 1)
    sd = 1 / math.sqrt(d)
    lim = min(1.0, 40 * sd)
    f = lambda u: oracle.coord_density(np.array([u]), d)[0]
    assert _quad(f, -lim, lim) == pytest.approx(1.0, abs=1e-11)
    assert _quad(lambda u: u * u * f(u), -lim, lim) == pytest.approx(1.0 / d, rel=1e-10)


def test_d3_density_is_uniform():
    # Archimedes: one coordinate of a uniform point on the 2-sphere is uniform on [-1, 1]
    u = np.linspace(-0.99, 0.99, 41)
    assert np.allclose(oracle.coord_density(u, 3), 0.5, rtol=0, atol=1e-15)
    assert np.allclose(oracle.coord_tail(u, 3), (1 - u) / 2, rtol=0, atol=1e-15)


@pytest.mark.parametrize("d", [4, 128, 1536])
def test_tail_matches_integral(d):
    f = lambda u: oracle.coord_density(np.array([u]), d)[0]
    for u in [-0.3, -0.05, 0.0, 0.01, 0.07, 0.2]:
        if abs(u) * math.sqrt(d) > 8:
            continue
        assert oracle.coord_tail(np.array([u]), d)[0] == pytest.approx(_quad(f, u, 1.0), rel=1e-10, abs=1e-15)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_d3_lloyd_max_is_uniform_quantizer(bits):
    # for the uniform law on [-1, 1] the optimal L-level quantizer is the uniform one
    L = 1 << bits
    c, t = oracle.lloyd_max(3, bits)
    assert np.allclose(c, -1 + (2 * np.arange(L) + 1) / L, atol=1e-12)
    assert np.allclose(t, -1 + 2 * np.arange(1, L) / L, atol=1e-12)


@pytest.mark.parametrize("d", [3, 4, 128, 256, 512, 1536])
def test_one_bit_centroid_closed_form(d):
    # b = 1: boundary 0, centroid E[U | U > 0] = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    c, t = oracle.lloyd_max(d, 1)
    with mpmath.workdps(40):
        expect = float(mpmath.gamma(mpmath.mpf(d) / 2) / (mpmath.sqrt(mpmath.pi) * mpmath.gamma(mpmath.mpf(d + 1) / 2)))
    assert t[0] == 0.0
    assert c[1] == pytest.approx(expect, rel=2e-15)
    assert c[0] == -c[1]


def test_one_bit_centroid_gaussian_limit():
    # -> sqrt(2/(pi d)) for large d
    d = 200000
    c, _ = oracle.lloyd_max(d, 1)
    assert c[1] * math.sqrt(d) == pytest.approx(math.sqrt(2 / math.pi), rel=1e-5)


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3), (128, 4), (256, 3), (512, 2), (1536, 3), (1536, 4)])
def test_lloyd_max_optimality_conditions(d, bits):
    """Centroid = conditional mean of its cell (independent quadrature), boundary = midpoint, symmetry."""
    c, t = oracle.lloyd_max(d, bits)
    L = 1 << bits
    assert np.all(np.diff(c) > 0)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-17)
    assert np.array_equal(c, -c[::-1])
    assert t[L // 2 - 1] == 0.0
    f = lambda u: oracle.coord_density(np.array([u]), d)[0]
    edges = np.concatenate(([-1.0], t, [1.0]))
    sd = 1 / math.sqrt(d)
    for k in range(L // 2, L):  # positive half (the negative half is the mirror)
        lo, hi = edges[k], min(edges[k + 1], 40 * sd)
        m0 = _quad(f, lo, hi)
        m1 = _quad(lambda u: u * f(u), lo, hi)
        assert c[k] == pytest.approx(m1 / m0, rel=1e-10)


def test_gaussian_lloyd_max_matches_textbook_table():
    tab = json.load(open(os.path.join(GOLDEN, "gaussian_lloyd_max_textbook.json")))
    for b, levels in tab["levels"].items():
        c, _ = oracle.gaussian_lloyd_max(int(b))
        pos = c[len(c) // 2:]
        assert np.allclose(pos, levels, atol=tab["tolerance"]), (b, pos, levels)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_sphere_codebook_tends_to_gaussian(bits):
    d = 100000
    c, _ = oracle.lloyd_max(d, bits)
    g, _ = oracle.gaussian_lloyd_max(bits)
    assert np.allclose(c * math.sqrt(d), g, rtol=2e-4)


@pytest.mark.parametrize("d", [128, 1536])
def test_distortion_by_quadrature_and_bound(d):
    """D(b) = E||x - x~||^2 for unit x: quadrature of (u - c_k)^2 over each cell, times d.

    Pins: D(1) = 1 - d c^2 (closed form); D(b) <= (sqrt(3) pi / 2) 4^-b; the
    b = 1 ratio to 4^-1 and the bound factor reproduce the printed figures.
    """
    figs = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    f = lambda u: oracle.coord_density(np.array([u]), d)[0]
    sd = 1 / math.sqrt(d)
    for bits in [1, 2, 3, 4]:
        c, t = oracle.lloyd_max(d, bits)
        edges = np.concatenate(([-1.0], t, [1.0]))
        D = 0.0
        for k in range(len(c)):
            lo, hi = max(edges[k], -40 * sd), min(edges[k + 1], 40 * sd)
            D += _quad(lambda u: (u - c[k]) ** 2 * f(u), lo, hi)
        D *= d
        assert D == pytest.approx(distortion(d, c, t), rel=1e-9)
        assert D <= math.sqrt(3) * math.pi / 2 * 4.0 ** -bits
        if bits == 1:
            assert D == pytest.approx(1 - d * c[1] ** 2, rel=1e-10)
    assert round(math.sqrt(3) * math.pi / 2, 1) == figs["distortion_bound_factor"]["value"]


def test_one_bit_ratio_page_figure():
    figs = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    d = 200000
    c, t = oracle.lloyd_max(d, 1)
    ratio = distortion(d, c, t) / 0.25
    assert ratio == pytest.approx(4 * (1 - 2 / math.pi), rel=1e-4)
    assert round(ratio, 2) == figs["one_bit_distortion_over_bound"]["value"]


def test_survey_d128_values():
    # values recomputed independently while surveying the method (d = 128)
    c1, _ = oracle.lloyd_max(128, 1)
    assert c1[1] == pytest.approx(0.07066157, abs=5e-9)
    for bits, D in [(2, 0.116000), (3, 0.033966), (4, 0.009315)]:
        c, t = oracle.lloyd_max(128, bits)
        assert distortion(128, c, t) == pytest.approx(D, abs=2e-6)
