"""Coordinate law after a random rotation, and its Lloyd-Max scalar codebook.

Test infrastructure only (see the package docstring).

Pages followed:
* AiBoss overview "TurboQuant - Googleのベクトル量子化アルゴリズム", section
  "TurboQuantの技術原理": after a random rotation every coordinate follows a
  Beta-shaped law and coordinates are nearly independent; an optimal scalar
  quantizer per coordinate is found once, ahead of time, by Lloyd-Max (a
  continuous one-dimensional k-means on that law).
* ai-navigate-news Gemma 4 post, section "仕組み（技術的）": Algorithm 1 is
  rotation, then Lloyd-Max scalar quantization of the Beta-distributed
  coordinates, then the inverse rotation.
* techblog-plum explainer, section "TurboQuantの仕組み", step 1: the buckets are
  precomputed once, so inference pays nothing for them.

Reading taken where the pages are silent: the law is that of one coordinate of
a point drawn uniformly on the unit sphere S^{d-1}, density
    f_d(u) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1-u^2)^((d-3)/2),  |u| <= 1,
i.e. (u+1)/2 ~ Beta((d-1)/2, (d-1)/2).  Its limit for large d is N(0, 1/d).
"""
from __future__ import annotations

import functools

import mpmath
import numpy as np
from scipy.special import betainc, ndtri
from scipy.stats import norm as _norm


@functools.lru_cache(maxsize=None)
def _log_norm_const(d: int) -> float:
    """log of Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)), the density's normalising constant.

    Evaluated with 50-digit log-gammas: in fp64 the difference of the two
    log-gammas loses up to 4e-11 of relative precision at d = 65536.
    """
    with mpmath.workdps(50):
        v = mpmath.loggamma(mpmath.mpf(d) / 2) - mpmath.loggamma(mpmath.mpf(d - 1) / 2) - mpmath.log(mpmath.pi) / 2
        return float(v)


def coord_density(u, d: int):
    """f_d(u), the density of one coordinate of a uniform point on S^{d-1}."""
    u = np.asarray(u, dtype=np.float64)
    out = np.zeros_like(u)
    inside = np.abs(u) < 1.0
    out[inside] = np.exp(_log_norm_const(d) + 0.5 * (d - 3) * np.log1p(-u[inside] ** 2))
    return out


def coord_tail(u, d: int):
    """P(U > u) for U ~ f_d, via the regularized incomplete beta function."""
    a = 0.5 * (d - 1)
    u = np.clip(np.asarray(u, dtype=np.float64), -1.0, 1.0)
    return betainc(a, a, 0.5 * (1.0 - u))


def _first_moment_between(lo, hi, d: int):
    """Integral of u f_d(u) over [lo, hi], closed form.

    d/du (1-u^2)^((d-1)/2) = -(d-1) u (1-u^2)^((d-3)/2), so the integral is
    C_d [ (1-lo^2)^((d-1)/2) - (1-hi^2)^((d-1)/2) ] / (d-1).
    """
    def pw(u):
        u = np.asarray(u, dtype=np.float64)
        r = np.zeros_like(u)
        m = np.abs(u) < 1.0
        r[m] = np.exp(0.5 * (d - 1) * np.log1p(-u[m] ** 2))
        return r
    return np.exp(_log_norm_const(d)) * (pw(lo) - pw(hi)) / (d - 1)


def lloyd_max(d: int, bits: int, max_iter: int = 20000):
    """Lloyd-Max quantizer for f_d with L = 2**bits cells.

    Returns (centroids[L] ascending, bounds[L-1]) in fp64, in the unit-sphere
    coordinate domain (a vector of norm n is compared against bounds * n).

    Steps, in the usual Lloyd-Max order:
      start from the Gaussian-limit quantiles c_k = Phi^{-1}((k+1/2)/L)/sqrt(d);
      repeat: boundaries are midpoints of neighbouring centroids, each centroid
      becomes the conditional mean of its cell; keep the codebook symmetric
      (c[L-1-k] = -c[k]); stop when the update falls to the fp64 floor.
    """
    if bits < 0:
        raise ValueError("bits must be >= 0")
    if bits == 0:
        # one cell, the whole interval: its conditional mean is the mean of the symmetric law.  This
        # is Algorithm 1 at 0 bits, the first stage of Algorithm 2 at b = 1 (the 1-bit mode of the
        # AiBoss overview, section "TurboQuantの主な機能": the sign of S x and the norm alone)
        return np.zeros(1), np.zeros(0)
    L = 1 << bits
    c = ndtri((np.arange(L) + 0.5) / L) / np.sqrt(d)
    for _ in range(max_iter):
        t = np.concatenate(([-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
        lo, hi = t[:-1], t[1:]
        mass = coord_tail(lo, d) - coord_tail(hi, d)
        new = _first_moment_between(lo, hi, d) / mass
        new = 0.5 * (new - new[::-1])
        step = np.max(np.abs(new - c))
        c = new
        if step <= 1e-16 * np.max(np.abs(c)):
            break
    return c, 0.5 * (c[:-1] + c[1:])


def gaussian_lloyd_max(bits: int, max_iter: int = 20000):
    """Lloyd-Max for the standard normal law (the large-d limit, scaled by sqrt(d)).

    Independent of lloyd_max(): it uses the normal pdf/cdf only.  Conditional
    mean of N(0,1) on [a, b] is (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
    """
    L = 1 << bits
    c = ndtri((np.arange(L) + 0.5) / L)
    for _ in range(max_iter):
        t = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        lo, hi = t[:-1], t[1:]
        mass = _norm.sf(lo) - _norm.sf(hi)
        new = (_norm.pdf(lo) - _norm.pdf(hi)) / mass
        new = 0.5 * (new - new[::-1])
        step = np.max(np.abs(new - c))
        c = new
        if step <= 1e-16 * np.max(np.abs(c)):
            break
    return c, 0.5 * (c[:-1] + c[1:])


def distortion(d: int, centroids, bounds) -> float:
    """Expected squared error of the scalar quantizer on one coordinate, times d.

    For a unit vector this is E||x - x_hat||^2 under Algorithm 1 with exact
    norms: d * sum_k integral over cell k of (u - c_k)^2 f_d(u) du, evaluated
    as d * (E[U^2] - sum_k c_k^2 P(cell k)) using that each c_k is its cell's
    conditional mean; E[U^2] = 1/d for the sphere law.
    """
    t = np.concatenate(([-1.0], np.asarray(bounds, dtype=np.float64), [1.0]))
    mass = coord_tail(t[:-1], d) - coord_tail(t[1:], d)
    return float(d * (1.0 / d - np.sum(np.asarray(centroids) ** 2 * mass)))
