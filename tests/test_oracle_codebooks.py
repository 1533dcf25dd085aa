"""Pins for the oracle's Lloyd-Max codebooks, against things the oracle does not compute.

* Gaussian levels, decisions and distortion: the textbook table of Max (1960)
  (tests/golden/lloyd_max_gaussian_max1960.json) and the 1-bit closed forms.
* Both densities: every level is the conditional mean of its cell, recomputed by
  numerical quadrature of the density (scipy.integrate.quad), and every decision is the
  midpoint of its neighbours (the pages' definition of a boundary: VeloxQuant-MLX blog,
  "rvq" tag page, "What 'quantize' means here, precisely").
* Laplace 1-bit: the closed form E|X| = beta.
* The stage-2 scale: MSE_G(b) against quadrature and a Monte Carlo estimate.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import codebooks as cb

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian_max1960.json")))


def _tol(v: float) -> float:
    # one unit in the last printed digit of the four-significant-digit table (the 1960
    # computation is not always correctly rounded in its last digit)
    digits = 4 - (int(math.floor(math.log10(abs(v)))) + 1)
    return 10.0 ** (-digits) + 1e-9


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_levels_match_max_1960(bits):
    g = GOLD["levels"][str(bits)]
    pos = cb.lloyd_max_positive_half(bits, "gauss")
    assert len(pos) == len(g["outputs"])
    for got, want in zip(pos, g["outputs"]):
        assert abs(got - want) <= _tol(want), (bits, got, want)
    dec = 0.5 * (pos[:-1] + pos[1:])
    for got, want in zip(dec, g["decisions"]):
        assert abs(got - want) <= _tol(want), (bits, got, want)
    assert abs(cb.gaussian_mse(pos) - g["mse"]) <= max(_tol(g["mse"]), 1e-5)


def test_one_bit_closed_forms():
    g = cb.lloyd_max_positive_half(1, "gauss")
    assert abs(g[0] - math.sqrt(2.0 / math.pi)) < 1e-14
    assert abs(cb.gaussian_mse(g) - (1.0 - 2.0 / math.pi)) < 1e-14
    lap = cb.lloyd_max_positive_half(1, "laplace")
    assert abs(lap[0] - 1.0 / math.sqrt(2.0)) < 1e-14  # E|X| = beta for unit variance


def _pdf(density):
    if density == "gauss":
        return stats.norm.pdf
    beta = 1.0 / math.sqrt(2.0)
    return lambda x: math.exp(-abs(x) / beta) / (2.0 * beta)


@pytest.mark.parametrize("density", ["gauss", "laplace"])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_levels_are_cell_centroids_by_quadrature(density, bits):
    pos = cb.lloyd_max_positive_half(bits, density)
    full = cb.full_codebook(pos)
    edges = np.concatenate(([-np.inf], 0.5 * (full[:-1] + full[1:]), [np.inf]))
    f = _pdf(density)
    total = 0.0
    for k, c in enumerate(full):
        a, b = edges[k], edges[k + 1]
        mass = integrate.quad(f, a, b, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        first = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        assert abs(first / mass - c) < 1e-9, (density, bits, k, first / mass, c)
        total += mass
    assert abs(total - 1.0) < 1e-10


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_mse_by_quadrature_and_monte_carlo(bits):
    pos = cb.lloyd_max_positive_half(bits, "gauss")
    full = cb.full_codebook(pos)
    edges = np.concatenate(([-np.inf], 0.5 * (full[:-1] + full[1:]), [np.inf]))
    q = sum(integrate.quad(lambda x, c=c: (x - c) ** 2 * stats.norm.pdf(x), a, b,
                           epsabs=1e-15, epsrel=1e-13, limit=200)[0]
            for a, b, c in zip(edges[:-1], edges[1:], full))
    assert abs(q - cb.gaussian_mse(pos)) < 1e-12
    # stage-1 distortion on 10**6 samples of N(0, 1/128) within 1% of MSE_G * sigma1^2
    t = cb.build_tables(128, bits)
    x = np.random.default_rng(7).standard_normal(1_000_000) * t.sigma1
    qx = full[np.searchsorted(edges[1:-1], x / t.sigma1)] * t.sigma1
    emp = np.mean((x - qx) ** 2)
    assert abs(emp / (t.mse_g * t.sigma1 ** 2) - 1.0) < 0.01


@pytest.mark.parametrize("d", [8, 16, 64, 128, 256, 1024])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_float32_tables(d, bits):
    t = cb.build_tables(d, bits)
    k = 1 << bits
    for c, b, sig in ((t.c1, t.b1, t.sigma1), (t.c2, t.b2, t.sigma2)):
        assert c.dtype == np.float32 and b.dtype == np.float32
        assert c.shape == (k,) and b.shape == (k - 1,)
        assert np.all(np.diff(c) > 0)
        assert np.array_equal(c, -c[::-1])  # exactly antisymmetric
        assert np.array_equal(b, -b[::-1])
        assert b[(k - 1) // 2] == 0.0 and not np.signbit(b[(k - 1) // 2])
        # boundaries are the float32-rounded exact midpoints of neighbouring levels
        mid = (c[:-1].astype(np.float64) + c[1:].astype(np.float64)) / 2.0
        assert np.array_equal(b, mid.astype(np.float32))
        assert np.all(c[:-1] < b) and np.all(b < c[1:])
    assert t.sigma1 == 1.0 / math.sqrt(d)
    assert abs(t.sigma2 ** 2 / (t.mse_g * t.sigma1 ** 2) - 1.0) < 1e-14
