"""Lloyd-Max scalar codebooks for the two RVQ stages (oracle side; test infrastructure).

What the pages fix (VeloxQuant-MLX blog):
  * "rvq" tag page, "The pipeline, as it actually runs": stage 1 quantizes the rotated
    coordinate against a Gaussian codebook, stage 2 quantizes the residual against a
    Laplacian-fit codebook; each stage has 2**b levels.
  * "rvq" tag page, "What 'quantize' means here, precisely": the boundaries are the
    midpoints of the sorted centroids.
  * "turboquant" tag page, "Kernel 2": the codebook is a Lloyd-Max codebook.
  * "kivi" tag page (second post), "Where KIVI fits": RVQ's codebooks are analytical and
    need no calibration data.

Readings taken where the pages are silent:
  * Stage 1 is the 2**b-level Lloyd-Max quantizer of N(0, sigma1**2) with sigma1**2 = 1/P,
    the per-coordinate variance of a rotated unit vector of P coordinates. P = D for a
    power-of-two head dimension; any other D in [8, 1024] is rotated zero-padded to the
    next power of two P (see rvq.py), so its tables are those of P.
  * Stage 2 is the 2**b-level Lloyd-Max quantizer of a zero-mean Laplace density whose
    variance equals the stage-1 mean squared error, sigma2**2 = MSE_G(b) * sigma1**2,
    where MSE_G(b) is the distortion of the unit-variance Gaussian Lloyd-Max quantizer.
  * Lloyd-Max iteration in float64 on the positive half of the (symmetric) density, from
    quantile starting points, until the centroids stop moving; the negative half is the
    mirror image, so the tables are exactly antisymmetric and the middle boundary is 0.
  * float32 tables: c32 = RN32(sigma * c_unit); boundary_k = RN32((c32_k + c32_{k+1}) / 2)
    with the midpoint taken in float64 (exact for two float32 values).

Conditional means used by the iteration (standard results):
  Gaussian, cell [a, b]:            (phi(a) - phi(b)) / (Phi(b) - Phi(a))
  Laplace of scale beta, 0<=a<b:    ((a+beta) e^{-a/beta} - (b+beta) e^{-b/beta})
                                     / (e^{-a/beta} - e^{-b/beta})
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy import special

_SQRT2PI = math.sqrt(2.0 * math.pi)


def _phi(x):
    return np.exp(-0.5 * x * x) / _SQRT2PI


def _gauss_cond_mean(lo, hi):
    """E[X | lo < X < hi] for X ~ N(0, 1), per cell; the last cell has hi = +inf."""
    out = np.empty_like(lo)
    fin = np.isfinite(hi)
    a, b = lo[fin], hi[fin]
    # cell mass as a difference of upper tails (0 <= a < b), better conditioned than
    # Phi(b) - Phi(a) far from the origin
    out[fin] = (_phi(a) - _phi(b)) / (special.ndtr(-a) - special.ndtr(-b))
    a = lo[~fin]
    out[~fin] = _phi(a) / special.ndtr(-a)
    return out


def _laplace_cond_mean(lo, hi, beta):
    """E[X | lo < X < hi] for Laplace(0, beta), 0 <= lo < hi; the last cell has hi = +inf."""
    out = np.empty_like(lo)
    fin = np.isfinite(hi)
    a, b = lo[fin], hi[fin]
    ea, eb = np.exp(-a / beta), np.exp(-b / beta)
    out[fin] = ((a + beta) * ea - (b + beta) * eb) / (ea - eb)
    out[~fin] = lo[~fin] + beta  # memoryless tail
    return out


def lloyd_max_positive_half(bits: int, density: str, max_iter: int = 100000, tol: float = 1e-15):
    """Positive-half centroids (ascending, float64) of the unit-variance Lloyd-Max quantizer.

    density is "gauss" (N(0, 1)) or "laplace" (Laplace with beta = 1/sqrt(2), variance 1).
    Returns an array of 2**(bits-1) positive centroids.
    """
    m = 1 << (bits - 1)
    beta = 1.0 / math.sqrt(2.0)
    # starting points: conditional medians of equal-probability cells on the positive half
    q = (np.arange(m) + 0.5) / m  # quantiles of |X|
    if density == "gauss":
        c = special.ndtri(0.5 + 0.5 * q)
    elif density == "laplace":
        c = -beta * np.log1p(-q)
    else:
        raise ValueError(density)
    for _ in range(max_iter):
        t = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        lo, hi = t[:-1], t[1:]
        if density == "gauss":
            c_new = _gauss_cond_mean(lo, hi)
        else:
            c_new = _laplace_cond_mean(lo, hi, beta)
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol:
            break
    return c


def full_codebook(pos: np.ndarray) -> np.ndarray:
    """Mirror the positive-half centroids into the full ascending codebook."""
    return np.concatenate((-pos[::-1], pos))


def gaussian_mse(pos: np.ndarray) -> float:
    """Distortion E[(X - Q(X))^2] of the unit Gaussian quantizer with these centroids.

    For a quantizer whose levels are the conditional means of their cells,
    E[(X - Q)^2] = E[X^2] - E[Q^2] = 1 - sum_k c_k^2 P_k.
    """
    t = np.concatenate(([0.0], 0.5 * (pos[:-1] + pos[1:]), [np.inf]))
    p = special.ndtr(t[1:]) - special.ndtr(t[:-1])  # probability of each positive cell
    return float(1.0 - 2.0 * np.sum(pos * pos * p))


@dataclass(frozen=True)
class Tables:
    d: int  # head dimension: coordinates of an input and of a reconstruction
    bits: int
    sigma1: float
    sigma2: float
    mse_g: float
    c1: np.ndarray  # float32 [2**bits], ascending
    b1: np.ndarray  # float32 [2**bits - 1]
    c2: np.ndarray
    b2: np.ndarray
    p: int = 0  # rotation length: the power of two >= d (the number of codes per vector)


def midpoints32(c32: np.ndarray) -> np.ndarray:
    """float32 boundaries: RN32 of the exact midpoint of neighbouring float32 centroids."""
    c = c32.astype(np.float64)
    return (0.5 * (c[:-1] + c[1:])).astype(np.float32)


def rotation_length(d: int) -> int:
    """The power of two >= d: the length of the Hadamard rotation (d itself when d is one)."""
    p = 1
    while p < d:
        p *= 2
    return p


def build_tables(d: int, bits: int) -> Tables:
    """Both stages' float32 centroid and boundary tables for head dimension d (rotated at
    length P = rotation_length(d))."""
    if bits < 1 or bits > 4:
        raise ValueError("bits must be in 1..4")
    g = lloyd_max_positive_half(bits, "gauss")
    lap = lloyd_max_positive_half(bits, "laplace")
    mse = gaussian_mse(g)
    P = rotation_length(d)
    sigma1 = 1.0 / math.sqrt(P)
    sigma2 = math.sqrt(mse) * sigma1
    c1 = (sigma1 * full_codebook(g)).astype(np.float32)
    c2 = (sigma2 * full_codebook(lap)).astype(np.float32)
    return Tables(d, bits, sigma1, sigma2, mse, c1, midpoints32(c1), c2, midpoints32(c2), P)
