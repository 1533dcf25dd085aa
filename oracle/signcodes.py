"""1-bit sign-code encoders, written as plainly as possible (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

RaBitQ-style code ("rvq" tag page, "A fusion this codebase had already proven out": one
kernel rotates, binarizes with y >= 0, packs the sign bits and writes the magnitude), per
head vector x (fp16, length D):
    n = ||x||,  y = H diag(s) x / (n sqrt(D))  (the codec's rotation, rvq.py),
    bit i = [y_i >= 0]  (a zero vector has y = 0 and every bit set),
    bits packed LSB-first, 32 per uint32 word (packing.py with b = 1), n kept as float32.

QJL sketch ("turboquant" tag page, "Kernel 4: QJL Encode"), per key x with a sketch
matrix S [m, D] (fp16 here):
    bit j = [(S x)_j >= 0] for the exact value of (S x)_j,
    bits packed LSB-first (bit j of the sequence is sketch dimension j; the pages' byte k,
    bit i is bit 8k + i, the same bytes as uint32 words on a little-endian machine),
    the norm ||x|| rounded to fp16.
(S x)_j is a sum of products of fp16 values. Those products are exact in float64 but the
sum need not be, so every dot whose float64 value could carry the wrong sign (|value| at
most the float64 error bound of the sum) is recomputed exactly in integers: an fp16 value
is an integer multiple of 2**-24.
"""
from __future__ import annotations

import numpy as np

from . import packing
from .rvq import norms_and_rotation

CHUNK = 8192


def rabitq_encode(x16: np.ndarray, signs: np.ndarray) -> dict:
    """x16: float16 [N, D]; signs: +-1 [D]. Returns packed uint32 [N, ceil(D / 32)],
    norms float32 [N] and the rotated coordinates y (float32, as the decisions see them)."""
    x16 = np.asarray(x16, dtype=np.float16)
    if x16.ndim != 2:
        raise ValueError("x16 must be [N, D]")
    norm, y = norms_and_rotation(x16, signs)
    bits = (y >= 0).astype(np.uint8)  # -0.0 >= 0 holds, as in the definition
    return {"packed": packing.pack(bits, 1), "norms": norm.astype(np.float32), "norm64": norm, "y": y,
            "bits": bits}


def _exact_dot(xrow: np.ndarray, srow: np.ndarray) -> int:
    """2**48 (S_j . x) as an exact integer from float64 copies of fp16 values."""
    a = [int(v) for v in np.asarray(xrow, np.float64) * 2.0 ** 24]
    b = [int(v) for v in np.asarray(srow, np.float64) * 2.0 ** 24]
    return sum(p * q for p, q in zip(a, b))


def qjl_dots(x16: np.ndarray, sketch16: np.ndarray):
    """(dots, absdots, exact_sign) for x16 [N, D] and sketch16 [m, D]:
    dots = S x in float64 [N, m], absdots = sum_i |S_ji x_i| [N, m] (the scale of each
    dot's rounding error) and exact_sign in {-1, 0, +1} of the exact S x."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    S = np.asarray(sketch16, dtype=np.float16).astype(np.float64)
    if x.ndim != 2 or S.ndim != 2 or x.shape[1] != S.shape[1]:
        raise ValueError("x16 [N, D] and sketch16 [m, D] must share D")
    d = x.shape[1]
    dots = np.empty((x.shape[0], S.shape[0]))
    absdots = np.empty_like(dots)
    for a in range(0, x.shape[0], CHUNK):
        dots[a:a + CHUNK] = x[a:a + CHUNK] @ S.T
        absdots[a:a + CHUNK] = np.abs(x[a:a + CHUNK]) @ np.abs(S).T
    sign = np.sign(dots).astype(np.int8)
    # float64 sum of d exact products: |error| <= d * 2**-53 * sum|products| (any order)
    unsure = np.abs(dots) <= 2.0 * d * 2.0 ** -53 * absdots
    for i, j in zip(*np.nonzero(unsure)):
        e = _exact_dot(x[i], S[j])
        sign[i, j] = (e > 0) - (e < 0)
    return dots, absdots, sign


def qjl_encode(x16: np.ndarray, sketch16: np.ndarray) -> dict:
    """Packed sign sketch uint32 [N, m / 32] and fp16 norms [N] (see the module docstring)."""
    x16 = np.asarray(x16, dtype=np.float16)
    m = np.asarray(sketch16).shape[0]
    if m % 32:
        raise ValueError("m must be a multiple of 32 (whole words)")
    dots, absdots, sign = qjl_dots(x16, sketch16)
    bits = (sign >= 0).astype(np.uint8)
    x = x16.astype(np.float64)
    norm64 = np.sqrt(np.sum(x * x, axis=1))
    with np.errstate(over="ignore"):
        norms = norm64.astype(np.float16)  # one rounding from float64 (inf past 65504 + half a step)
    return {"packed": packing.pack(bits, 1), "norms": norms, "norm64": norm64, "dots": dots, "absdots": absdots,
            "bits": bits}
