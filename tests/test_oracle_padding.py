"""Pins of the oracle's reading for head dimensions that are not a power of two: the vector
is zero-padded to P, the next power of two, rotated at length P, all P codes are stored, and
the decode returns the first D reconstructed coordinates (oracle/rvq.py docstring; the pages'
fused kernel takes only powers of two, VeloxQuant-MLX blog, "rvq" tag page, "Wired in as a
fallback, not a replacement").

Each pin checks the oracle against something it does not compute itself: scipy's Hadamard
matrix, closed forms, a hand-derived one-hot example, and the power-of-two path (pinned by
the other oracle tests) on the explicitly padded vector.
"""
import math

import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import codebooks as cb
from oracle import packing, rvq

D_PAD = [24, 40, 80, 96, 192, 576, 9, 13, 100, 127, 1023]  # multiples of 8 and not


def _x(d, n, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, d)) * 1.5).astype(np.float16)


def _signs(d, seed):
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1, 1).astype(np.int8)


@pytest.mark.parametrize("d", D_PAD)
def test_rotation_is_scipy_hadamard_of_the_zero_padded_vector(d):
    p = cb.rotation_length(d)
    assert p > d and p & (p - 1) == 0 and p // 2 < d
    x, s = _x(d, 9, d), _signs(d, 100 + d)
    n, y = rvq.norms_and_rotation(x, s, p)
    assert y.shape == (9, p)
    xp = np.zeros((9, p))
    xp[:, :d] = x.astype(np.float64) * s.astype(np.float64)
    ref = (xp @ hadamard(p).T.astype(np.float64)) / (np.linalg.norm(x.astype(np.float64), axis=1) * math.sqrt(p))[:, None]
    assert np.array_equal(y, ref.astype(np.float32))
    assert np.allclose(n, np.linalg.norm(x.astype(np.float64), axis=1), rtol=1e-15)


@pytest.mark.parametrize("d", D_PAD)
def test_rotation_preserves_the_unit_norm(d):
    # a scale of 1/sqrt(D) instead of 1/sqrt(P) would give |y|^2 = P/D
    _, y = rvq.norms_and_rotation(_x(d, 50, 7 * d), _signs(d, d), cb.rotation_length(d))
    assert np.allclose(np.sum(y.astype(np.float64) ** 2, axis=1), 1.0, atol=1e-6)


@pytest.mark.parametrize("d", D_PAD)
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_tables_are_those_of_the_rotation_length(d, bits):
    t, tp = cb.build_tables(d, bits), cb.build_tables(cb.rotation_length(d), bits)
    assert t.d == d and t.p == tp.p == tp.d == cb.rotation_length(d)
    for a in ("c1", "b1", "c2", "b2"):
        assert np.array_equal(getattr(t, a), getattr(tp, a))
    assert t.sigma1 == 1.0 / math.sqrt(t.p)
    if bits == 1:  # closed form: the 1-bit Gaussian levels are +-sqrt(2/pi) sigma1
        assert np.allclose(t.c1, [-math.sqrt(2 / math.pi) * t.sigma1, math.sqrt(2 / math.pi) * t.sigma1], rtol=1e-7)


@pytest.mark.parametrize("d", D_PAD)
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_padded_encode_and_decode_are_those_of_the_padded_vector(d, bits):
    p = cb.rotation_length(d)
    x, s = _x(d, 33, 3 * d + bits), _signs(d, 17 + d)
    xp = np.zeros((33, p), np.float16)
    xp[:, :d] = x
    sp = np.ones(p, np.int8)
    sp[:d] = s
    t, tp = cb.build_tables(d, bits), cb.build_tables(p, bits)
    e, ep = rvq.encode(x, s, t), rvq.encode(xp, sp, tp)
    assert e["packed1"].shape == (33, packing.n_words(p, bits))
    for k in ("packed1", "packed2", "norms"):
        assert np.array_equal(e[k], ep[k]), k
    for norms in (None, e["norms"]):
        dec = rvq.decode(e["packed1"], e["packed2"], norms, s, t)
        decp = rvq.decode(ep["packed1"], ep["packed2"], norms, sp, tp)
        assert dec.shape == (33, d) and np.array_equal(dec, decp[:, :d])
    m = rvq.encode_mse(x, s, t)
    mp = rvq.encode_mse(xp, sp, tp)
    assert np.array_equal(m["packed"], mp["packed"])
    assert np.array_equal(rvq.decode_mse(m["packed"], m["norms"], s, t), rvq.decode_mse(mp["packed"], mp["norms"], sp, tp)[:, :d])


def test_one_hot_worked_example_d24_b2():
    """x = 3 e_5 at D = 24 (P = 32), signs +1, b = 2. By hand: |x| = 3, y_i = H32[i][5] / sqrt(32)
    = +-0.17678; sigma1 = 1/sqrt(32), so the stage-1 levels are +-0.45278 sigma1 = +-0.08004
    and +-1.51042 sigma1 = +-0.26701, with the boundary between them at 0.98160 sigma1 =
    0.17353 < 0.17678: code 3 where H32[i][5] = +1, code 0 where it is -1. The residual is
    -+0.09023; sigma2 = sqrt(0.11748) sigma1 = 0.06059 and the Laplace levels are
    +-0.41976 sigma2 = +-0.02543, +-1.83403 sigma2 = +-0.11112 with their boundary at 0.06828
    < 0.09023: stage-2 code 3 - code1. Decoding gives z = (0.26701 - 0.11112) H32[:, 5]
    = 0.15589 H32[:, 5], and H32 H32[:, 5] = 32 e_5, so the reconstruction is
    3 * sqrt(32) * 0.15589 e_5 = 2.6456 e_5 (zeros elsewhere)."""
    x = np.zeros((1, 24), np.float16)
    x[0, 5] = 3.0
    s = np.ones(24, np.int8)
    t = cb.build_tables(24, 2)
    e = rvq.encode(x, s, t)
    h5 = np.array([1 if bin(i & 5).count("1") % 2 == 0 else -1 for i in range(32)])
    i1 = np.where(h5 > 0, 3, 0)
    assert np.array_equal(packing.unpack(e["packed1"], 2, 32)[0], i1)
    assert np.array_equal(packing.unpack(e["packed2"], 2, 32)[0], 3 - i1)
    assert e["norms"][0] == np.float32(3.0)
    out = rvq.decode(e["packed1"], e["packed2"], e["norms"], s, t).astype(np.float64)[0]
    want = 3.0 * math.sqrt(32.0) * (float(t.c1[3]) + float(t.c2[0]))
    assert abs(want - 2.6456) < 2e-4
    assert out[5] == np.float64(np.float16(want)) and np.count_nonzero(out) == 1
