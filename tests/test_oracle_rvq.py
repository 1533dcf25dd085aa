"""Pins for the oracle's rotation, quantizer, packing, encode and decode.

Each pin checks the oracle against something it does not itself compute:
  * rotation: H H = D I in integers; H equals scipy.linalg.hadamard (Sylvester order) and
    the in-place range butterfly described on the VeloxQuant-MLX blog ("turboquant" tag
    page, "Kernel 3"); norm preservation; closed-form images of basis and constant vectors;
  * quantizer: counting boundary crossings ("rvq" tag page, "What 'quantize' means here,
    precisely") equals the oracle's nearest-centroid argmin, by brute force over many
    values, except inside the half-ulp gap between an exact midpoint and its float32
    rounding;
  * packing: hand-computed words ("rvq" tag page, "The kernel": LSB-first), round trips,
    zero padding;
  * encode/decode: the hand-derived worked examples in tests/golden/worked_examples.json;
  * decode inverts the rotation exactly on unquantized data;
  * reconstruction quality: a loose statistical band only (parity unpinned: the pages
    give no distortion figure for this codec).
A final group plants plausible mistakes in the oracle and checks a pin catches each.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
from scipy import integrate

from oracle import codebooks as cb
from oracle import packing, rvq

EX = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))["cases"]


# ------------------------------------------------------------------------------ rotation

@pytest.mark.parametrize("d", [1, 2, 8, 16, 128, 1024])
def test_hadamard_is_sylvester(d):
    H = rvq.hadamard(d)
    assert np.array_equal(H, scipy.linalg.hadamard(d).astype(np.float64))
    Hi = H.astype(np.int64)
    assert np.array_equal(Hi @ Hi, d * np.eye(d, dtype=np.int64))
    assert np.array_equal(H, H.T)


def _butterfly(v):
    """In-place WHT in the range form: for stride 1, 2, 4, ... each element's partner is
    stride away inside its 2*stride block; the lower one becomes the sum and the upper one
    the lower minus the upper, both read from the previous pass."""
    v = list(v)
    d = len(v)
    stride = 1
    while stride < d:
        prev = v[:]
        for lane in range(d):
            upper = (lane % (2 * stride)) >= stride
            if upper:
                v[lane] = prev[lane - stride] - prev[lane]
            else:
                v[lane] = prev[lane] + prev[lane + stride]
        stride *= 2
    return v


@pytest.mark.parametrize("d", [2, 8, 32])
def test_matrix_equals_range_butterfly(d):
    H = rvq.hadamard(d)
    rng = np.random.default_rng(d)
    for _ in range(5):
        x = rng.integers(-100, 100, size=d)
        assert np.array_equal(H.astype(np.int64) @ x, np.array(_butterfly(x.tolist())))


@pytest.mark.parametrize("d", [8, 128, 1024])
def test_rotation_preserves_norm_and_closed_forms(d):
    rng = np.random.default_rng(3)
    s = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
    x = rng.standard_normal((64, d)).astype(np.float16)
    norm, y = rvq.norms_and_rotation(x, s)
    assert np.all(np.abs(np.linalg.norm(y.astype(np.float64), axis=1) - 1.0) < 1e-5)
    # basis vector j: y = s_j * column j / sqrt(D)
    for j in (0, 1, d // 2 + 1, d - 1):
        e = np.zeros((1, d), np.float16)
        e[0, j] = 2.0
        n_e, y_e = rvq.norms_and_rotation(e, s)
        want = (s[j] * rvq.hadamard(d)[:, j] / math.sqrt(d)).astype(np.float32)
        assert n_e[0] == 2.0 and np.array_equal(y_e[0], want)
    # constant vector with s = +1 maps to e0
    ones = np.ones((1, d), np.float16)
    _, y1 = rvq.norms_and_rotation(ones, np.ones(d, np.int8))
    assert y1[0, 0] == 1.0 and np.all(y1[0, 1:] == 0.0)
    # zero vector: norm 0, y = 0
    nz, yz = rvq.norms_and_rotation(np.zeros((1, d), np.float16), s)
    assert nz[0] == 0.0 and np.all(yz == 0.0)


# ------------------------------------------------------------------------------ quantizer

def _count(v32, b32):
    return np.sum(v32.astype(np.float32)[..., None] > b32.astype(np.float32), axis=-1)


@pytest.mark.parametrize("d", [8, 128])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_boundary_count_equals_nearest_centroid(d, bits):
    t = cb.build_tables(d, bits)
    rng = np.random.default_rng(bits * 1000 + d)
    for c, b, sig in ((t.c1, t.b1, t.sigma1), (t.c2, t.b2, t.sigma2)):
        vals = [np.float32(0.0), np.float32(-0.0), np.float32(10 * sig), np.float32(-10 * sig)]
        for bk in b:
            vals += [bk, np.nextafter(bk, np.float32(np.inf)), np.nextafter(bk, np.float32(-np.inf))]
        vals += list(c)
        v = np.concatenate([np.array(vals, np.float32),
                            (rng.standard_normal(200_000) * 2 * sig).astype(np.float32)])
        got_argmin = rvq.nearest(v, c).astype(np.int64)
        got_count = _count(v, b)
        diff = got_argmin != got_count
        if diff.any():
            # allowed only between the exact midpoint and its float32 rounding
            mid = (c[:-1].astype(np.float64) + c[1:].astype(np.float64)) / 2.0
            for vi, ia, ic in zip(v[diff], got_argmin[diff], got_count[diff]):
                k = min(ia, ic)
                assert abs(ia - ic) == 1
                lo, hi = sorted((mid[k], float(b[k])))
                assert lo <= float(vi) <= hi, (vi, ia, ic, mid[k], b[k])


def test_nearest_first_minimum_wins():
    c = np.array([-1.0, -0.25, 0.25, 1.0], np.float32)
    assert rvq.nearest(np.array([0.0, -0.625, 0.625], np.float32), c).tolist() == [1, 0, 2]


# ------------------------------------------------------------------------------ packing

def test_packing_hand_computed_words():
    # b=2: codes 1,2,3,0 then zeros -> 1 | 2<<2 | 3<<4 = 57
    assert packing.pack(np.array([[1, 2, 3, 0] + [0] * 12]), 2).tolist() == [[57]]
    # b=1, D=40: two words, bit j of word j//32; codes 1 at j = 0, 31, 32, 39
    codes = np.zeros((1, 40), np.uint8)
    codes[0, [0, 31, 32, 39]] = 1
    assert packing.pack(codes, 1).tolist() == [[0x80000001, 0x81]]
    # b=3, D=12: ten codes per word, top two bits zero; second word holds codes 10, 11
    codes = np.array([[7, 1, 0, 0, 0, 0, 0, 0, 0, 7, 5, 2]])
    assert packing.pack(codes, 3).tolist() == [[7 | (1 << 3) | (7 << 27), 5 | (2 << 3)]]
    # b=4: eight codes per word, nibble j holds code j
    assert packing.pack(np.array([list(range(8))]), 4).tolist() == [[0x76543210]]


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [8, 16, 40, 128, 1024])
def test_packing_round_trip_and_padding(bits, d):
    rng = np.random.default_rng(bits + d)
    for codes in (rng.integers(0, 1 << bits, size=(7, d)),
                  np.zeros((2, d), np.int64),
                  np.full((2, d), (1 << bits) - 1)):
        w = packing.pack(codes, bits)
        assert w.dtype == np.uint32 and w.shape[-1] == packing.n_words(d, bits)
        assert np.array_equal(packing.unpack(w, bits, d), codes)
        assert np.all((w & packing.padding_mask(d, bits)) == 0)
    assert packing.n_words(128, 1) == 4 and packing.n_words(128, 2) == 8
    assert packing.n_words(128, 3) == 13 and packing.n_words(128, 4) == 16


# ------------------------------------------------------------------------------ worked examples

@pytest.mark.parametrize("case", EX, ids=[c["name"] for c in EX])
def test_worked_example_encode(case):
    t = cb.build_tables(case["D"], case["bits"])
    x = np.array([case["x"]], np.float16)
    s = np.array(case["signs"], np.int8)
    out = rvq.encode(x, s, t)
    assert out["i1"][0].tolist() == case["codes1"]
    assert out["i2"][0].tolist() == case["codes2"]
    assert out["packed1"][0].tolist() == case["packed1"]
    assert out["packed2"][0].tolist() == case["packed2"]
    assert out["norms"][0] == np.float32(case["norm"])


@pytest.mark.parametrize("case", [c for c in EX if c["decoded_unit"] is not None],
                         ids=[c["name"] for c in EX if c["decoded_unit"] is not None])
def test_worked_example_decode(case):
    t = cb.build_tables(case["D"], case["bits"])
    s = np.array(case["signs"], np.int8)
    p1 = np.array([case["packed1"]], np.uint32)
    p2 = np.array([case["packed2"]], np.uint32)
    unit = rvq.decode(p1, p2, None, s, t).astype(np.float64)[0]
    assert np.all(np.abs(unit - np.array(case["decoded_unit"])) < 5e-4)
    scaled = rvq.decode(p1, p2, np.array([case["norm"]], np.float32), s, t).astype(np.float64)[0]
    assert np.all(np.abs(scaled - case["norm"] * np.array(case["decoded_unit"])) < 5e-4 * max(1.0, case["norm"]))


@pytest.mark.parametrize("d", [8, 128])
def test_decode_inverts_rotation(d):
    """With the quantization taken out (z = y exactly) decode returns x / ||x||."""
    rng = np.random.default_rng(11)
    s = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
    x = rng.standard_normal((16, d)).astype(np.float16)
    norm, y = rvq.norms_and_rotation(x, s)
    H = rvq.hadamard(d)
    u_hat = (y.astype(np.float64) @ H.T) / math.sqrt(d) * s[None, :]
    u = x.astype(np.float64) / norm[:, None]
    assert np.max(np.abs(u_hat - u)) < 1e-6


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_reconstruction_quality_band(bits):
    """Parity unpinned: only a loose band around MSE_G(b) * MSE_L(b) per unit vector."""
    d = 128
    t = cb.build_tables(d, bits)
    rng = np.random.default_rng(5)
    s = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
    x = rng.standard_normal((2048, d)).astype(np.float16)
    enc = rvq.encode(x, s, t)
    rec = rvq.decode(enc["packed1"], enc["packed2"], None, s, t).astype(np.float64)
    u = x.astype(np.float64) / enc["norm64"][:, None]
    err = np.mean(np.sum((rec - u) ** 2, axis=1))
    lap = cb.full_codebook(cb.lloyd_max_positive_half(bits, "laplace"))
    beta = 1 / math.sqrt(2)
    edges = np.concatenate(([-np.inf], 0.5 * (lap[:-1] + lap[1:]), [np.inf]))
    mse_l = sum(integrate.quad(lambda v, c=c: (v - c) ** 2 * math.exp(-abs(v) / beta) / (2 * beta), a, b)[0]
                for a, b, c in zip(edges[:-1], edges[1:], lap))
    model = t.mse_g * mse_l
    assert 0.4 * model < err < 2.5 * model, (err, model)


# ------------------------------------------------------------------------------ planted mistakes

def _sign_after_h(x16, signs, p=0):
    x = np.asarray(x16, np.float16).astype(np.float64)
    d = x.shape[1]
    n = np.sqrt(np.sum(x * x, axis=1))
    u = np.where((n > 0)[:, None], x / np.where(n > 0, n, 1)[:, None], 0.0)
    y = (u @ rvq.hadamard(d).T) / math.sqrt(d) * np.asarray(signs, np.float64)[None, :]
    return n, y.astype(np.float32)


def _last_minimum(v32, c32):
    dist = np.abs(v32.astype(np.float64)[..., None] - c32.astype(np.float64))
    return (dist.shape[-1] - 1 - np.argmin(dist[..., ::-1], axis=-1)).astype(np.uint8)


def _msb_first_pack(codes, bits):
    codes = np.asarray(codes)
    d = codes.shape[-1]
    epw = 32 // bits
    out = np.zeros(codes.shape[:-1] + (packing.n_words(d, bits),), np.uint64)
    for j in range(d):
        w, k = divmod(j, epw)
        out[..., w] |= codes[..., j].astype(np.uint64) << np.uint64(32 - (k + 1) * bits)
    return out.astype(np.uint32)


def _flipped_residual(y32, t):
    i1 = rvq.nearest(y32, t.c1)
    r = (t.c1[i1] - y32).astype(np.float32)
    return i1, r, rvq.nearest(r, t.c2)


def _all_examples_pass():
    for case in EX:
        t = cb.build_tables(case["D"], case["bits"])
        out = rvq.encode(np.array([case["x"]], np.float16), np.array(case["signs"], np.int8), t)
        if (out["packed1"][0].tolist() != case["packed1"]
                or out["packed2"][0].tolist() != case["packed2"]):
            return False
    return True


@pytest.mark.parametrize("target,replacement", [
    ("norms_and_rotation", _sign_after_h),
    ("nearest", _last_minimum),
    ("quantize_two_stage", _flipped_residual),
])
def test_planted_oracle_mistakes_are_caught(monkeypatch, target, replacement):
    assert _all_examples_pass()
    monkeypatch.setattr(rvq, target, replacement)
    assert not _all_examples_pass()


def test_planted_packing_and_scale_mistakes_are_caught(monkeypatch):
    monkeypatch.setattr(packing, "pack", _msb_first_pack)
    assert not _all_examples_pass()
    monkeypatch.undo()
    real = cb.build_tables

    def same_scale(d, bits):  # stage 2 at the stage-1 scale
        t = real(d, bits)
        lap = cb.full_codebook(cb.lloyd_max_positive_half(bits, "laplace"))
        c2 = (t.sigma1 * lap).astype(np.float32)
        return cb.Tables(t.d, t.bits, t.sigma1, t.sigma1, t.mse_g, t.c1, t.b1, c2, cb.midpoints32(c2), t.p)
    monkeypatch.setattr(cb, "build_tables", same_scale)
    assert not _all_examples_pass()
