"""Pins of the oracle's single-stage codec (encode_mse / decode_mse) against results it does
not compute itself.

  * the hand-derived stage-1 codes and packed words of the worked examples
    (tests/golden/worked_examples.json; the single-stage codes are the first stage);
  * closed forms of the decode: a constant code vector rotates back onto e_0
    (H 1 = D e_0), and changing one code adds a scaled Hadamard column, with the
    Hadamard matrix taken from scipy rather than from the oracle;
  * the reconstruction error of unit vectors against the Gaussian Lloyd-Max distortion
    MSE_G(b) of the Max (1960) tables: each rotated coordinate of a random unit vector is
    close to N(0, 1/D), so the mean squared error of the whole vector is close to MSE_G(b);
  * a planted mistake (decoding with the stage-2 table) must break that pin.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import codebooks as cbk
from oracle import flips, packing, rvq

EX = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))["cases"]
MAX1960 = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian_max1960.json")))


@pytest.mark.parametrize("case", EX, ids=[c["name"] for c in EX])
def test_worked_examples_first_stage(case):
    t = cbk.build_tables(case["D"], case["bits"])
    out = rvq.encode_mse(np.array([case["x"]], np.float16), np.array(case["signs"], np.int8), t)
    assert out["i1"][0].tolist() == case["codes1"]
    assert out["packed"][0].tolist() == case["packed1"]
    assert out["norms"][0] == np.float32(case["norm"])


@pytest.mark.parametrize("d", [8, 64, 256])
@pytest.mark.parametrize("bits", [1, 2, 4])
def test_decode_constant_codes_and_one_change(d, bits):
    t = cbk.build_tables(d, bits)
    rng = np.random.default_rng(d + bits)
    s = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
    k, k2, j = (1 << bits) - 1, 0, d // 3
    codes = np.full((2, d), k, np.uint8)
    codes[1, j] = k2
    got = rvq.decode_mse(packing.pack(codes, bits), None, s, t).astype(np.float64)
    c, c2 = float(t.c1[k]), float(t.c1[k2])
    # constant codes: z = c 1, H z = D c e_0
    want0 = np.zeros(d)
    want0[0] = s[0] * c * math.sqrt(d)
    # one changed code: plus (c2 - c) H[:, j] / sqrt(D), signs applied
    Hs = scipy.linalg.hadamard(d).astype(np.float64)
    want1 = want0 + s * (c2 - c) * Hs[:, j] / math.sqrt(d)
    for got_row, want in ((got[0], want0), (got[1], want1)):
        assert np.max(np.abs(got_row - want) / np.maximum(np.abs(want), 2.0 ** -14)) <= 2.0 ** -10


def _mse_unit(bits: int, table: str = "c1") -> float:
    d, n = 128, 4000
    t = cbk.build_tables(d, bits)
    rng = np.random.default_rng(100 + bits)
    s = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
    x = rng.standard_normal((n, d)).astype(np.float16)
    out = rvq.encode_mse(x, s, t)
    if table == "c1":
        xh = rvq.decode_mse(out["packed"], None, s, t)
    else:  # planted mistake: dequantize from the stage-2 table
        i1 = packing.unpack(out["packed"], bits, d)
        z = t.c2[i1].astype(np.float32)
        xh = rvq._unrotate(z, None, s, d)
    u = x.astype(np.float64) / np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True)
    return float(np.mean(np.sum((u - xh.astype(np.float64)) ** 2, axis=1)))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_unit_vector_error_matches_max_1960_distortion(bits):
    want = MAX1960["levels"][str(bits)]["mse"]
    got = _mse_unit(bits)
    assert abs(got / want - 1.0) < 0.05, (got, want)


def test_planted_stage2_table_breaks_the_distortion_pin():
    want = MAX1960["levels"]["2"]["mse"]
    assert abs(_mse_unit(2, table="c2") / want - 1.0) > 0.5


def test_single_stage_comparison_rule():
    """The comparison accepts an identical stream and rejects a far-from-boundary change."""
    d, bits = 16, 2
    t = cbk.build_tables(d, bits)
    s = np.ones(d, np.int8)
    x = np.random.default_rng(3).standard_normal((4, d)).astype(np.float16)
    ref = rvq.encode_mse(x, s, t)
    rep = flips.compare_encode_single(ref["packed"].copy(), ref["norms"], ref, t)
    assert rep.ok(0.0, 1e-6) and rep.n_codes == 4 * d
    codes = ref["i1"].copy()
    far = np.argmax(np.abs(ref["y"]).ravel())
    codes.ravel()[far] ^= 1
    bad = flips.compare_encode_single(packing.pack(codes, bits), ref["norms"], ref, t)
    assert bad.bad_stage1 == 1 and not bad.ok(1.0, 1e-6)
