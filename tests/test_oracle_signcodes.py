"""Pins of the oracle's 1-bit sign-code encoders (oracle/signcodes.py) against results it
does not compute itself.

RaBitQ-style code (bit j = [y_j >= 0] of the rotated vector):
  * one-hot inputs: y is a signed, scaled Hadamard column, taken here from scipy;
  * a hand-derived D = 8 example with exact zeros in y (bits and packed word);
  * the zero vector sets every bit (y = 0 >= 0);
  * planted mistakes (strict > instead of >=, signs applied after H) break a pin.
QJL sketch (bit j = [(S x)_j >= 0], fp16 norm):
  * exact signs by brute force in rational arithmetic (fractions.Fraction) on small
    random inputs, and on cancellations that float64 gets wrong;
  * identity and shifted-identity sketches: bit j is the sign of x_j (x_{j+1}), with the
    packed word derived by hand;
  * the sign-random-projection law: for Gaussian rows the probability that the bits of x
    and y differ is angle(x, y) / pi (Goemans and Williamson 1995; Charikar 2002);
  * norms: closed forms and fp16 rounding of sqrt(2) and of overflow;
  * planted mistakes (strict >, a transposed sketch, MSB-first packing) break a pin.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import synth
from oracle import packing, rvq, signcodes


# ----------------------------------------------------------------------------- RaBitQ code

@pytest.mark.parametrize("d", [8, 32, 128, 1024])
def test_rabitq_one_hot_is_a_hadamard_column(d):
    rng = np.random.default_rng(d)
    s = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
    H = scipy.linalg.hadamard(d)
    js = [0, 1, d // 2 - 1, d - 1]
    x = np.zeros((len(js), d), np.float16)
    for r, j in enumerate(js):
        x[r, j] = 0.75 if r % 2 == 0 else -3.0
    out = signcodes.rabitq_encode(x, s)
    for r, j in enumerate(js):
        sign_x = 1 if r % 2 == 0 else -1
        want = (sign_x * s[j] * H[:, j] > 0).astype(np.uint8)  # no zeros here
        assert out["bits"][r].tolist() == want.tolist()
        assert out["packed"][r].tolist() == packing.pack(want[None, :], 1)[0].tolist()
        assert out["norms"][r] == np.float32(abs(float(x[r, j])))


def test_rabitq_hand_example_with_exact_zeros():
    # D = 8, s = +1, x = e_3 - e_5: y_i is proportional to H[i,3] - H[i,5] =
    # (-1)^popcount(i & 3) - (-1)^popcount(i & 5) = 0, 0, -2, 2, 2, -2, 0, 0 for i = 0..7,
    # so the bits are 1,1,0,1,1,0,1,1 and the word is 1 + 2 + 8 + 16 + 64 + 128 = 219.
    x = np.zeros((1, 8), np.float16)
    x[0, 3], x[0, 5] = 1.0, -1.0
    out = signcodes.rabitq_encode(x, np.ones(8, np.int8))
    assert out["bits"][0].tolist() == [1, 1, 0, 1, 1, 0, 1, 1]
    assert out["packed"][0].tolist() == [219]
    assert out["norms"][0] == np.float32(math.sqrt(2.0))


@pytest.mark.parametrize("d", [8, 16, 64, 1024])
def test_rabitq_zero_vector_sets_every_bit(d):
    out = signcodes.rabitq_encode(np.zeros((2, d), np.float16), np.ones(d, np.int8))
    assert out["bits"].min() == 1 and out["norms"].max() == 0.0
    want = np.uint32(0xFFFFFFFF) & ~packing.padding_mask(d, 1)
    assert (out["packed"] == want[None, :]).all()


def test_rabitq_planted_mistakes_fail():
    x = np.zeros((1, 8), np.float16)
    x[0, 3], x[0, 5] = 1.0, -1.0
    _, y = rvq.norms_and_rotation(x, np.ones(8, np.int8))
    assert (y > 0).astype(int)[0].tolist() != [1, 1, 0, 1, 1, 0, 1, 1]  # strict > loses the zeros
    # signs applied after H instead of before: one-hot e_1 with s_1 = -1 and s_0 = +1
    d = 8
    s = np.ones(d, np.int8)
    s[1] = -1
    H = scipy.linalg.hadamard(d)
    e1 = np.zeros((1, d), np.float16)
    e1[0, 1] = 1.0
    good = signcodes.rabitq_encode(e1, s)["bits"][0]
    after = (s * H[:, 1] > 0).astype(np.uint8)  # diag(s) H e_1
    assert good.tolist() != after.tolist()


# ------------------------------------------------------------------------------- QJL sketch

def _fraction_signs(x16, S16):
    xs = [[Fraction(float(v)) for v in row] for row in np.asarray(x16, np.float16)]
    ss = [[Fraction(float(v)) for v in row] for row in np.asarray(S16, np.float16)]
    out = np.zeros((len(xs), len(ss)), np.int8)
    for i, xr in enumerate(xs):
        for j, sr in enumerate(ss):
            t = sum(a * b for a, b in zip(xr, sr))
            out[i, j] = (t > 0) - (t < 0)
    return out


@pytest.mark.parametrize("d,m,seed", [(32, 32, 1), (64, 64, 2), (16, 96, 3)])
def test_qjl_signs_equal_rational_arithmetic(d, m, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((40, d)).astype(np.float16)
    S = rng.standard_normal((m, d)).astype(np.float16)
    # a few rows of small integers give exact zeros and near-ties
    x[:8] = rng.integers(-2, 3, (8, d)).astype(np.float16)
    S[:8] = rng.integers(-1, 2, (8, d)).astype(np.float16)
    _, _, sign = signcodes.qjl_dots(x, S)
    assert (sign == _fraction_signs(x, S)).all()
    assert (_fraction_signs(x[:8], S[:8]) == 0).any()  # the exact-zero case is exercised
    out = signcodes.qjl_encode(x, S)
    assert (out["bits"] == (_fraction_signs(x, S) >= 0)).all()


def test_qjl_cancellation_float64_gets_wrong():
    # (S x)_0 = 65504^2 - 2^-24 - 65504^2 = -2^-24 exactly; float64 rounds the partial sum
    # 65504^2 - 2^-24 back to 65504^2 and returns 0 (which would set the bit).
    d = 32
    S = np.zeros((32, d), np.float16)
    x = np.zeros((2, d), np.float16)
    S[0, :3] = [65504.0, -1.0, -65504.0]
    S[1, :3] = [65504.0, 1.0, -65504.0]
    x[0, :3] = [65504.0, 2.0 ** -24, 65504.0]
    x[1, :3] = [65504.0, 2.0 ** -24, 65504.0]
    naive = x.astype(np.float64) @ S.astype(np.float64).T
    assert naive[0, 0] == 0.0  # the trap is real
    out = signcodes.qjl_encode(x, S)
    assert out["bits"][0, 0] == 0 and out["bits"][0, 1] == 1
    assert (_fraction_signs(x[:1], S[:2]) == [[-1, 1]]).all()


def _hand_x():
    # d = 32: +1 at 0, 4, 31; 0 at 1; -0.0 at 2; -1 elsewhere. [x_j >= 0] is set at
    # 0, 1, 2, 4, 31: word 1 + 2 + 4 + 16 + 2^31 = 0x80000017.
    x = np.full((1, 32), -1.0, np.float16)
    x[0, [0, 4, 31]] = 1.0
    x[0, 1] = 0.0
    x[0, 2] = np.float16(-0.0)
    return x


def test_qjl_identity_sketch_hand_word():
    out = signcodes.qjl_encode(_hand_x(), np.eye(32, dtype=np.float16))
    assert out["packed"][0].tolist() == [0x80000017]
    # shifted identity: row j = e_{(j + 1) % 32}, so bit j = [x_{j+1} >= 0]: set at
    # j = 0, 1, 3, 30, 31 (x_1, x_2, x_4, x_31, x_0): word 1 + 2 + 8 + 2^30 + 2^31
    shift = np.roll(np.eye(32, dtype=np.float16), 1, axis=1)
    out = signcodes.qjl_encode(_hand_x(), shift)
    assert out["packed"][0].tolist() == [0xC000000B]


@pytest.mark.parametrize("theta", [math.pi / 6, math.pi / 2, 2 * math.pi / 3])
def test_qjl_sign_random_projection_law(theta):
    d, m = 64, 4096
    S = synth.rows(synth.TensorSpec(1, 1, m, d, "gauss", 11)).numpy()
    rng = np.random.default_rng(int(theta * 1000))
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    w = rng.standard_normal(d)
    w -= (w @ u) * u
    w /= np.linalg.norm(w)
    x = np.stack([u, math.cos(theta) * u + math.sin(theta) * w]) * 8.0
    out = signcodes.qjl_encode(x.astype(np.float16), S)
    frac = float(np.mean(out["bits"][0] != out["bits"][1]))
    p = theta / math.pi
    assert abs(frac - p) <= 4.0 * math.sqrt(p * (1 - p) / m) + 2e-3


def test_qjl_norms():
    x = np.zeros((4, 32), np.float16)
    x[0, :2] = [3.0, 4.0]       # 5 exactly
    x[1, :2] = [1.0, 1.0]       # sqrt(2) -> fp16 1.4140625 (0x3DA8)
    x[3, :] = 65504.0           # 65504 sqrt(32) overflows fp16 -> inf
    out = signcodes.qjl_encode(x, np.eye(32, dtype=np.float16))
    n = out["norms"]
    assert n.dtype == np.float16
    assert n[0] == 5.0 and n[1].view(np.uint16) == 0x3DA8 and n[2] == 0.0 and np.isinf(n[3])
    assert out["packed"][2].tolist() == [0xFFFFFFFF]  # the zero vector: every dot is 0


def test_qjl_planted_mistakes_fail():
    x = _hand_x()
    I = np.eye(32, dtype=np.float16)
    dots, _, sign = signcodes.qjl_dots(x, I)
    strict = packing.pack((sign > 0).astype(np.uint8), 1)[0].tolist()
    assert strict != [0x80000017]
    shift = np.roll(I, 1, axis=1)
    transposed = signcodes.qjl_encode(x, np.ascontiguousarray(shift.T))["packed"][0].tolist()
    assert transposed != [0xC000000B]
    bits = signcodes.qjl_encode(x, I)["bits"][0]
    msb_first = int("".join(str(int(b)) for b in bits), 2)
    assert msb_first != 0x80000017
