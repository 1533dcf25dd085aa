"""Pins of the oracle's attention over packed caches (oracle/attend.py) against results it
does not compute itself:

  * one cached position: the output is that value's reconstruction, i.e. the oracle's
    two-stage decode (pinned by the worked examples) rounded to fp16, bit for bit;
  * identical keys: uniform weights, so the output is the mean of the values, recomputed
    here with scipy's Hadamard matrix;
  * a dominant key: with a large scale the output tends to the value of the key that best
    matches the query;
  * brute force on tiny random caches: reconstruction with scipy's Hadamard matrix, scores,
    scipy.special.softmax and the weighted sum, written independently here;
  * the grouped-query head mapping (query head h reads key/value head h // (Hq / Hkv)),
    with a planted wrong mapping that must disagree.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import scipy.special

from oracle import attend, packing, rvq
from oracle import codebooks as cbk


def _signs(seed, d):
    rng = np.random.default_rng(seed)
    return np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)


def _cache(B, Hkv, S, d, bits, seed, signs):
    """A packed cache made by the oracle's own encoder from random fp16 vectors."""
    t = cbk.build_tables(d, bits)
    x = np.random.default_rng(seed).standard_normal((B * Hkv * S, d)).astype(np.float16)
    e = rvq.encode(x, signs, t)
    nw = e["packed1"].shape[1]
    return (e["packed1"].reshape(B, Hkv, S, nw), e["packed2"].reshape(B, Hkv, S, nw),
            e["norms"].reshape(B, Hkv, S)), t


def _recon_scipy(p1, p2, n, signs, t):
    d = t.d
    z = (t.c1[packing.unpack(p1, t.bits, d)] + t.c2[packing.unpack(p2, t.bits, d)]).astype(np.float32)
    Hs = scipy.linalg.hadamard(d).astype(np.float64)
    return (z.astype(np.float64) @ Hs) / math.sqrt(d) * signs.astype(np.float64) * n.astype(np.float64)[:, None]


def test_single_position_is_the_decoded_value():
    d, bits = 64, 2
    s = _signs(1, d)
    kc, t = _cache(1, 2, 1, d, bits, 10, s)
    vc, _ = _cache(1, 2, 1, d, bits, 11, s)
    q = np.random.default_rng(2).standard_normal((1, 4, 3, d)).astype(np.float16)
    out = attend.attend(q, kc, vc, s, s, t, t, 1, 0.125)
    for h in range(4):
        g = h // 2
        want = rvq.decode(vc[0][0, g], vc[1][0, g], vc[2][0, g], s, t)[0]
        for sq in range(3):
            assert out[0, h, sq].tobytes() == want.tobytes()


def test_identical_keys_give_the_mean_value():
    d, bits, S = 32, 3, 9
    sk, sv = _signs(3, d), _signs(4, d)
    kc, t = _cache(1, 1, 1, d, bits, 12, sk)
    kc = tuple(np.repeat(a, S, axis=2) for a in kc)
    vc, _ = _cache(1, 1, S, d, bits, 13, sv)
    q = np.random.default_rng(5).standard_normal((1, 1, 1, d)).astype(np.float16)
    got = attend.attend64(q, kc, vc, sk, sv, t, t, S, 0.3)[0, 0, 0]
    want = _recon_scipy(vc[0][0, 0], vc[1][0, 0], vc[2][0, 0], sv, t).mean(axis=0)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_dominant_key_selects_its_value():
    d, bits, S = 128, 4, 20
    s = _signs(6, d)
    kc, t = _cache(1, 1, S, d, bits, 14, s)
    vc, _ = _cache(1, 1, S, d, bits, 15, s)
    K = _recon_scipy(kc[0][0, 0], kc[1][0, 0], kc[2][0, 0], s, t)
    j = 7
    q = (K[j] / np.linalg.norm(K[j])).astype(np.float16)[None, None, None, :]
    got = attend.attend64(q, kc, vc, s, s, t, t, S, 200.0)[0, 0, 0]
    scores = K @ q[0, 0, 0].astype(np.float64)
    assert int(np.argmax(scores)) == j
    want = _recon_scipy(vc[0][0, 0], vc[1][0, 0], vc[2][0, 0], s, t)[j]
    gap = 200.0 * (np.sort(scores)[-1] - np.sort(scores)[-2])
    assert gap > 30.0  # the runner-up weight is below e^-30
    assert np.max(np.abs(got - want)) <= 1e-9 * np.max(np.abs(want)) * S


@pytest.mark.parametrize("d,bits,B,Hq,Hkv,Sq,S_cap,S_kv", [(8, 1, 2, 2, 1, 3, 7, 5), (16, 2, 1, 6, 3, 2, 11, 11),
                                                            (64, 3, 1, 4, 4, 1, 33, 30), (128, 4, 2, 4, 2, 2, 9, 4)])
def test_brute_force_tiny(d, bits, B, Hq, Hkv, Sq, S_cap, S_kv):
    sk, sv = _signs(d, d), _signs(d + 1, d)
    kc, t = _cache(B, Hkv, S_cap, d, bits, 20 + d, sk)
    vc, _ = _cache(B, Hkv, S_cap, d, bits, 21 + d, sv)
    q = np.random.default_rng(22).standard_normal((B, Hq, Sq, d)).astype(np.float16)
    scale = 1.0 / math.sqrt(d)
    got = attend.attend64(q, kc, vc, sk, sv, t, t, S_kv, scale)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            K = _recon_scipy(kc[0][b, g, :S_kv], kc[1][b, g, :S_kv], kc[2][b, g, :S_kv], sk, t)
            V = _recon_scipy(vc[0][b, g, :S_kv], vc[1][b, g, :S_kv], vc[2][b, g, :S_kv], sv, t)
            for sq in range(Sq):
                p = scipy.special.softmax(scale * np.einsum("j,tj->t", q[b, h, sq].astype(np.float64), K))
                want = np.einsum("t,tj->j", p, V)
                assert np.max(np.abs(got[b, h, sq] - want)) <= 1e-12 * (1.0 + np.max(np.abs(want)))


def test_grouped_query_mapping_and_planted_mistake():
    d, bits, B, Hq, Hkv, S = 16, 2, 1, 4, 2, 6
    s = _signs(30, d)
    kc, t = _cache(B, Hkv, S, d, bits, 31, s)
    vc, _ = _cache(B, Hkv, S, d, bits, 32, s)
    q = np.random.default_rng(33).standard_normal((B, Hq, 1, d)).astype(np.float16)
    out = attend.attend64(q, kc, vc, s, s, t, t, S, 0.25)
    # swapping the two key/value heads swaps which query heads see which cache
    kc2 = tuple(a[:, ::-1].copy() for a in kc)
    vc2 = tuple(a[:, ::-1].copy() for a in vc)
    q2 = q[:, [2, 3, 0, 1]].copy()
    out2 = attend.attend64(q2, kc2, vc2, s, s, t, t, S, 0.25)
    assert np.array_equal(out2[:, [2, 3, 0, 1]], out)
    # a planted wrong mapping (h % Hkv) gives a different answer for head 1
    K = _recon_scipy(kc[0][0, 1], kc[1][0, 1], kc[2][0, 1], s, t)
    V = _recon_scipy(vc[0][0, 1], vc[1][0, 1], vc[2][0, 1], s, t)
    p = scipy.special.softmax(0.25 * K @ q[0, 1, 0].astype(np.float64))
    assert np.max(np.abs(out[0, 1, 0] - p @ V)) > 1e-3
