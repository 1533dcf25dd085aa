"""Self-tests of the device-vs-oracle comparison rule (oracle/flips.py), on the CPU.

Each test plants one kind of disagreement into an oracle encode and checks the rule
accepts what it should (one-level flips inside the boundary window, including the
stage-2 cascade they cause) and rejects the rest.
"""
import numpy as np

from oracle import codebooks as cb
from oracle import flips, packing, rvq

REL = 1e-5


def _ref_from_y(y32, t):
    i1, r, i2 = rvq.quantize_two_stage(y32, t)
    return {"y": y32, "r": r, "i1": i1, "i2": i2,
            "packed1": packing.pack(i1, t.bits), "packed2": packing.pack(i2, t.bits),
            "norm64": np.ones(y32.shape[0]), "norms": np.ones(y32.shape[0], np.float32)}


def _setup(bits=2, d=16, n=32, seed=0):
    t = cb.build_tables(d, bits)
    y = (np.random.default_rng(seed).standard_normal((n, d)) * t.sigma1).astype(np.float32)
    return t, y


def test_identical_is_clean():
    t, y = _setup()
    ref = _ref_from_y(y, t)
    rep = flips.compare_encode(ref["packed1"], ref["packed2"], ref["norms"], ref, t, REL)
    assert rep.flips == 0 and rep.ok(0.0, 0.0), rep.summary()


def test_far_from_boundary_flip_is_rejected():
    t, y = _setup()
    y[0, 0] = t.c1[2]  # on a centroid: far from every boundary
    ref = _ref_from_y(y, t)
    i1 = ref["i1"].copy()
    i1[0, 0] = 1
    rep = flips.compare_encode(packing.pack(i1, t.bits), ref["packed2"], ref["norms"], ref, t, REL)
    assert rep.bad_stage1 == 1 and not rep.ok(1.0, 1.0)


def test_near_boundary_one_level_flip_with_cascade_is_accepted():
    t, y = _setup()
    beta = t.b1[2]
    y[3, 5] = np.nextafter(beta, np.float32(np.inf))  # oracle picks level 3
    ref = _ref_from_y(y, t)
    assert ref["i1"][3, 5] == 3
    i1 = ref["i1"].copy()
    i1[3, 5] = 2  # the device saw y a hair below the boundary
    r_dev = (y - t.c1[i1]).astype(np.float32)
    i2 = rvq.nearest(r_dev, t.c2)  # the device's stage 2 follows its own residual
    rep = flips.compare_encode(packing.pack(i1, t.bits), packing.pack(i2, t.bits), ref["norms"], ref, t, REL)
    assert rep.bad_stage1 == 0 and rep.bad_stage2 == 0 and rep.stage1_diff == 1
    assert rep.ok(1.0 / (2 * y.size) + 1e-12, 0.0), rep.summary()
    assert not rep.ok(0.0, 0.0)  # the cap still counts it
    # the same stage-1 flip with the stage-2 code left at the oracle's value is rejected
    rep2 = flips.compare_encode(packing.pack(i1, t.bits), ref["packed2"], ref["norms"], ref, t, REL)
    if ref["i2"][3, 5] != i2[3, 5]:
        assert rep2.bad_stage2 == 1


def test_two_level_flip_near_boundary_is_rejected():
    t, y = _setup()
    y[1, 1] = np.nextafter(t.b1[2], np.float32(np.inf))
    ref = _ref_from_y(y, t)
    i1 = ref["i1"].copy()
    i1[1, 1] = 1  # two levels below 3
    rep = flips.compare_encode(packing.pack(i1, t.bits), ref["packed2"], ref["norms"], ref, t, REL)
    assert rep.bad_stage1 == 1


def test_window_scale_at_zero_boundary():
    t, y = _setup()
    y[2, 2] = np.float32(0.5 * REL * t.sigma1)  # inside the window of the boundary 0
    y[2, 3] = np.float32(3.0 * REL * t.sigma1)  # outside it
    ref = _ref_from_y(y, t)
    i1 = ref["i1"].copy()
    i1[2, 2] -= 1
    i1[2, 3] -= 1
    r_dev = (y - t.c1[i1]).astype(np.float32)
    i2 = rvq.nearest(r_dev, t.c2)
    rep = flips.compare_encode(packing.pack(i1, t.bits), packing.pack(i2, t.bits), ref["norms"], ref, t, REL)
    assert rep.stage1_diff == 2 and rep.bad_stage1 == 1


def test_padding_and_norm_are_checked():
    t = cb.build_tables(8, 3)  # 8 three-bit codes leave 8 padding bits per word
    y = (np.random.default_rng(1).standard_normal((4, 8)) * t.sigma1).astype(np.float32)
    ref = _ref_from_y(y, t)
    p1 = ref["packed1"].copy()
    p1[0, 0] |= np.uint32(1 << 30)
    rep = flips.compare_encode(p1, ref["packed2"], ref["norms"], ref, t, REL)
    assert rep.padding_bad == 1 and not rep.ok(1.0, 1.0)
    norms = ref["norms"].copy()
    norms[2] *= np.float32(1.0 + 1e-4)
    rep = flips.compare_encode(ref["packed1"], ref["packed2"], norms, ref, t, REL)
    assert 5e-5 < rep.norm_max_rel < 2e-4 and not rep.ok(1.0, 1e-6)


def test_small_sample_allowance_is_the_poisson_tail_bound():
    """The per-sample flip allowance of the GPU parity tests: the smallest k >= 1 with
    P(Poisson(1e-6 n) > k) <= 1e-3, checked against scipy's Poisson survival function."""
    from scipy import stats

    from tests import gpu_util as gu
    for n in [1, 10, 1000, 10 ** 5, 384_000, 768_256, 10 ** 6, 3 * 10 ** 6, 10 ** 7 - 1]:
        k = gu.small_sample_allowance(n)
        lam = gu.MAX_FLIP_FRACTION * n
        assert k >= 1 and stats.poisson.sf(k, lam) <= gu.SMALL_SAMPLE_TAIL
        assert k == 1 or stats.poisson.sf(k - 1, lam) > gu.SMALL_SAMPLE_TAIL
        assert gu.flip_cap(n) * n >= k
    for n in [10 ** 7, 10 ** 9]:  # workload-sized samples: the rate itself
        assert gu.flip_cap(n) == gu.MAX_FLIP_FRACTION
