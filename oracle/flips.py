"""The comparison rule between a device encode and the oracle (test infrastructure).

A device computes the rotated coordinate y with a float32 butterfly while the oracle
rounds a float64 product once, so the two y values differ by a few float32 ulps. Where
y sits that close to a quantization boundary the two sides may legitimately choose
neighbouring levels. The rule:

  * every code of every packed word must equal the oracle's, and every padding bit must
    be zero, EXCEPT
  * a stage-1 code may differ from the oracle's by exactly one level when the oracle's y
    lies within `window` of the boundary between those two levels, where the window is
    rel * max(|boundary|, sigma1) (a relative window degenerates at the boundary 0, so
    the stage's scale sets its floor);
  * the stage-2 code is judged against the oracle's stage-2 decision for the residual
    the device actually formed, y - c1[i1_device] (a stage-1 flip changes the residual),
    with the same one-level-inside-the-window allowance (scale sigma2);
  * the fraction of differing codes over all 2*N*D codes must not exceed a cap.

Norms are compared with a relative tolerance. All tolerances are arguments: each test
states its own numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import packing
from .codebooks import Tables
from .rvq import nearest


@dataclass
class Report:
    n_vectors: int
    n_codes: int
    stage1_diff: int = 0
    stage2_diff: int = 0
    bad_stage1: int = 0
    bad_stage2: int = 0
    padding_bad: int = 0
    norm_max_rel: float = 0.0
    examples: list = field(default_factory=list)

    @property
    def flips(self) -> int:
        return self.stage1_diff + self.stage2_diff

    @property
    def flip_fraction(self) -> float:
        return self.flips / max(1, self.n_codes)

    def ok(self, max_flip_fraction: float, norm_rel_tol: float) -> bool:
        return (self.bad_stage1 == 0 and self.bad_stage2 == 0 and self.padding_bad == 0
                and self.flip_fraction <= max_flip_fraction and self.norm_max_rel <= norm_rel_tol)

    def summary(self) -> str:
        return (f"N={self.n_vectors} codes={self.n_codes} stage1_diff={self.stage1_diff} "
                f"stage2_diff={self.stage2_diff} bad1={self.bad_stage1} bad2={self.bad_stage2} "
                f"padding_bad={self.padding_bad} flip_frac={self.flip_fraction:.3e} "
                f"norm_max_rel={self.norm_max_rel:.3e} examples={self.examples[:5]}")


def _judge(v_or: np.ndarray, code_dev: np.ndarray, code_or: np.ndarray, bounds: np.ndarray,
           scale: float, rel: float):
    """Counts (differing, differing-but-not-allowed) for one stage; returns the masks too."""
    diff = code_dev != code_or
    if not diff.any():
        return 0, 0, diff, diff
    lo = np.minimum(code_dev, code_or).astype(np.int64)
    step = np.abs(code_dev.astype(np.int64) - code_or.astype(np.int64))
    lo_c = np.clip(lo, 0, len(bounds) - 1)
    beta = bounds[lo_c].astype(np.float64)
    win = rel * np.maximum(np.abs(beta), scale)
    near = np.abs(v_or.astype(np.float64) - beta) <= win
    bad = diff & ~((step == 1) & near)
    return int(diff.sum()), int(bad.sum()), diff, bad


def compare_encode(dev_p1: np.ndarray, dev_p2: np.ndarray, dev_norms: np.ndarray,
                   ref: dict, t: Tables, rel: float = 1e-5) -> Report:
    """Judge device packed streams [N, n_words] and norms [N] against an oracle encode."""
    n, d = ref["y"].shape
    rep = Report(n_vectors=n, n_codes=2 * n * d)
    pad = packing.padding_mask(d, t.bits)
    rep.padding_bad = int(np.count_nonzero(dev_p1 & pad) + np.count_nonzero(dev_p2 & pad))
    i1d = packing.unpack(dev_p1, t.bits, d)
    i2d = packing.unpack(dev_p2, t.bits, d)
    y = ref["y"]
    rep.stage1_diff, rep.bad_stage1, diff1, bad1 = _judge(y, i1d, ref["i1"], t.b1, t.sigma1, rel)
    # stage 2 against the oracle's decision on the residual the device formed
    r_dev = (y - t.c1[i1d]).astype(np.float32)
    i2o = nearest(r_dev, t.c2) if diff1.any() else ref["i2"]
    rep.stage2_diff, rep.bad_stage2, diff2, bad2 = _judge(r_dev, i2d, i2o, t.b2, t.sigma2, rel)
    for name, badm, v in (("stage1", bad1, y), ("stage2", bad2, r_dev)):
        if badm.any():
            for (vi, ci) in np.argwhere(badm)[:5]:
                rep.examples.append((name, int(vi), int(ci), float(v[vi, ci]),
                                     int(i1d[vi, ci] if name == "stage1" else i2d[vi, ci]),
                                     int(ref["i1"][vi, ci] if name == "stage1" else i2o[vi, ci])))
    nr = ref["norm64"]
    dn = np.abs(np.asarray(dev_norms, dtype=np.float64) - nr)
    rel_err = np.where(nr > 0, dn / np.where(nr > 0, nr, 1.0), dn)
    rep.norm_max_rel = float(rel_err.max()) if rel_err.size else 0.0
    return rep


def compare_encode_single(dev_p: np.ndarray, dev_norms: np.ndarray, ref: dict, t: Tables,
                          rel: float = 1e-5) -> Report:
    """The same rule for the single-stage codec: one stream, stage-1 codes only."""
    n, d = ref["y"].shape
    rep = Report(n_vectors=n, n_codes=n * d)
    rep.padding_bad = int(np.count_nonzero(dev_p & packing.padding_mask(d, t.bits)))
    i1d = packing.unpack(dev_p, t.bits, d)
    y = ref["y"]
    rep.stage1_diff, rep.bad_stage1, _, bad1 = _judge(y, i1d, ref["i1"], t.b1, t.sigma1, rel)
    for (vi, ci) in np.argwhere(bad1)[:5]:
        rep.examples.append(("stage1", int(vi), int(ci), float(y[vi, ci]), int(i1d[vi, ci]), int(ref["i1"][vi, ci])))
    nr = ref["norm64"]
    dn = np.abs(np.asarray(dev_norms, dtype=np.float64) - nr)
    rel_err = np.where(nr > 0, dn / np.where(nr > 0, nr, 1.0), dn)
    rep.norm_max_rel = float(rel_err.max()) if rel_err.size else 0.0
    return rep
