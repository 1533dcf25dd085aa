"""The small-sample allowance, pooled. Samples smaller than a workload may each carry the
few in-window flips that a Poisson count at the 1e-6 rate reaches with probability 10^-3
(tests/gpu_util.py, flip_cap); over every sample judged in this session together, the
flips must still stay within the 1e-6 rate of all their codes. Runs
after the other GPU tests (pytest collects files in name order); alone, it has nothing to
judge and skips."""
import pytest

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_pooled_flip_rate_of_small_samples():
    p = gu.POOLED
    if p["samples"] == 0:
        pytest.skip("no small samples were judged in this session")
    rate = p["flips"] / p["codes"]
    print(f"pooled over {p['samples']} samples: {p['flips']} flips in {p['codes']} codes = {rate:.3e}", flush=True)
    assert rate <= gu.MAX_FLIP_FRACTION, p
