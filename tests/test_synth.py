"""The seeded input generator: determinism, slice independence, distribution shape."""
import math

import numpy as np
import torch

import synth


def test_splitmix64_reference_values():
    # SplitMix64's output function on the state sequence k*G (k = 1, 2, 3) from seed 0
    # is the published SplitMix64 stream for seed 0.
    out = synth.mix64(torch.arange(1, 4, dtype=torch.int64) * synth._G)
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [int(v) & ((1 << 64) - 1) for v in out] == want


def test_rows_are_position_addressable_and_deterministic():
    spec = synth.TensorSpec(2, 4, 16, 32, "gauss_laplace_heads", 9)
    full = synth.tensor(spec).reshape(-1, 32)
    part = synth.rows(spec, 37, 11)
    assert torch.equal(full[37:48], part)
    pick = torch.tensor([100, 3, 64], dtype=torch.int64)
    assert torch.equal(synth.rows_at(spec, pick), full[pick])
    assert torch.equal(synth.tensor(spec).reshape(-1, 32), full)


def test_distributions():
    g = synth.rows(synth.TensorSpec(1, 1, 4096, 128, "gauss", 1)).float()
    assert abs(g.mean()) < 0.01 and abs(g.std() - 1) < 0.01
    o = synth.rows(synth.TensorSpec(1, 1, 4096, 128, "gauss_outliers", 2)).float()
    assert abs(o[:, 37].std() - 20) < 0.6 and abs(o[:, 36].std() - 1) < 0.05
    lap = synth.rows(synth.TensorSpec(1, 2, 8192, 128, "gauss_laplace_heads", 3), 8192, 8192).float()
    assert abs(lap.abs().mean() - 1.0) < 0.02  # E|X| = 1 for Laplace(0, 1)
    ts = synth.rows(synth.TensorSpec(2, 4, 256, 128, "gauss_token_scale", 4)).float().reshape(2, 4, 256, 128)
    sd = ts.std(dim=-1)  # per (b, h, s)
    assert torch.allclose(sd[:, 0], sd[:, 3], rtol=0.5)  # one scale per token, shared by heads
    lsd = torch.log(sd[:, 0])
    assert lsd.min() > math.log(0.1) - 0.5 and lsd.max() < math.log(10) + 0.5


def test_signs():
    s = synth.signs(102, 128)
    assert s.dtype == torch.int8 and set(s.tolist()) == {-1, 1}
    assert torch.equal(s, synth.signs(102, 128)) and not torch.equal(s, synth.signs(103, 128))
