"""GPU parity of the single-stage codec (kvq_mse_encode_pack / kvq_mse_unpack_decode)
against the oracle's encode_mse / decode_mse, under the same comparison rule as the
two-stage codec: codes bit-exact except in-window one-level flips (at most 1e-6 of the
codes), norms within 1e-6 relative, decoders fed the oracle's words agree within 1e-3 on
unit vectors."""
import numpy as np
import pytest
import torch

import residual_vq_encode_amd as kvq
import synth
from oracle import rvq
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
DEV = "cuda"
D_ALL = [8, 16, 32, 64, 128, 256, 512, 1024]


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("d", D_ALL)
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_grid(d, bits):
    _say(f"mse grid d={d} bits={bits}")
    for n in (1, 33):
        x = synth.tensor(synth.TensorSpec(1, 1, n, d, "gauss_outliers", 300 + d + bits + n), device=DEV)
        gu.check_encode_mse(x, synth.signs(3000 + d, d).numpy(), bits)


@pytest.mark.parametrize("d", D_ALL)
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_decode_grid(d, bits):
    _say(f"mse decode d={d} bits={bits}")
    spec = synth.TensorSpec(2, 3, 21, d, "gauss", 500 + d + bits)
    s = synth.signs(4000 + d, d).numpy()
    ref = rvq.encode_mse(synth.rows(spec).numpy().reshape(-1, d), s, gu.tables(d, bits))
    gu.check_decode_mse_from_oracle_words(ref, s, bits, (2, 3, 21, d))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_mse_llama_layer(bits):
    w = synth.WORKLOADS["llama_layer"]
    _say(f"mse llama_layer [1,32,8192,128] b={bits}")
    x = synth.tensor(w.tensors[0], device=DEV)
    rep, (p, nrm), ref = gu.check_encode_mse(x, synth.signs(w.sign_seed, 128).numpy(), bits)
    _say(rep.summary())


@pytest.mark.parametrize("bits", [2, 3])
def test_mse_cache_window_and_ragged(bits):
    """Write into a cache window (S < S_cap, s_offset > 0) with a ragged tile count."""
    _say(f"mse window bits={bits}")
    x = synth.tensor(synth.TensorSpec(3, 5, 37, 128, "gauss", 77 + bits), device=DEV)
    rep, (p, nrm), _ = gu.check_encode_mse(x, synth.signs(9, 128).numpy(), bits, S_cap=100, s_offset=41)
    # nothing outside the window was written
    assert bool((p[:, :, :41] == -1).all()) and bool((p[:, :, 78:] == -1).all())
    assert bool(torch.isnan(nrm[:, :, :41]).all()) and bool(torch.isnan(nrm[:, :, 78:]).all())


def test_mse_stream_equals_two_stage_first_stream():
    """The single-stage stream is the two-stage codec's first stream, word for word."""
    x = synth.tensor(synth.TensorSpec(1, 4, 999, 128, "gauss_outliers", 12), device=DEV)
    s = synth.signs(12, 128).numpy()
    for bits in (1, 2, 3, 4):
        cb = kvq.build_codebooks(128, bits, s)
        p1, _, n2 = kvq.encode(x, cb)
        p, n1 = kvq.encode_mse(x, cb)
        torch.cuda.synchronize()
        assert torch.equal(p, p1) and torch.equal(n1, n2)
