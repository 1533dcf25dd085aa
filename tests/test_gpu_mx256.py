"""The matrix-core encode at D = 256 (H_256 = H_8 (x) H_32: sixteen MFMA products per tile of
16 vectors, three butterfly stages across the eight 32-coordinate blocks, two 4 x 4
transposes of the code pieces) against the oracle: both codecs and the sign code, at 1, 2 and
4 bits, into contiguous caches and into cache windows, with ragged last tiles, waves that
walk many tiles, and the full head-dimension-256 workload judged on every vector. (3-bit
codes at D = 256 take the butterfly kernel.)

Method: "rvq" tag page, "The pipeline, as it actually runs"; "turboquant" tag page,
"Kernel 3" (y = H diag(s) x / sqrt(D)). Comparison rule: tests/gpu_util.py.
"""
import pytest
import torch

import synth
from tests import gpu_util as gu
from tests.test_gpu_signcodes import check_rabitq

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 256


def _say(msg):
    print(msg, flush=True)


def _signs(seed):
    return synth.signs(seed, D).numpy()


@pytest.mark.parametrize("bits", [1, 2, 4])
@pytest.mark.parametrize("n", [1, 5, 15, 16, 17, 33, 1000, 33333])
def test_two_stage_contiguous(bits, n):
    _say(f"mx256 two-stage contiguous bits={bits} n={n}")
    spec = synth.TensorSpec(1, 1, n, D, "gauss_outliers", 4100 + 7 * n + bits)
    gu.check_encode(synth.tensor(spec, device=DEV), _signs(41 + bits), bits)


@pytest.mark.parametrize("bits", [1, 2, 4])
def test_two_stage_cache_window(bits):
    """[2, 3, 700, 256] written at s_offset = 123 into S_cap = 1000: every vector's codes and
    norm against the oracle, and every cell outside the window untouched."""
    B, H, S, S_cap, off = 2, 3, 700, 1000, 123
    _say(f"mx256 two-stage window bits={bits}")
    s = _signs(51 + bits)
    x = synth.tensor(synth.TensorSpec(B, H, S, D, "gauss", 4200 + bits), device=DEV)
    p1, p2, nrm = gu.gpu_encode(x, s, bits, S_cap=S_cap, s_offset=off, fill=-1)
    nw = p1.shape[-1]
    win = slice(off, off + S)
    rep = gu.judge_all(x.reshape(-1, D), s, bits, p1[:, :, win].reshape(-1, nw), p2[:, :, win].reshape(-1, nw),
                       nrm[:, :, win].reshape(-1))
    _say(rep.summary())
    assert rep.n_vectors == B * H * S
    assert rep.ok(gu.capped(rep.n_codes, rep.flips), gu.NORM_REL_TOL), rep.summary()
    outside = torch.ones(S_cap, dtype=torch.bool, device=DEV)
    outside[win] = False
    assert bool((p1[:, :, outside] == -1).all()) and bool((p2[:, :, outside] == -1).all())
    assert bool(torch.isnan(nrm[:, :, outside]).all())


@pytest.mark.parametrize("bits", [1, 2, 4])
@pytest.mark.parametrize("window", [False, True])
def test_single_stage(bits, window):
    _say(f"mx256 single-stage bits={bits} window={window}")
    x = synth.tensor(synth.TensorSpec(2, 2, 900, D, "gauss_outliers", 4300 + bits), device=DEV)
    if window:
        gu.check_encode_mse(x, _signs(61 + bits), bits, S_cap=1200, s_offset=211)
    else:
        gu.check_encode_mse(x, _signs(61 + bits), bits)


@pytest.mark.parametrize("window", [False, True])
def test_sign_code(window):
    """The 1-bit sign code [y >= 0] of the rotated vector and its float32 norm, under the
    sign-code tests' rule."""
    B, H, S = 2, 2, 777
    _say(f"mx256 sign code window={window}")
    x = synth.tensor(synth.TensorSpec(B, H, S, D, "gauss", 4400), device=DEV)
    if window:
        check_rabitq(x, _signs(71), S_cap=1000, s_offset=99)
    else:
        check_rabitq(x, _signs(71))


@pytest.mark.parametrize("bits", [2, 4])
def test_head_dim_256_workload_every_vector(bits):
    """The head-dimension-256 workload [1,32,4096,256] in one launch (waves walking several
    tiles), every one of its 131,072 vectors judged against the oracle."""
    w = synth.WORKLOADS["head_dim_256"]
    spec = w.tensors[0]
    s = synth.signs(w.sign_seed, D).numpy()
    _say(f"mx256 workload head_dim_256 [1,32,4096,256] b={bits}, every vector")
    x = synth.tensor(spec, device=DEV)
    p1, p2, nrm = gu.gpu_encode(x, s, bits)
    nw = p1.shape[-1]
    rep = gu.judge_all(x.reshape(-1, D), s, bits, p1.reshape(-1, nw), p2.reshape(-1, nw), nrm.reshape(-1))
    _say(rep.summary())
    assert rep.n_vectors == spec.rows
    assert rep.ok(gu.capped(rep.n_codes, rep.flips), gu.NORM_REL_TOL), rep.summary()
