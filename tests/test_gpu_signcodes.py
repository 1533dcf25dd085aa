"""GPU parity of the 1-bit sign-code encoders against the oracle (oracle/signcodes.py).

RaBitQ-style code (kvq_rabitq_encode_pack): bit j = [y_j >= 0] of the rotated vector. The
device decides on its float32 butterfly, the oracle on the exact rotation rounded once, so
a bit may differ only where the oracle's y lies within 1e-5 sigma1 of the boundary 0 (the
codec's rule at its middle boundary), at most flip_cap of the bits. Norms within 1e-6.

QJL sketch (kvq_qjl_encode_pack): bit j = [(S x)_j >= 0]. The device multiplies the fp16
values exactly and sums in float32, so its sum is within d 2^-24 sum_i |S_ji x_i| of the
exact dot; a bit may differ from the exact sign only inside that bound. The fp16 norm must
be the fp16 rounding of a value within 1e-6 (relative) of the exact norm.

Inputs for degenerate cases (zeros, one-hot, small integers) are exact on both sides and
must match with no difference at all.
"""
import math

import numpy as np
import pytest
import torch

import residual_vq_encode_amd as kvq
import synth
from oracle import packing, signcodes
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
DEV = "cuda"
D_ALL = [8, 16, 32, 64, 128, 256, 512, 1024]
QJL_SHAPES = [(d, m) for d in (32, 64, 128, 256) for m in range(32, 257, 32)
              if 2 * m * d + 4 * 32 * d * 2 <= 160 * 1024]


def _say(msg):
    print(msg, flush=True)


def _window_rows(t, S, s_offset):
    B, H = t.shape[:2]
    return t[:, :, s_offset:s_offset + S].reshape(B * H * S, *t.shape[3:])


# ------------------------------------------------------------------------------ RaBitQ code

def check_rabitq(x, signs, S_cap=None, s_offset=0, max_flip=None):
    B, H, S, D = x.shape
    S_cap = S if S_cap is None else S_cap
    cb = kvq.build_codebooks(D, 1, signs)
    p = torch.full((B, H, S_cap, cb.n_words), -1, dtype=torch.int32, device=DEV)
    nrm = torch.full((B, H, S_cap), float("nan"), dtype=torch.float32, device=DEV)
    kvq.kvq_rabitq_encode_pack(cb, x, p, nrm, s_offset)
    torch.cuda.synchronize()
    rows = x.detach().cpu().numpy().reshape(-1, D)
    ref = signcodes.rabitq_encode(rows, np.asarray(signs, np.int8))
    pw = gu.as_u32(_window_rows(p, S, s_offset))
    nw = _window_rows(nrm, S, s_offset).cpu().numpy()
    assert not (pw & packing.padding_mask(D, 1)[None, :]).any(), "padding bits must be zero"
    diff = packing.unpack(pw, 1, D) != ref["bits"]
    n_diff = int(diff.sum())
    cap = gu.capped(diff.size, int(diff.sum())) if max_flip is None else max_flip
    assert n_diff <= cap * diff.size, (n_diff, diff.size)
    if n_diff:
        assert np.all(np.abs(ref["y"][diff]) <= 1e-5 / math.sqrt(D)), "bit differs outside the window"
    n64 = ref["norm64"]
    assert np.all(np.abs(nw - n64) <= gu.NORM_REL_TOL * n64)
    if S_cap > S:  # nothing outside the window was written
        assert bool((p[:, :, :s_offset] == -1).all()) and bool((p[:, :, s_offset + S:] == -1).all())
        assert bool(torch.isnan(nrm[:, :, :s_offset]).all()) and bool(torch.isnan(nrm[:, :, s_offset + S:]).all())
    return n_diff, diff.size


@pytest.mark.parametrize("d", D_ALL)
def test_rabitq_grid(d):
    _say(f"rabitq d={d}")
    for n in (1, 33, 200):
        x = synth.tensor(synth.TensorSpec(1, 2, n, d, "gauss_outliers", 40 + d + n), device=DEV)
        check_rabitq(x, synth.signs(4100 + d, d).numpy())


@pytest.mark.parametrize("d", [8, 32, 128, 1024])
def test_rabitq_degenerate_inputs_exact(d):
    """Zero vectors, one-hot vectors, pairs e_i +- e_j (exact zeros in y) and constants:
    every value the device sums is exact, so no bit may differ."""
    _say(f"rabitq degenerate d={d}")
    rows = [np.zeros(d)]
    for j in (0, 1, d // 2, d - 1):
        e = np.zeros(d)
        e[j] = 1.0
        rows += [e, -2.0 * e]
    for i, j in ((0, 1), (3, 5 % d), (1, d - 1)):
        e = np.zeros(d)
        e[i] += 1.0
        e[j] += 1.0
        f = np.zeros(d)
        f[i] += 1.0
        f[j] -= 1.0
        rows += [e, f]
    rows += [np.full(d, 0.5), np.full(d, -65504.0), np.full(d, 2.0 ** -24)]
    x = torch.from_numpy(np.array(rows, np.float16).reshape(1, 1, len(rows), d)).to(DEV)
    for s in (np.ones(d, np.int8), synth.signs(17 + d, d).numpy()):
        check_rabitq(x, s, max_flip=0.0)


def test_rabitq_llama_layer():
    w = synth.WORKLOADS["llama_layer"]
    _say("rabitq llama_layer [1,32,8192,128]")
    x = synth.tensor(w.tensors[0], device=DEV)
    n_diff, n = check_rabitq(x, synth.signs(w.sign_seed, 128).numpy())
    _say(f"  differing bits {n_diff} of {n}")


def test_rabitq_cache_window_and_ragged():
    _say("rabitq window")
    x = synth.tensor(synth.TensorSpec(3, 5, 37, 128, "gauss", 91), device=DEV)
    check_rabitq(x, synth.signs(12, 128).numpy(), S_cap=100, s_offset=41)


# -------------------------------------------------------------------------------- QJL sketch

def check_qjl(x, sketch, S_cap=None, s_offset=0, max_diff=None):
    B, H, S, D = x.shape
    m = sketch.shape[0]
    S_cap = S if S_cap is None else S_cap
    p = torch.full((B, H, S_cap, m // 32), -1, dtype=torch.int32, device=DEV)
    nrm = torch.full((B, H, S_cap), float("nan"), dtype=torch.float16, device=DEV)
    kvq.kvq_qjl_encode_pack(sketch, x, p, nrm, s_offset)
    torch.cuda.synchronize()
    rows = x.detach().cpu().numpy().reshape(-1, D)
    ref = signcodes.qjl_encode(rows, sketch.cpu().numpy())
    pw = gu.as_u32(_window_rows(p, S, s_offset))
    nw = _window_rows(nrm, S, s_offset).cpu().numpy()
    diff = packing.unpack(pw, 1, m) != ref["bits"]
    n_diff = int(diff.sum())
    if n_diff:
        bound = D * 2.0 ** -24 * ref["absdots"][diff]
        assert np.all(np.abs(ref["dots"][diff]) <= bound), "sign differs outside the float32 error bound"
    if max_diff is not None:
        assert n_diff <= max_diff, n_diff
    n64 = ref["norm64"]
    with np.errstate(over="ignore"):
        lo = (n64 * (1 - 1e-6)).astype(np.float16)
        hi = (n64 * (1 + 1e-6)).astype(np.float16)
    ok = (nw == lo) | (nw == hi)
    assert ok.all(), (nw[~ok][:4], n64[~ok][:4])
    if S_cap > S:
        assert bool((p[:, :, :s_offset] == -1).all()) and bool((p[:, :, s_offset + S:] == -1).all())
        assert bool(torch.isnan(nrm[:, :, :s_offset]).all()) and bool(torch.isnan(nrm[:, :, s_offset + S:]).all())
    return n_diff, diff.size


def _sketch(m, d, seed):
    return synth.tensor(synth.TensorSpec(1, 1, m, d, "gauss", seed), device=DEV).reshape(m, d).contiguous()


@pytest.mark.parametrize("d,m", QJL_SHAPES)
def test_qjl_grid(d, m):
    _say(f"qjl d={d} m={m}")
    sk = _sketch(m, d, 500 + d + m)
    for n in (1, 31, 33, 100):
        x = synth.tensor(synth.TensorSpec(1, 1, n, d, "gauss_outliers", 600 + d + m + n), device=DEV)
        check_qjl(x, sk)


@pytest.mark.parametrize("d", [32, 128, 256])
def test_qjl_exact_inputs(d):
    """Small-integer sketch and keys (every product and partial sum exact in float32),
    zero keys (of either sign) and one-hot keys: no bit may differ, exact zeros set the bit."""
    _say(f"qjl exact d={d}")
    m = 64
    rng = np.random.default_rng(d)
    S = rng.integers(-2, 3, (m, d)).astype(np.float16)
    X = rng.integers(-3, 4, (70, d)).astype(np.float16)
    X[0] = 0.0
    X[1] = 0.0
    X[1, d - 1] = 1.0
    X[2] = 0.0
    X[2, 0] = -1.0
    X[3] = np.float16(-0.0)  # every product with the all-positive row 0 is -0: the dot is 0, bit set
    S[0] = 1.0
    x = torch.from_numpy(X.reshape(1, 1, 70, d)).to(DEV)
    n_diff, _ = check_qjl(x, torch.from_numpy(S).to(DEV), max_diff=0)


def test_qjl_tiny_and_huge_values():
    """fp16 subnormal keys (the products are exact in float32) and keys whose norm
    overflows fp16 (stored as inf on both sides)."""
    _say("qjl subnormal / overflow")
    d, m = 128, 128
    sk = _sketch(m, d, 71)
    rng = np.random.default_rng(5)
    X = (rng.standard_normal((64, d)) * 2.0 ** -20).astype(np.float16)  # mostly subnormal
    X[60:] = np.float16(60000.0) * np.sign(rng.standard_normal((4, d))).astype(np.float16)
    x = torch.from_numpy(X.reshape(1, 1, 64, d)).to(DEV)
    check_qjl(x, sk)


def test_qjl_llama_layer():
    """The whole Llama layer's keys [1,32,8192,128], m = 128 (one bit per coordinate)."""
    w = synth.WORKLOADS["llama_layer"]
    _say("qjl llama_layer [1,32,8192,128] m=128")
    x = synth.tensor(w.tensors[0], device=DEV)
    n_diff, n = check_qjl(x, _sketch(128, 128, 707))
    _say(f"  differing bits {n_diff} of {n}")
    assert n_diff <= 1e-6 * n


def test_qjl_cache_window_and_ragged():
    _say("qjl window")
    x = synth.tensor(synth.TensorSpec(3, 5, 37, 64, "gauss", 92), device=DEV)
    check_qjl(x, _sketch(96, 64, 93), S_cap=100, s_offset=41)
