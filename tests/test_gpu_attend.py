"""GPU parity of kvq_rvq_attend (attention over packed key/value caches) against the
oracle's plain definition (oracle/attend.py).

Both sides read the same packed caches, written by the oracle's encoder and uploaded. The
device works in float32 in the rotated domain (rotated query, per-coordinate table lookups
and FMAs, online softmax in base 2, chunked and merged); the oracle in float64 on the
reconstructed keys and values. Tolerance per output vector: |gpu - oracle| <=
2^-10 |oracle| + 1e-3 max|oracle vector|. The first term is one fp16 step (the two sides
round slightly different values to fp16). The second covers the float32 arithmetic: scores
carry a relative error of a few 1e-6 of |q| |k| scale, so the weights and hence the output
move by about 1e-4 of the output's scale, well inside 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import residual_vq_encode_amd as kvq
import synth
from oracle import attend as oatt
from oracle import codebooks as ocb
from oracle import rvq

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _cache(B, Hkv, S_cap, d, bits, seed, signs, kind="gauss"):
    t = ocb.build_tables(d, bits)
    x = synth.rows(synth.TensorSpec(B, Hkv, S_cap, d, kind, seed)).numpy()
    e = rvq.encode(x, signs, t)
    nw = e["packed1"].shape[1]
    host = (e["packed1"].reshape(B, Hkv, S_cap, nw), e["packed2"].reshape(B, Hkv, S_cap, nw),
            e["norms"].reshape(B, Hkv, S_cap))
    dev = tuple(torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a).to(DEV) for a in host)
    return host, dev, t


def _check(d, bits, B, Hq, Hkv, Sq, S_cap, S_kv, seed=0, scale=None, kind="gauss"):
    sk = synth.signs(700 + d + seed, d).numpy()
    sv = synth.signs(800 + d + seed, d).numpy()
    kh, kd, t = _cache(B, Hkv, S_cap, d, bits, 900 + seed, sk, kind)
    vh, vd, _ = _cache(B, Hkv, S_cap, d, bits, 950 + seed, sv, kind)
    q = synth.tensor(synth.TensorSpec(B, Hq, Sq, d, "gauss", 990 + seed), device=DEV)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    cbk, cbv = kvq.build_codebooks(d, bits, sk), kvq.build_codebooks(d, bits, sv)
    out = kvq.attend(q, kd, vd, cbk, cbv, S_kv, scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = oatt.attend(q.cpu().numpy(), kh, vh, sk, sv, t, t, S_kv, scale).astype(np.float64)
    assert np.all(np.isfinite(got))
    rowmax = np.max(np.abs(want), axis=-1, keepdims=True)
    excess = np.abs(got - want) - (2.0 ** -10 * np.abs(want) + 1e-3 * rowmax)
    worst = float(np.max(excess))
    assert worst <= 0.0, (worst, float(np.max(np.abs(got - want) / np.maximum(rowmax, 1e-30))))
    return out


@pytest.mark.parametrize("d", [8, 16, 32, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_attend_grid(d, bits):
    _say(f"attend grid d={d} bits={bits}")
    _check(d, bits, B=2, Hq=4, Hkv=2, Sq=2, S_cap=45, S_kv=37, seed=d + bits)


# (Hq, Hkv, Sq): query vectors per key/value head 1, 2, 4 (all from Sq) and 6 (2 heads x 3
# positions), so that waves carry 1, 2, 4 and 2 queries and the query-to-head map is mixed.
@pytest.mark.parametrize("d", [8, 16, 32, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("bits", [1, 3])
@pytest.mark.parametrize("shape", [(3, 3, 1), (6, 3, 1), (2, 2, 4), (4, 2, 3)])
def test_attend_queries_per_wave(d, bits, shape):
    Hq, Hkv, Sq = shape
    _say(f"attend d={d} bits={bits} Hq={Hq} Hkv={Hkv} Sq={Sq}")
    _check(d, bits, B=2, Hq=Hq, Hkv=Hkv, Sq=Sq, S_cap=70, S_kv=61, seed=3 * d + bits + Hq)


@pytest.mark.parametrize("S_kv", [1, 2, 15, 16, 17, 127, 128, 129, 1000, 4097])
def test_attend_lengths(S_kv):
    _say(f"attend S_kv={S_kv}")
    _check(128, 2, B=1, Hq=8, Hkv=2, Sq=1, S_cap=S_kv + 3, S_kv=S_kv, seed=S_kv)


@pytest.mark.parametrize("scale", [0.0, 0.35, -0.2])
def test_attend_scales(scale):
    _say(f"attend scale={scale}")
    _check(64, 4, B=1, Hq=2, Hkv=1, Sq=3, S_cap=300, S_kv=290, seed=5, scale=scale)


def test_attend_outlier_channels_and_laplace():
    _say("attend outliers / laplace heads")
    _check(128, 2, B=1, Hq=4, Hkv=4, Sq=1, S_cap=600, S_kv=600, seed=6, kind="gauss_outliers")
    _check(128, 4, B=1, Hq=8, Hkv=8, Sq=1, S_cap=500, S_kv=450, seed=7, kind="gauss_laplace_heads")


def test_attend_llama_decode_step():
    """One decode step of a Llama-style GQA layer: 32 query heads over 8 key/value heads,
    8192 cached positions."""
    _say("attend llama decode step Hq=32 Hkv=8 S_kv=8192")
    _check(128, 2, B=1, Hq=32, Hkv=8, Sq=1, S_cap=8192, S_kv=8192, seed=8)


def test_attend_long_context_many_chunks():
    """One query over 300k positions: about 1900 chunks meet in the combine pass."""
    _say("attend long context S_kv=300000 d=64")
    _check(64, 2, B=1, Hq=1, Hkv=1, Sq=1, S_cap=300000, S_kv=299999, seed=9)


def test_attend_ignores_positions_past_s_kv_and_is_deterministic():
    d, bits, S_cap, S_kv = 128, 2, 200, 150
    sk = synth.signs(1, d).numpy()
    kh, kd, _ = _cache(1, 2, S_cap, d, bits, 40, sk)
    vh, vd, _ = _cache(1, 2, S_cap, d, bits, 41, sk)
    cb = kvq.build_codebooks(d, bits, sk)
    q = synth.tensor(synth.TensorSpec(1, 4, 2, d, "gauss", 42), device=DEV)
    a = kvq.attend(q, kd, vd, cb, cb, S_kv)
    kd2 = tuple(t.clone() for t in kd)
    vd2 = tuple(t.clone() for t in vd)
    for t in kd2 + vd2:
        t[:, :, S_kv:] = 12345 if t.dtype == torch.int32 else 7.0
    b = kvq.attend(q, kd2, vd2, cb, cb, S_kv)
    c = kvq.attend(q, kd, vd, cb, cb, S_kv)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
