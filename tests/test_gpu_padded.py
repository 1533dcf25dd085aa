"""GPU parity for head dimensions that are not powers of two (any d in [8, 1024]).

The Walsh-Hadamard rotation exists at powers of two only ("rvq" tag page, "The pipeline, as
it actually runs": normalise, then rotate by the sign-flipped Hadamard transform); such a
vector is rotated zero-padded to the next power of two P, all P rotated coordinates are
coded, and the decoder rotates the P reconstructed coordinates back and keeps the first d.
The oracle (oracle/rvq.py, pinned by tests/test_oracle_padding.py) implements that reading
directly; the device's dense loads, zero fill and partial-row stores are judged against it
with the same rule as every other shape: codes bit-exact up to in-window one-level flips,
norms within 1e-6 relative, decoders fed the oracle's words within 1e-3 on unit vectors.
"""
import numpy as np
import pytest
import torch

import residual_vq_encode_amd as kvq
import synth
from oracle import rvq
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
DEV = "cuda"
# Multiples of 8, whose rows are whole 16-byte chunks: rotation lengths 32 (24), 64 (40),
# 128 (80, 96, 120), 256 (192, 200), 1024 (576, 1016). Any other d, whose rows are moved as
# dwords and may start in the middle of one: 16 (9, 12), 32 (20), 64 (33), 128 (100, 127),
# 256 (130), 512 (257), 1024 (514, 1023).
D_PAD = [24, 40, 80, 96, 120, 192, 200, 576, 1016]
D_RAGGED = [9, 12, 20, 33, 100, 127, 130, 257, 514, 1023]


def _say(msg):
    print(msg, flush=True)


def _signs(seed, d):
    return synth.signs(seed, d).numpy()


@pytest.mark.parametrize("d", D_PAD + D_RAGGED)
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("n", [1, 37, 3001])
def test_padded_encode_decode(d, bits, n):
    """Encode against the oracle, then decode the oracle's words (unit and scaled) on both
    sides; n spans one vector, a ragged tile, and many tiles per wave with a ragged tail."""
    _say(f"padded d={d} bits={bits} n={n}")
    spec = synth.TensorSpec(1, 1, n, d, "gauss", 7 * d + bits + n)
    x = synth.tensor(spec, device=DEV)
    s = _signs(300 + d, d)
    cb = kvq.build_codebooks(d, bits, s)
    assert cb.n_words == kvq.n_words(d, bits) == -(-kvq.rotation_length(d) // (32 // bits))
    rep, _, ref = gu.check_encode(x, s, bits)
    assert ref["i1"].shape[1] == kvq.rotation_length(d)
    gu.check_decode_from_oracle_words(ref, s, bits, tuple(x.shape))


@pytest.mark.parametrize("d", D_PAD + D_RAGGED)
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_padded_single_stage(d, bits):
    _say(f"padded single stage d={d} bits={bits}")
    spec = synth.TensorSpec(2, 3, 45, d, "gauss_outliers", 5 * d + bits)
    x = synth.tensor(spec, device=DEV)
    s = _signs(400 + d, d)
    rep, _, ref = gu.check_encode_mse(x, s, bits)
    gu.check_decode_mse_from_oracle_words(ref, s, bits, tuple(x.shape))


def _degenerate_rows(d):
    rows = [np.zeros(d), np.ones(d), -np.ones(d), np.full(d, 65504.0), np.full(d, 2.0 ** -24)]
    for j in (0, 1, d // 2, d - 1):
        e = np.zeros(d)
        e[j] = 3.0
        rows.append(e)
        rows.append(-e)
    rows.append(np.where(np.arange(d) % 2 == 0, 1.0, -1.0))
    rows.append(np.full(d, -0.0))
    rows.append(np.random.default_rng(11).standard_normal(d) * 1e-4)
    return np.stack(rows).astype(np.float16)


@pytest.mark.parametrize("d", [24, 96, 576, 9, 127, 1023])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_padded_degenerate(d, bits):
    """Zero, constant, one-hot (at the first and last real coordinates too), extreme and
    subnormal rows: the padding's zeros must not change a norm or a code."""
    _say(f"padded degenerate d={d} bits={bits}")
    s = _signs(500 + d, d)
    x = torch.from_numpy(_degenerate_rows(d)).to(DEV).reshape(1, 1, -1, d)
    rep, _, ref = gu.check_encode(x, s, bits, max_flip=0.0)
    gu.check_decode_from_oracle_words(ref, s, bits, tuple(x.shape))


@pytest.mark.parametrize("d", [24, 96, 192, 576, 9, 100, 127, 1023])
@pytest.mark.parametrize("S,S_cap,s_offset", [(1, 9, 4), (70, 200, 13)])
def test_padded_cache_window(d, S, S_cap, s_offset):
    """Writes into a window of a larger cache (the row-mapped kernels), positions outside it
    untouched, and the window decoded back from the oracle's words."""
    bits = 3
    _say(f"padded window d={d} S={S} S_cap={S_cap} s_offset={s_offset}")
    x = synth.tensor(synth.TensorSpec(2, 3, S, d, "gauss", d + S), device=DEV)
    s = _signs(600 + d, d)
    nw = kvq.n_words(d, bits)
    p1, p2, nrm = gu.gpu_encode(x, s, bits, S_cap=S_cap, s_offset=s_offset, fill=-1)
    win = slice(s_offset, s_offset + S)
    rep, ref = gu.judge(x.cpu().numpy().reshape(-1, d), s, bits, gu.as_u32(p1[:, :, win]).reshape(-1, nw),
                        gu.as_u32(p2[:, :, win]).reshape(-1, nw), nrm[:, :, win].cpu().numpy().reshape(-1))
    assert rep.ok(gu.capped(rep.n_codes, rep.flips), gu.NORM_REL_TOL), rep.summary()
    outside = torch.ones(S_cap, dtype=torch.bool)
    outside[win] = False
    assert bool((p1[:, :, outside] == -1).all()) and bool((p2[:, :, outside] == -1).all())
    assert bool(torch.isnan(nrm[:, :, outside]).all())
    cb = kvq.build_codebooks(d, bits, s)
    c1 = torch.zeros_like(p1)
    c2 = torch.zeros_like(p2)
    c1[:, :, win] = torch.from_numpy(ref["packed1"].view(np.int32)).reshape(2, 3, S, nw).to(DEV)
    c2[:, :, win] = torch.from_numpy(ref["packed2"].view(np.int32)).reshape(2, 3, S, nw).to(DEV)
    # the output sits between guard elements (16 bytes on either side, so that it stays
    # 16-byte aligned): a store past the last real element of a row or of the run shows
    ne = 2 * 3 * S * d
    guard = torch.full((ne + 16,), 7.0, dtype=torch.float16, device=DEV)
    out = guard[8:8 + ne].view(2, 3, S, d)
    kvq.kvq_rvq_unpack_decode(cb, c1, c2, None, out, s_offset=s_offset)
    torch.cuda.synchronize()
    want = rvq.decode(ref["packed1"], ref["packed2"], None, s, gu.tables(d, bits)).astype(np.float64)
    assert np.max(np.abs(out.cpu().numpy().reshape(-1, d).astype(np.float64) - want)) <= gu.DECODE_UNIT_ATOL
    assert bool((guard[:8] == 7.0).all()) and bool((guard[8 + ne:] == 7.0).all())


@pytest.mark.parametrize("d,shape", [(96, (2, 8, 4096)), (80, (1, 8, 4099)), (576, (1, 4, 2048)),
                                     (192, (1, 8, 4096)), (100, (2, 8, 4096)), (127, (1, 8, 4099)),
                                     (1023, (1, 4, 2047))])
@pytest.mark.parametrize("bits", [2, 4])
def test_padded_every_vector_at_scale(d, shape, bits):
    """Larger launches (several rounds of the persistent grid): every vector judged, and
    a decode of the device's own output back to within the codec's distortion of x."""
    B, H, S = shape
    _say(f"padded at scale d={d} shape={shape} bits={bits}")
    x = synth.tensor(synth.TensorSpec(B, H, S, d, "gauss_outliers", d * 31 + bits), device=DEV)
    s = _signs(700 + d, d)
    p1, p2, nrm = gu.gpu_encode(x, s, bits)
    rows = x.reshape(-1, d)
    rep = gu.judge_all(rows, s, bits, p1.reshape(rows.shape[0], -1), p2.reshape(rows.shape[0], -1),
                       nrm.reshape(-1))
    assert rep.ok(gu.capped(rep.n_codes, rep.flips), gu.NORM_REL_TOL), rep.summary()
    cb = kvq.build_codebooks(d, bits, s)
    out = kvq.decode(p1, p2, nrm, cb)
    torch.cuda.synchronize()
    # relative reconstruction error of the two-stage codec (the mean over vectors): well
    # under that of stage 1 alone at this width, sqrt(mse_g), and far from 1
    xf = rows.float()
    err = (out.reshape(-1, d).float() - xf).norm(dim=1) / xf.norm(dim=1).clamp_min(1e-30)
    assert float(err.mean()) < float(np.sqrt(cb.mse_g))


def test_padded_empty_and_sign_code_rejected():
    cb = kvq.build_codebooks(96, 2)
    x = torch.empty((0, 4, 16, 96), dtype=torch.float16, device=DEV)
    p1, p2, nrm = kvq.encode(x, cb)
    assert p1.numel() == 0 and p1.shape[-1] == kvq.n_words(96, 2) == 8
    cb1 = kvq.build_codebooks(96, 1)
    x = torch.zeros((1, 1, 4, 96), dtype=torch.float16, device=DEV)
    p = torch.zeros((1, 1, 4, 4), dtype=torch.int32, device=DEV)
    n = torch.zeros((1, 1, 4), dtype=torch.float32, device=DEV)
    with pytest.raises((kvq.KvqError, ValueError)):
        kvq.kvq_rabitq_encode_pack(cb1, x, p, n)
