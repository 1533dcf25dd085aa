"""Full-size GPU parity of the decoders and of cache-window writes, at the workloads' own
sizes and in the launch configuration the bench uses (persistent grids whose waves walk many
tiles), against the oracle on every vector.

Decoders are fed the oracle's packed words and norms (uploaded), never the device's own, so
a flipped code on the encode side cannot mask or cause a decode difference (VeloxQuant-MLX
blog, "rvq" tag page, "Bit-exactness, checked the boring way": identical output on every
shape). Tolerances are those of the other parity tests: 1e-3 absolute on unit
reconstructions, 1e-3 relative to the vector's norm with norms; codes bit-exact except
in-window one-level flips, at most 1e-6 of them; cells outside a cache window untouched.
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


def _say(msg):
    print(msg, flush=True)


def _workload(name):
    w = synth.WORKLOADS[name]
    spec = w.tensors[0]
    return spec, synth.signs(w.sign_seed, spec.D).numpy()


@pytest.mark.parametrize("bits", [1, 4])
def test_gqa_long_decode_every_vector(bits):
    """The GQA workload's caches [1,8,32768,128] at b = 1 and 4 (4 and 16 words per stream),
    decoded from the oracle's words: 262,144 vectors, 16,384 tiles over the resident grid."""
    spec, s = _workload("gqa_long")
    _say(f"decode gqa_long [1,8,32768,128] b={bits}: oracle words, every vector")
    ref = rvq.encode(synth.rows(spec).numpy(), s, gu.tables(128, bits))
    err_unit, err_rel = gu.check_decode_from_oracle_words(ref, s, bits, (spec.B, spec.H, spec.S, spec.D))
    _say(f"max |err| unit {err_unit:.3e}, relative to the norm {err_rel:.3e}")


def test_llama_layer_b3_encode_and_decode_every_vector():
    """[1,32,8192,128] at 3 bits (10 codes per word, words straddling the lanes): the encode
    judged on every vector, the decode fed the oracle's words."""
    spec, s = _workload("llama_layer")
    _say("llama_layer [1,32,8192,128] b=3: encode and decode, every vector")
    x = synth.tensor(spec, device=DEV)
    rep, _, ref = gu.check_encode(x, s, 3, max_flip=gu.MAX_FLIP_FRACTION)
    _say(rep.summary())
    gu.check_decode_from_oracle_words(ref, s, 3, tuple(x.shape))


def test_llama_layer_single_stage_decode_every_vector():
    """The single-stage codec's [1,32,8192,128] b = 2 cache decoded from the oracle's words,
    in unit mode and with norms."""
    spec, s = _workload("llama_layer")
    _say("llama_layer [1,32,8192,128] single-stage b=2 decode, every vector")
    ref = rvq.encode_mse(synth.rows(spec).numpy(), s, gu.tables(128, 2))
    gu.check_decode_mse_from_oracle_words(ref, s, 2, (spec.B, spec.H, spec.S, spec.D))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_llama_layer_into_cache_window(bits):
    """The Llama layer [1,32,8192,128] written into caches with S_cap = 8400 at s_offset = 200
    (the general row mapping, every wave walking several tiles): every vector's codes against
    the oracle, cells outside the window untouched, and the window decoded back from the
    oracle's words in the same geometry."""
    spec, s = _workload("llama_layer")
    B, H, S, D = spec.B, spec.H, spec.S, spec.D
    S_cap, off = 8400, 200
    _say(f"llama_layer into a cache window S_cap={S_cap} s_offset={off} b={bits}")
    x = synth.tensor(spec, device=DEV)
    p1, p2, nrm = gu.gpu_encode(x, s, bits, S_cap=S_cap, s_offset=off, fill=-1)
    nw = p1.shape[-1]
    win = slice(off, off + S)
    rep = gu.judge_all(x.reshape(-1, D), s, bits, p1[:, :, win].reshape(-1, nw), p2[:, :, win].reshape(-1, nw),
                       nrm[:, :, win].reshape(-1))
    _say(rep.summary())
    assert rep.n_vectors == spec.rows
    assert rep.ok(gu.MAX_FLIP_FRACTION, gu.NORM_REL_TOL), rep.summary()
    outside = torch.ones(S_cap, dtype=torch.bool, device=DEV)
    outside[win] = False
    assert bool((p1[:, :, outside] == -1).all()) and bool((p2[:, :, outside] == -1).all())
    assert bool(torch.isnan(nrm[:, :, outside]).all())
    del p1, p2, nrm

    ref = rvq.encode(synth.rows(spec).numpy(), s, gu.tables(D, bits))
    cb = kvq.build_codebooks(D, bits, s)
    c1 = torch.zeros((B, H, S_cap, nw), dtype=torch.int32, device=DEV)
    c2 = torch.zeros_like(c1)
    cn = torch.zeros((B, H, S_cap), dtype=torch.float32, device=DEV)
    c1[:, :, win] = torch.from_numpy(ref["packed1"].view(np.int32)).reshape(B, H, S, nw).to(DEV)
    c2[:, :, win] = torch.from_numpy(ref["packed2"].view(np.int32)).reshape(B, H, S, nw).to(DEV)
    cn[:, :, win] = torch.from_numpy(ref["norms"]).reshape(B, H, S).to(DEV)
    t = gu.tables(D, bits)
    out = torch.empty((B, H, S, D), dtype=torch.float16, device=DEV)
    kvq.kvq_rvq_unpack_decode(cb, c1, c2, None, out, s_offset=off)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, D).astype(np.float64)
    want = rvq.decode(ref["packed1"], ref["packed2"], None, s, t).astype(np.float64)
    assert float(np.max(np.abs(got - want))) <= gu.DECODE_UNIT_ATOL
    kvq.kvq_rvq_unpack_decode(cb, c1, c2, cn, out, s_offset=off)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, D).astype(np.float64)
    want = rvq.decode(ref["packed1"], ref["packed2"], ref["norms"], s, t).astype(np.float64)
    n = ref["norms"].astype(np.float64)[:, None]
    assert float(np.max(np.abs(got - want) - (gu.DECODE_UNIT_ATOL * n + 2.0 ** -24))) <= 0.0
