"""The allocation-free attention entry point kvq_rvq_attend_noalloc, called through the C ABI,
against kvq_rvq_attend with a caller's workspace on the same inputs: the same checks, plan
and kernels, so the outputs must be identical bit for bit. Two calls in a row, the second on
smaller sizes (so it runs over the scratch the first call left behind), then a call on the
vector path; and plans larger than the scratch are refused on the host."""
import math

import pytest
import torch

import residual_vq_encode_amd as kvq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _caches(B, Hkv, S_cap, d, bits, seed):
    sk = synth.signs(31 + seed, d).numpy()
    sv = synth.signs(37 + seed, d).numpy()
    cbk, cbv = kvq.build_codebooks(d, bits, sk), kvq.build_codebooks(d, bits, sv)
    xk = synth.tensor(synth.TensorSpec(B, Hkv, S_cap, d, "gauss", 41 + seed), device=DEV)
    xv = synth.tensor(synth.TensorSpec(B, Hkv, S_cap, d, "gauss", 43 + seed), device=DEV)
    return cbk, cbv, kvq.encode(xk, cbk), kvq.encode(xv, cbv)


def _both(d, bits, B, Hq, Hkv, Sq, S_cap, S_kv, seed):
    cbk, cbv, kc, vc = _caches(B, Hkv, S_cap, d, bits, seed)
    q = synth.tensor(synth.TensorSpec(B, Hq, Sq, d, "gauss", 47 + seed), device=DEV)
    scale = 1.0 / math.sqrt(d)
    need = kvq.kvq_rvq_attend_workspace_size(d, bits, B, Hq, Sq, Hkv, S_kv)
    assert need <= kvq.ATTEND_SCRATCH_BYTES
    ref = kvq.attend(q, kc, vc, cbk, cbv, S_kv, scale)
    out = torch.full_like(q, float("nan"))
    kvq.kvq_rvq_attend_noalloc(cbk, cbv, q, kc, vc, S_kv, scale, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(ref.float()).all())
    assert torch.equal(out, ref), float((out.float() - ref.float()).abs().max())
    return need


def test_noalloc_matches_workspace_call_twice_then_smaller():
    # one decode step of a GQA layer: 32 query heads over 8 key/value heads x 32768 positions
    _say("noalloc: [1,32,1,128] over [1,8,32768,128], b=2")
    big = _both(128, 2, B=1, Hq=32, Hkv=8, Sq=1, S_cap=32768, S_kv=32768, seed=1)
    # right after it, smaller sizes over the same scratch
    _say("noalloc: [2,8,3,128] over [2,2,1200,128] (S_kv=1000), b=2")
    small = _both(128, 2, B=2, Hq=8, Hkv=2, Sq=3, S_cap=1200, S_kv=1000, seed=2)
    assert small < big
    # the vector path (3 bits)
    _say("noalloc: [1,4,2,256] over [1,2,700,256] (S_kv=650), b=3")
    _both(256, 3, B=1, Hq=4, Hkv=2, Sq=2, S_cap=700, S_kv=650, seed=3)


def test_noalloc_refuses_plans_beyond_the_scratch():
    d, bits, B, Hq, Sq, Hkv, S_kv = 128, 2, 1, 32, 4096, 8, 4096
    assert kvq.kvq_rvq_attend_workspace_size(d, bits, B, Hq, Sq, Hkv, S_kv) > kvq.ATTEND_SCRATCH_BYTES
    cbk, cbv, kc, vc = _caches(B, Hkv, S_kv, d, bits, 4)
    q = synth.tensor(synth.TensorSpec(B, Hq, Sq, d, "gauss", 5), device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_rvq_attend_noalloc(cbk, cbv, q, kc, vc, S_kv, 0.1, out)
    assert e.value.status == -4
