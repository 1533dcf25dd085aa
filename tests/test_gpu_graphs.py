"""The codec and the attention under HIP graph capture.

The library allocates nothing and records no memset, so its launches can be captured into a
graph by callers that replay a fixed sequence (a decode step, a prefill chunk). The graph
below captures an encode into a cache window, a decode of that window and the
allocation-free attention over the captured caches; it is replayed several times with
eager work (encodes of other inputs into other buffers) and synchronisations between the
replays, and every replay must reproduce the eager results bit for bit (the kernels are
deterministic). The eager results themselves are checked against the oracle by the parity
tests; here the encode is also judged against the oracle once.
"""
import math

import pytest
import torch

import residual_vq_encode_amd as kvq
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 4), (96, 3), (100, 2)])
def test_captured_codec_and_attention_replay_exactly(d, bits):
    _say(f"graph replay d={d} bits={bits}")
    B, H, S, S_cap, s_off = 2, 4, 200, 512, 37
    sk, sv = synth.signs(11 + d, d).numpy(), synth.signs(12 + d, d).numpy()
    cbk, cbv = kvq.build_codebooks(d, bits, sk), kvq.build_codebooks(d, bits, sv)
    x = synth.tensor(synth.TensorSpec(B, H, S, d, "gauss_outliers", 31 + d + bits), device=DEV)
    xv = synth.tensor(synth.TensorSpec(B, H, S, d, "gauss", 32 + d + bits), device=DEV)
    nw = cbk.n_words
    caches = [torch.zeros((B, H, S_cap, nw), dtype=torch.int32, device=DEV) for _ in range(4)]
    norms = [torch.zeros((B, H, S_cap), dtype=torch.float32, device=DEV) for _ in range(2)]
    out = torch.empty((B, H, S, d), dtype=torch.float16, device=DEV)
    pow2 = d & (d - 1) == 0
    q = synth.tensor(synth.TensorSpec(B, 2 * H, 1, d, "gauss", 33 + d), device=DEV)
    att = torch.zeros_like(q)

    def step(stream):
        kvq.kvq_rvq_encode_pack(cbk, x, caches[0], caches[1], norms[0], s_off, stream)
        kvq.kvq_rvq_encode_pack(cbv, xv, caches[2], caches[3], norms[1], s_off, stream)
        kvq.kvq_rvq_unpack_decode(cbk, caches[0], caches[1], norms[0], out, s_off, stream)
        if pow2:  # the attention takes powers of two only
            kvq.kvq_rvq_attend_noalloc(cbk, cbv, q, (caches[0], caches[1], norms[0]),
                                       (caches[2], caches[3], norms[1]), s_off + S, 1.0 / math.sqrt(d), att,
                                       stream)

    # eager reference
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [t.clone() for t in caches + norms] + [out.clone(), att.clone()]
    rows = x.reshape(-1, d)
    win = slice(s_off, s_off + S)
    rep = gu.judge_all(rows, sk, bits, caches[0][:, :, win].reshape(rows.shape[0], -1),
                       caches[1][:, :, win].reshape(rows.shape[0], -1), norms[0][:, :, win].reshape(-1))
    assert rep.ok(gu.capped(rep.n_codes, rep.flips), gu.NORM_REL_TOL), rep.summary()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for t in caches + norms:
            t.zero_()
        out.zero_()
        att.zero_()
        with torch.cuda.graph(g, stream=side):
            step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other = synth.tensor(synth.TensorSpec(B, H, S, d, "gauss", 99 + d), device=DEV)
    scratch = [torch.empty_like(caches[0]), torch.empty_like(caches[1]), torch.empty_like(norms[0])]
    for replay in range(4):
        for t in caches + norms:  # the graph must rewrite the window it owns
            t[:, :, win].fill_(-7)
        out.fill_(0)
        att.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        got = caches + norms + [out, att]
        for i, (u, v) in enumerate(zip(got, want)):
            assert torch.equal(u[:, :, win] if i < 6 else u, v[:, :, win] if i < 6 else v), (replay, i)
        # eager work between the replays, on other buffers
        kvq.kvq_rvq_encode_pack(cbk, other, scratch[0], scratch[1], scratch[2], 0, None)
        torch.cuda.synchronize()
