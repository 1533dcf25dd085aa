"""Every encoder's output for a vector depends on that vector alone: not on the tensor shape
it arrives in, on where it falls in a wave's tile (so on the grid), or on whether it is
written contiguously or into a window of a larger cache (a different kernel instantiation).
The same vectors encoded through all of those launch configurations must give the same
words and norms bit for bit, and decoding a window must give the same fp16 values as
decoding the contiguous cache. (The oracle parity tests bound each result against the
definition; these tests pin down that no launch-dependent path changes a single bit.)"""
import pytest
import torch

import residual_vq_encode_amd as kvq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128


def _say(msg):
    print(msg, flush=True)


def _x(B=2, H=3, S=77, seed=31, d=D):
    return synth.tensor(synth.TensorSpec(B, H, S, d, "gauss_outliers", seed), device=DEV)


def _bits_f32(t):
    return t.contiguous().view(torch.int32)


def _enc(kind, cb, x, S_cap=None, s_offset=0, sketch=None):
    """Encode x [B, H, S, d] into a cache of capacity S_cap at s_offset; returns the window's
    (words..., norm bits) as [B*H*S, ...] tensors."""
    B, H, S, d = x.shape
    S_cap = S if S_cap is None else S_cap
    if kind == "qjl":
        m = sketch.shape[0]
        p = torch.full((B, H, S_cap, m // 32), -1, dtype=torch.int32, device=DEV)
        n = torch.full((B, H, S_cap), float("nan"), dtype=torch.float16, device=DEV)
        kvq.kvq_qjl_encode_pack(sketch, x, p, n, s_offset)
        outs = [p]
        norms = n.view(torch.int16)
    else:
        p1 = torch.full((B, H, S_cap, cb.n_words), -1, dtype=torch.int32, device=DEV)
        p2 = torch.full_like(p1, -1)
        n = torch.full((B, H, S_cap), float("nan"), dtype=torch.float32, device=DEV)
        if kind == "rvq":
            kvq.kvq_rvq_encode_pack(cb, x, p1, p2, n, s_offset)
            outs = [p1, p2]
        elif kind == "mse":
            kvq.kvq_mse_encode_pack(cb, x, p1, n, s_offset)
            outs = [p1]
        else:
            kvq.kvq_rabitq_encode_pack(cb, x, p1, n, s_offset)
            outs = [p1]
        norms = _bits_f32(n)
    torch.cuda.synchronize()
    win = [o[:, :, s_offset:s_offset + S].reshape(B * H * S, -1) for o in outs]
    return win + [norms[:, :, s_offset:s_offset + S].reshape(B * H * S)]


CASES = [("rvq", 1), ("rvq", 2), ("rvq", 3), ("rvq", 4), ("mse", 2), ("mse", 3), ("rabitq", 1), ("qjl", 1)]


@pytest.mark.parametrize("kind,bits", CASES)
def test_encoders_do_not_depend_on_the_launch_configuration(kind, bits):
    _say(f"launch invariance {kind} b={bits}")
    x = _x()
    B, H, S, d = x.shape
    cb = kvq.build_codebooks(d, bits, synth.signs(55, d).numpy())
    sketch = None
    if kind == "qjl":
        sketch = synth.tensor(synth.TensorSpec(1, 1, 64, d, "gauss", 56), device=DEV).reshape(64, d).contiguous()
    ref = _enc(kind, cb, x, sketch=sketch)

    def same(got, what):
        for a, b in zip(ref, got):
            assert torch.equal(a, b), what

    # the same memory seen as other [B, H, S] shapes
    same(_enc(kind, cb, x.reshape(B * H, 1, S, d), sketch=sketch), "[B*H, 1, S]")
    same(_enc(kind, cb, x.reshape(1, 1, B * H * S, d), sketch=sketch), "[1, 1, B*H*S]")
    # written into windows of larger caches (the general row mapping)
    for S_cap, off in ((S + 23, 11), (S + 1, 1), (4 * S, 3 * S)):
        same(_enc(kind, cb, x, S_cap=S_cap, s_offset=off, sketch=sketch), f"window S_cap={S_cap} s_offset={off}")
    # shifted against the tiles: 5 other vectors in front
    flat = x.reshape(1, 1, B * H * S, d)
    pad = _x(1, 1, 5, seed=32)
    shifted = torch.cat([pad, flat], dim=2).contiguous()
    got = _enc(kind, cb, shifted, sketch=sketch)
    same([g[5:] for g in got], "shifted by 5 vectors")
    # one vector at a time, into its own window of a one-row-per-step cache
    for v in (0, 1, 63, 64, B * H * S - 1):
        one = flat[:, :, v:v + 1].contiguous()
        got = _enc(kind, cb, one, S_cap=7, s_offset=6, sketch=sketch)
        for a, b in zip(ref, got):
            assert torch.equal(a[v:v + 1], b), f"vector {v} alone"


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("stages", [1, 2])
def test_decoders_do_not_depend_on_the_launch_configuration(bits, stages):
    _say(f"decode invariance b={bits} stages={stages}")
    x = _x(seed=41)
    B, H, S, d = x.shape
    cb = kvq.build_codebooks(d, bits, synth.signs(57, d).numpy())
    S_cap, off = S + 30, 17
    p1 = torch.zeros((B, H, S_cap, cb.n_words), dtype=torch.int32, device=DEV)
    p2 = torch.zeros_like(p1)
    n = torch.zeros((B, H, S_cap), dtype=torch.float32, device=DEV)
    if stages == 2:
        kvq.kvq_rvq_encode_pack(cb, x, p1, p2, n, off)
    else:
        kvq.kvq_mse_encode_pack(cb, x, p1, n, off)

    def dec(pp1, pp2, nn, shape, s_offset):
        out = torch.empty(shape, dtype=torch.float16, device=DEV)
        if stages == 2:
            kvq.kvq_rvq_unpack_decode(cb, pp1, pp2, nn, out, s_offset)
        else:
            kvq.kvq_mse_unpack_decode(cb, pp1, nn, out, s_offset)
        torch.cuda.synchronize()
        return out.view(torch.int16).reshape(-1, d)

    from_window = dec(p1, p2, n, (B, H, S, d), off)
    # the same words copied into a contiguous cache
    c1 = p1[:, :, off:off + S].contiguous()
    c2 = p2[:, :, off:off + S].contiguous()
    cn = n[:, :, off:off + S].contiguous()
    assert torch.equal(from_window, dec(c1, c2, cn, (B, H, S, d), 0))
    # and seen as one long sequence
    flat = dec(c1.reshape(1, 1, B * H * S, -1), c2.reshape(1, 1, B * H * S, -1), cn.reshape(1, 1, B * H * S),
               (1, 1, B * H * S, d), 0)
    assert torch.equal(from_window, flat)
