"""Helpers for the GPU parity tests: run the HIP path through the C ABI binding and judge
it against the oracle with the comparison rule of oracle/flips.py.

Inputs come from the seeded generator (synth) or are built by hand; the oracle always
consumes the very bytes the device consumed, copied back to the host. Decoders are fed
the oracle's packed words (uploaded), never words produced by the device.
"""
import math

import numpy as np
import torch

import residual_vq_encode_amd as kvq
from oracle import codebooks as ocb
from oracle import flips, rvq

# Tolerances. Codes: bit-exact except one-level flips of values within 1e-5 (relative, with
# the stage scale as the floor at the boundary 0) of a boundary, at most 1e-6 of all
# codes. Norms: the device sums squares of float16 inputs in float32 with 4 accumulators of
# 16 pair-products each plus a 2-level tree, relative error <= 18 * 2^-24 on the square,
# half that after the square root, plus one rounding: below 1e-6 relative.
REL_WINDOW = 1e-5
MAX_FLIP_FRACTION = 1e-6


# Tail probability a small sample's flip count may reach under the allowance below.
SMALL_SAMPLE_TAIL = 1e-3


def small_sample_allowance(n_codes: int) -> int:
    """Flips a sample smaller than a workload may carry: the smallest k >= 1 that a Poisson
    count with the cap's mean (1e-6 n) exceeds with probability at most 10^-3."""
    lam = MAX_FLIP_FRACTION * n_codes
    k, term = 0, math.exp(-lam)
    cdf = term
    while k < 1 or 1.0 - cdf > SMALL_SAMPLE_TAIL:
        k += 1
        term *= lam / k
        cdf += term
    return k


# Codes of the smallest workload: samples of at least this many are held to the rate itself.
WORKLOAD_CODES = 10 ** 7


def flip_cap(n_codes: int) -> float:
    """The 1e-6 cap is a rate over a workload (every workload has more than 10^7 codes),
    which a smaller sample cannot resolve: at the cap's rate a sample of 10^5 codes holds
    0.1 flips on average, and two now and then. A smaller sample is therefore held to the
    count that the cap's rate exceeds with probability 10^-3 (each flip still in-window and
    one level), and every sample of a session is pooled and the pool held to the rate
    itself (tests/test_zy_pooled_flips.py); workload-sized samples get the rate itself."""
    if n_codes >= WORKLOAD_CODES:
        return MAX_FLIP_FRACTION
    return max(MAX_FLIP_FRACTION, small_sample_allowance(n_codes) / max(1, n_codes))


# Every sample judged under flip_cap in this session, pooled: one allowed flip per small
# sample must not add up to a rate above the cap over all of them together
# (tests/test_zy_pooled_flips.py checks the pool after the other GPU tests).
POOLED = {"flips": 0, "codes": 0, "samples": 0}


def capped(n_codes: int, flips: int) -> float:
    """flip_cap(n_codes) for a sample with `flips` differing codes, recorded in POOLED."""
    POOLED["flips"] += int(flips)
    POOLED["codes"] += int(n_codes)
    POOLED["samples"] += 1
    return flip_cap(n_codes)
NORM_REL_TOL = 1e-6
# Decode: on unit vectors (norms = NULL) the device and oracle reconstructions differ by
# float32 butterfly rounding plus at most one float16 ulp (2^-11 for |x| < 1).
DECODE_UNIT_ATOL = 1e-3

_TABLES: dict = {}


def _finite16(v: np.ndarray) -> np.ndarray:
    """float16 values as float64 with +-inf replaced by +-65536, the power of two where
    round-to-nearest-even overflows: a reconstruction that lands just past the float16 range
    on one side and just inside it on the other then differs by one float16 step (32), as
    it should, instead of producing inf - inf."""
    v = v.astype(np.float64)
    return np.where(np.isinf(v), np.sign(v) * 65536.0, v)


def tables(d, bits):
    if (d, bits) not in _TABLES:
        _TABLES[(d, bits)] = ocb.build_tables(d, bits)
    return _TABLES[(d, bits)]


def as_u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def gpu_encode(x: torch.Tensor, signs, bits, S_cap=None, s_offset=0, fill=None):
    """Encode fp16 [B, H, S, D] (cuda) into freshly allocated caches; returns cuda tensors."""
    B, H, S, D = x.shape
    S_cap = S if S_cap is None else S_cap
    cb = kvq.build_codebooks(D, bits, signs)
    p1 = torch.empty((B, H, S_cap, cb.n_words), dtype=torch.int32, device=x.device)
    p2 = torch.empty_like(p1)
    nrm = torch.empty((B, H, S_cap), dtype=torch.float32, device=x.device)
    if fill is not None:
        p1.fill_(fill), p2.fill_(fill), nrm.fill_(float("nan"))
    kvq.kvq_rvq_encode_pack(cb, x, p1, p2, nrm, s_offset)
    torch.cuda.synchronize()
    return p1, p2, nrm


def judge(x16_rows: np.ndarray, signs, bits, p1_rows: np.ndarray, p2_rows: np.ndarray, norm_rows: np.ndarray):
    d = x16_rows.shape[1]
    t = tables(d, bits)
    ref = rvq.encode(x16_rows, np.asarray(signs, np.int8), t)
    return flips.compare_encode(p1_rows, p2_rows, norm_rows, ref, t, REL_WINDOW), ref


def judge_all(x_rows: torch.Tensor, signs, bits, p1_rows: torch.Tensor, p2_rows: torch.Tensor,
              norm_rows: torch.Tensor, chunk: int = 1 << 18):
    """Every row of a large launch judged against the oracle, chunk by chunk (the oracle's
    memory stays bounded); the chunks' counts add up to one report over all rows."""
    d = x_rows.shape[1]
    t = tables(d, bits)
    s8 = np.asarray(signs, np.int8)
    total = flips.Report(n_vectors=0, n_codes=0)
    for r0 in range(0, x_rows.shape[0], chunk):
        r1 = min(x_rows.shape[0], r0 + chunk)
        ref = rvq.encode(x_rows[r0:r1].cpu().numpy(), s8, t)
        rep = flips.compare_encode(as_u32(p1_rows[r0:r1]), as_u32(p2_rows[r0:r1]), norm_rows[r0:r1].cpu().numpy(),
                                   ref, t, REL_WINDOW)
        total.n_vectors += rep.n_vectors
        total.n_codes += rep.n_codes
        total.stage1_diff += rep.stage1_diff
        total.stage2_diff += rep.stage2_diff
        total.bad_stage1 += rep.bad_stage1
        total.bad_stage2 += rep.bad_stage2
        total.padding_bad += rep.padding_bad
        total.norm_max_rel = max(total.norm_max_rel, rep.norm_max_rel)
        total.examples += [(r0 + e[1],) + tuple(e) for e in rep.examples[:2]]
    return total


def check_encode(x: torch.Tensor, signs, bits, max_flip=None):
    """Encode x on the GPU and require the oracle's codes and norms under the rule.
    max_flip=None applies flip_cap(); degenerate inputs pass 0.0 (no flips at all)."""
    B, H, S, D = x.shape
    p1, p2, nrm = gpu_encode(x, signs, bits)
    x_rows = x.detach().cpu().numpy().reshape(-1, D)
    rep, ref = judge(x_rows, signs, bits, as_u32(p1).reshape(-1, p1.shape[-1]),
                     as_u32(p2).reshape(-1, p2.shape[-1]), nrm.cpu().numpy().reshape(-1))
    cap = capped(rep.n_codes, rep.flips) if max_flip is None else max_flip
    assert rep.ok(cap, NORM_REL_TOL), rep.summary()
    return rep, (p1, p2, nrm), ref


def check_decode_from_oracle_words(ref: dict, signs, bits, shape, with_norms=True):
    """Feed the oracle's packed words to the GPU decoder and to the oracle decoder."""
    B, H, S, D = shape
    t = tables(D, bits)
    cb = kvq.build_codebooks(D, bits, signs)
    dev = torch.device("cuda")
    p1 = torch.from_numpy(ref["packed1"].view(np.int32)).reshape(B, H, S, -1).to(dev)
    p2 = torch.from_numpy(ref["packed2"].view(np.int32)).reshape(B, H, S, -1).to(dev)
    out = torch.empty((B, H, S, D), dtype=torch.float16, device=dev)
    kvq.kvq_rvq_unpack_decode(cb, p1, p2, None, out)
    torch.cuda.synchronize()
    got = _finite16(out.cpu().numpy().reshape(-1, D))
    want = _finite16(rvq.decode(ref["packed1"], ref["packed2"], None, np.asarray(signs), t))
    err_unit = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert err_unit <= DECODE_UNIT_ATOL, err_unit
    err_rel = 0.0
    if with_norms:
        nrm = torch.from_numpy(ref["norms"]).reshape(B, H, S).to(dev)
        kvq.kvq_rvq_unpack_decode(cb, p1, p2, nrm, out)
        torch.cuda.synchronize()
        got = _finite16(out.cpu().numpy().reshape(-1, D))
        want = _finite16(rvq.decode(ref["packed1"], ref["packed2"], ref["norms"], np.asarray(signs), t))
        # relative to the vector's norm (the unit bound scales with it), plus the absolute
        # spacing of float16 subnormals (2^-24) for vectors with tiny norms
        n = ref["norms"].astype(np.float64)[:, None]
        excess = np.abs(got - want) - (DECODE_UNIT_ATOL * n + 2.0 ** -24)
        err_rel = float(np.max(np.abs(got - want) / np.maximum(n, 1e-30))) if got.size else 0.0
        assert not got.size or float(np.max(excess)) <= 0.0, err_rel
    return err_unit, err_rel


# ----------------------------------------------------------------- single-stage codec

def check_encode_mse(x: torch.Tensor, signs, bits, max_flip=None, S_cap=None, s_offset=0):
    """Single-stage encode on the GPU against the oracle's encode_mse under the same rule."""
    B, H, S, D = x.shape
    S_cap = S if S_cap is None else S_cap
    cb = kvq.build_codebooks(D, bits, signs)
    p = torch.full((B, H, S_cap, cb.n_words), -1, dtype=torch.int32, device=x.device)
    nrm = torch.full((B, H, S_cap), float("nan"), dtype=torch.float32, device=x.device)
    kvq.kvq_mse_encode_pack(cb, x, p, nrm, s_offset)
    torch.cuda.synchronize()
    t = tables(D, bits)
    ref = rvq.encode_mse(x.detach().cpu().numpy().reshape(-1, D), np.asarray(signs, np.int8), t)
    win_p = as_u32(p[:, :, s_offset:s_offset + S]).reshape(-1, cb.n_words)
    win_n = nrm[:, :, s_offset:s_offset + S].cpu().numpy().reshape(-1)
    rep = flips.compare_encode_single(win_p, win_n, ref, t, REL_WINDOW)
    cap = capped(rep.n_codes, rep.flips) if max_flip is None else max_flip
    assert rep.ok(cap, NORM_REL_TOL), rep.summary()
    return rep, (p, nrm), ref


def check_decode_mse_from_oracle_words(ref: dict, signs, bits, shape):
    """Feed the oracle's single-stage words to the GPU decoder and to the oracle decoder."""
    B, H, S, D = shape
    t = tables(D, bits)
    cb = kvq.build_codebooks(D, bits, signs)
    dev = torch.device("cuda")
    p = torch.from_numpy(ref["packed"].view(np.int32)).reshape(B, H, S, -1).to(dev)
    out = torch.empty((B, H, S, D), dtype=torch.float16, device=dev)
    kvq.kvq_mse_unpack_decode(cb, p, None, out)
    torch.cuda.synchronize()
    got = _finite16(out.cpu().numpy().reshape(-1, D))
    want = _finite16(rvq.decode_mse(ref["packed"], None, np.asarray(signs), t))
    err_unit = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert err_unit <= DECODE_UNIT_ATOL, err_unit
    nrm = torch.from_numpy(ref["norms"]).reshape(B, H, S).to(dev)
    kvq.kvq_mse_unpack_decode(cb, p, nrm, out)
    torch.cuda.synchronize()
    got = _finite16(out.cpu().numpy().reshape(-1, D))
    want = _finite16(rvq.decode_mse(ref["packed"], ref["norms"], np.asarray(signs), t))
    n = ref["norms"].astype(np.float64)[:, None]
    assert not got.size or float(np.max(np.abs(got - want) - (DECODE_UNIT_ATOL * n + 2.0 ** -24))) <= 0.0
    return err_unit
