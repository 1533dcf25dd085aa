"""Seeded, counter-addressable synthetic inputs for the two-stage RVQ KV-cache codec.

This module is shared by the tests, the bench and the checker side. It holds none of
the codec's arithmetic: it only turns (seed, stream, element index) into bits, and bits
into fp16 key/value tensors and +-1 sign vectors of the shapes and distributions the
workloads use. Because every element is a pure function of its index, any row range of
a tensor can be regenerated on its own (the checker regenerates sampled rows of large
tensors without producing the rest), on the CPU or on a GPU.

Generator definition (all arithmetic modulo 2**64):
  * mix64 is the output function of SplitMix64 (Steele, Lea & Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014):
        z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
        z ^= z >> 31
  * key(seed, stream) = mix64(seed * G + stream), G = 0x9E3779B97F4A7C15
  * bits(seed, stream, i) = mix64(key + (i + 1) * G)
  * uniform(i) = ((bits >> 11) + 0.5) * 2**-53, strictly inside (0, 1)
  * standard normal: Box-Muller on the uniform pair (2p, 2p+1) of p = i // 2, cosine
    branch for even i and sine branch for odd i, in float64
  * Laplace(0, 1): inverse CDF of one uniform, in float64
  * every value is rounded float64 -> float32 -> float16, round-to-nearest-even each
    step, so the bytes are the same on every device.

torch int64 tensors carry the uint64 state: multiplication wraps, and a logical right
shift is an arithmetic shift followed by a mask.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import torch

_M64 = (1 << 64) - 1


def _s64(v: int) -> int:
    """Reinterpret an unsigned 64-bit constant as the int64 with the same bits."""
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


_G = _s64(0x9E3779B97F4A7C15)
_C1 = _s64(0xBF58476D1CE4E5B9)
_C2 = _s64(0x94D049BB133111EB)

STREAM_DATA = 0
STREAM_SCALE = 1
STREAM_SIGNS = 2


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    return (z >> k) & ((1 << (64 - k)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _C1
    z = (z ^ _lsr(z, 27)) * _C2
    return z ^ _lsr(z, 31)


def _key(seed: int, stream: int) -> int:
    z = ((seed * 0x9E3779B97F4A7C15) + stream) & _M64
    # scalar SplitMix64 output function on Python ints
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & _M64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & _M64
    z ^= z >> 31
    return _s64(z)


def bits(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """64 random bits (as int64) for each element index in ``idx`` (int64 tensor)."""
    return mix64(_key(seed, stream) + (idx + 1) * _G)


def uniform(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """float64 uniforms strictly inside (0, 1)."""
    return (_lsr(bits(seed, stream, idx), 11).to(torch.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """Standard normal float64 values, one per element index (Box-Muller)."""
    pair = idx // 2
    u1 = uniform(seed, stream, 2 * pair)
    u2 = uniform(seed, stream, 2 * pair + 1)
    r = torch.sqrt(-2.0 * torch.log(u1))
    theta = (2.0 * math.pi) * u2
    return torch.where((idx & 1) == 0, r * torch.cos(theta), r * torch.sin(theta))


def laplace(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """Laplace(0, 1) float64 values (density exp(-|x|)/2), inverse CDF."""
    u = uniform(seed, stream, idx) - 0.5
    return -torch.sign(u) * torch.log1p(-2.0 * torch.abs(u))


def to_fp16(v: torch.Tensor) -> torch.Tensor:
    return v.to(torch.float32).to(torch.float16)


# --------------------------------------------------------------------------------------
# Workload presets
# --------------------------------------------------------------------------------------

KINDS = ("gauss", "gauss_outliers", "gauss_laplace_heads", "gauss_token_scale")
OUTLIER_CHANNELS = (3, 37, 71, 101)
OUTLIER_GAIN = 20.0
TOKEN_SCALE_LO, TOKEN_SCALE_HI = 0.1, 10.0


@dataclass(frozen=True)
class TensorSpec:
    """One [B, H, S, D] fp16 tensor of synthetic keys or values.

    kind:
      gauss               i.i.d. N(0, 1)
      gauss_outliers      N(0, 1) with channels 3, 37, 71, 101 multiplied by 20 before
                          rounding (a few key channels with huge magnitudes)
      gauss_laplace_heads heads h < H/2 are N(0, 1), the rest Laplace(0, 1)
      gauss_token_scale   N(0, 1) times one log-uniform scale in [0.1, 10] per (b, s)
                          token position, shared by all heads
    """

    B: int
    H: int
    S: int
    D: int
    kind: str
    seed: int

    @property
    def rows(self) -> int:
        return self.B * self.H * self.S

    def __post_init__(self):
        if self.kind not in KINDS:
            raise ValueError(f"unknown kind {self.kind!r}")


def rows(spec: TensorSpec, row_start: int = 0, row_count: Optional[int] = None,
         device: str | torch.device = "cpu") -> torch.Tensor:
    """Rows [row_start, row_start + row_count) of the flattened (B*H*S, D) tensor, fp16."""
    if row_count is None:
        row_count = spec.rows - row_start
    if row_start < 0 or row_count < 0 or row_start + row_count > spec.rows:
        raise ValueError("row range outside the tensor")
    r = torch.arange(row_start, row_start + row_count, dtype=torch.int64, device=device)
    return rows_at(spec, r)


def rows_at(spec: TensorSpec, r: torch.Tensor) -> torch.Tensor:
    """The rows whose flattened indices are in the int64 tensor ``r`` (any order), fp16."""
    device = r.device
    if r.numel() and (int(r.min()) < 0 or int(r.max()) >= spec.rows):
        raise ValueError("row index outside the tensor")
    D = spec.D
    d = torch.arange(D, dtype=torch.int64, device=device)
    idx = r[:, None] * D + d[None, :]
    if spec.kind == "gauss":
        v = normal(spec.seed, STREAM_DATA, idx)
    elif spec.kind == "gauss_outliers":
        v = normal(spec.seed, STREAM_DATA, idx)
        gain = torch.ones(D, dtype=torch.float64, device=device)
        for c in OUTLIER_CHANNELS:
            if c < D:
                gain[c] = OUTLIER_GAIN
        v = v * gain[None, :]
    elif spec.kind == "gauss_laplace_heads":
        h = (r // spec.S) % spec.H
        g = normal(spec.seed, STREAM_DATA, idx)
        lap = laplace(spec.seed, STREAM_DATA, idx)
        v = torch.where((h < spec.H // 2)[:, None], g, lap)
    else:  # gauss_token_scale
        s = r % spec.S
        b = r // (spec.H * spec.S)
        tok = b * spec.S + s
        u = uniform(spec.seed, STREAM_SCALE, tok)
        lo, hi = math.log(TOKEN_SCALE_LO), math.log(TOKEN_SCALE_HI)
        scale = torch.exp(lo + u * (hi - lo))
        v = normal(spec.seed, STREAM_DATA, idx) * scale[:, None]
    return to_fp16(v)


def tensor(spec: TensorSpec, device: str | torch.device = "cpu",
           chunk_rows: int = 1 << 18) -> torch.Tensor:
    """The whole tensor as fp16 [B, H, S, D], generated in row chunks."""
    out = torch.empty((spec.rows, spec.D), dtype=torch.float16, device=device)
    for r0 in range(0, spec.rows, chunk_rows):
        n = min(chunk_rows, spec.rows - r0)
        out[r0:r0 + n] = rows(spec, r0, n, device=device)
    return out.view(spec.B, spec.H, spec.S, spec.D)


def signs(seed: int, D: int) -> torch.Tensor:
    """A +-1 int8 sign vector of length D (bit 0 of the counter hash picks the sign)."""
    b = bits(seed, STREAM_SIGNS, torch.arange(D, dtype=torch.int64))
    return torch.where((b & 1) == 1, -1, 1).to(torch.int8)


# The five workloads: (name, tensor specs, bits per stage list, sign seed or None for all +1).
@dataclass(frozen=True)
class Workload:
    name: str
    tensors: tuple
    bits: tuple
    sign_seed: Optional[int]
    note: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", (TensorSpec(1, 2, 64, 128, "gauss", 1),), (2,), None,
                     "keys [1,2,64,128] N(0,1); b=2; signs all +1"),
    "llama_layer": Workload("llama_layer", (TensorSpec(1, 32, 8192, 128, "gauss_outliers", 2),),
                            (2,), 102, "one layer's keys [1,32,8192,128], outlier channels; b=2"),
    "gqa_long": Workload("gqa_long", (TensorSpec(1, 8, 32768, 128, "gauss_laplace_heads", 3),),
                         (1, 4), 103, "GQA keys [1,8,32768,128], half Gaussian half Laplace heads; b in {1,4}"),
    "prefill_kv": Workload("prefill_kv", (TensorSpec(16, 32, 4096, 128, "gauss_token_scale", 4),
                                          TensorSpec(16, 32, 4096, 128, "gauss_token_scale", 5)),
                           (4,), 104, "prefill flush: keys and values [16,32,4096,128], per-token scales; b=4"),
    "decode_append": Workload("decode_append", (TensorSpec(256, 8, 2000, 128, "gauss", 6),), (2,), 106,
                              "2000 decode steps of [256,8,1,128] appended into S_cap=32768 caches; b=2"),
    # other head dimensions at the Llama layer's byte size (67 MB of fp16 keys)
    "head_dim_64": Workload("head_dim_64", (TensorSpec(1, 32, 16384, 64, "gauss", 8),), (2,), 108,
                            "keys [1,32,16384,64] N(0,1); b=2"),
    "head_dim_256": Workload("head_dim_256", (TensorSpec(1, 32, 4096, 256, "gauss", 9),), (2,), 109,
                             "keys [1,32,4096,256] N(0,1); b=2"),
    "head_dim_512": Workload("head_dim_512", (TensorSpec(1, 32, 2048, 512, "gauss", 10),), (2,), 110,
                             "keys [1,32,2048,512] N(0,1); b=2"),
    "head_dim_1024": Workload("head_dim_1024", (TensorSpec(1, 32, 1024, 1024, "gauss", 11),), (2,), 111,
                              "keys [1,32,1024,1024] N(0,1); b=2"),
}

DECODE_APPEND_S_CAP = 32768


def step_rows(spec: TensorSpec, step: int, device="cpu") -> torch.Tensor:
    """The [B, H, 1, D] slice for one decode step of a decode-append workload.

    The workload's S axis indexes steps, so step t is the token at s = t of every (b, h).
    """
    B, H, S, D = spec.B, spec.H, spec.S, spec.D
    bh = torch.arange(B * H, dtype=torch.int64, device=device)
    return rows_at(spec, bh * S + step).view(B, H, 1, D)
