"""Two-stage residual-VQ encode and decode, written as plainly as possible (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Per head vector x (fp16, length D), following the VeloxQuant-MLX blog. A head dimension D
that is not a power of two (any D in [8, 1024]) is taken as the vector zero-padded to
P = the next power of two: the norm is unchanged, the rotation below is of length P (the
padded coordinates' signs are +1; they multiply zeros), all P rotated coordinates are
quantized and packed, and the decode reconstructs P coordinates and returns the first D.
(The pages' fused kernel takes only powers of two and leaves other shapes to a fallback:
"rvq" tag page, "Wired in as a fallback, not a replacement"; zero-padding is this codec's
reading of how such shapes are stored.) For a power of two, P = D and nothing changes.
  1. n = ||x||, u = x / n (u = 0 when n = 0).  ["rvq" tag page, "The pipeline, as it
     actually runs": the cache encodes the unit vector and keeps its norm; the norm is
     stored as float32.]
  2. y = H diag(s) u / sqrt(D), with H the D x D Sylvester-ordered Hadamard matrix,
     H[i, j] = (-1)**popcount(i & j), and s the +-1 sign vector.  ["turboquant" tag page,
     "Kernel 3": the sign flip multiplies each coordinate before the in-place butterfly,
     then the result is scaled by 1/sqrt(D).]  Computed in float64 and rounded once to
     float32: the value every quantization decision is taken on is a float32, as in the
     pages' kernels, which read the rotated coordinate as a float.
  3. i1 = index of the nearest stage-1 centroid to y, first minimum on ties.
     ["turboquant" tag page, "Kernel 2"; "rvq" tag page, "What 'quantize' means here,
     precisely": counting boundary crossings reaches the same index.]
  4. r = y - c1[i1], one float32 subtraction.  ["rvq" tag page, "The kernel".]
  5. i2 = index of the nearest stage-2 centroid to r.
  6. each code stream packed LSB-first into uint32 words (packing.py).
Single-stage variant (encode_mse / decode_mse): steps 1-3 and 6 for one stream; decode
z = c1[i1].
Decode ("turboquant" tag page, "Kernel 5": the dequantized coordinate is
c1[i1] + c2[i2], in the rotated domain):
  z = c1[i1] + c2[i2] (float32 add);  u_hat = diag(s) H z / sqrt(D)  (the inverse of step 2,
  since H is symmetric and H H = D I);  x_hat = RN16(n * u_hat), or RN16(u_hat) for unit
  reconstructions. Products and sums of the inverse rotation are float64, rounded once.
"""
from __future__ import annotations

import math

import numpy as np

from . import packing
from .codebooks import Tables

CHUNK = 8192  # vectors per block of work; blocking changes no arithmetic


def hadamard(d: int) -> np.ndarray:
    """Explicit D x D Sylvester Hadamard matrix, entries +-1 as float64."""
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


_H_CACHE: dict[int, np.ndarray] = {}


def _H(d: int) -> np.ndarray:
    if d not in _H_CACHE:
        _H_CACHE[d] = hadamard(d)
    return _H_CACHE[d]


def pad_to(x: np.ndarray, p: int, fill) -> np.ndarray:
    """The last axis of x extended to length p with `fill`."""
    d = x.shape[-1]
    if d == p:
        return x
    out = np.full(x.shape[:-1] + (p,), fill, dtype=x.dtype)
    out[..., :d] = x
    return out


def norms_and_rotation(x16: np.ndarray, signs: np.ndarray, p: int = 0):
    """x16: float16 [N, D]; signs: +-1 [D]; p: rotation length (0: D).  Returns
    (norm float64 [N], y float32 [N, P]): x and the signs are zero- and one-padded to P.

    The rotation is linear, so y = H diag(s) (x / n) / sqrt(D) = (H diag(s) x) / (n sqrt(D)).
    The oracle forms H diag(s) x on the float16 values themselves: every float16 is an
    integer multiple of 2**-24 below 2**16 in magnitude, so a signed sum of at most 1024 of
    them is an integer multiple of 2**-24 below 2**26, exactly representable in float64.
    That product is therefore exact (exact cancellations give exactly 0), and the only
    roundings are the norm, the one division and the final rounding to float32.
    """
    p = p or x16.shape[1]
    x = pad_to(np.asarray(x16, dtype=np.float16).astype(np.float64), p, 0.0)
    n, d = x.shape
    if d > 1024:
        raise ValueError("exactness argument holds for D <= 1024")
    s = pad_to(np.asarray(signs, dtype=np.float64), p, 1.0)
    H = _H(d)
    norm = np.sqrt(np.sum(x * x, axis=1))
    y = np.empty((n, d), dtype=np.float32)
    for a in range(0, n, CHUNK):
        xb, nb = x[a:a + CHUNK], norm[a:a + CHUNK]
        w = (xb * s[None, :]) @ H.T
        den = np.where(nb > 0.0, nb * math.sqrt(d), 1.0)
        y[a:a + CHUNK] = np.where((nb > 0.0)[:, None], w / den[:, None], 0.0).astype(np.float32)
    return norm, y


def nearest(v32: np.ndarray, c32: np.ndarray) -> np.ndarray:
    """Index of the nearest centroid (ascending c32) to each float32 value, exactly.

    The first minimum wins a true tie. Distances are taken in float64; rounding is
    monotone, so float64 distances never reverse the order of two exact distances but
    can tie two that differ by less than an ulp (a value a few float32 ulps from the
    middle boundary 0 is the extreme case). Such a tie between neighbours k and k+1 is
    settled by comparing v with their exact midpoint (exact in float64 for two float32
    values), which is the comparison an exact argmin makes.
    """
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    c = np.asarray(c32, dtype=np.float32).astype(np.float64)
    dist = np.abs(v[..., None] - c)
    k = np.argmin(dist, axis=-1)
    kk = np.minimum(k + 1, len(c) - 1)
    dk = np.take_along_axis(dist, k[..., None], axis=-1)[..., 0]
    dn = np.take_along_axis(dist, kk[..., None], axis=-1)[..., 0]
    tie = (kk > k) & (dn == dk)
    mid = 0.5 * (c[k] + c[kk])
    k = np.where(tie & (v > mid), kk, k)
    return k.astype(np.uint8)


def quantize_two_stage(y32: np.ndarray, t: Tables):
    """(i1, r, i2) for float32 rotated coordinates y32."""
    i1 = nearest(y32, t.c1)
    r = (y32.astype(np.float32) - t.c1[i1]).astype(np.float32)
    i2 = nearest(r, t.c2)
    return i1, r, i2


def encode(x16: np.ndarray, signs: np.ndarray, t: Tables) -> dict:
    """Encode float16 [N, D] vectors.  Returns packed streams, norms and intermediates."""
    x16 = np.asarray(x16, dtype=np.float16)
    if x16.ndim != 2 or x16.shape[1] != t.d:
        raise ValueError("x16 must be [N, D] with D matching the tables")
    norm, y = norms_and_rotation(x16, signs, t.p)
    i1 = np.empty(y.shape, dtype=np.uint8)
    i2 = np.empty(y.shape, dtype=np.uint8)
    r = np.empty(y.shape, dtype=np.float32)
    for a in range(0, y.shape[0], CHUNK):
        i1[a:a + CHUNK], r[a:a + CHUNK], i2[a:a + CHUNK] = quantize_two_stage(y[a:a + CHUNK], t)
    return {
        "packed1": packing.pack(i1, t.bits),
        "packed2": packing.pack(i2, t.bits),
        "norms": norm.astype(np.float32),
        "norm64": norm,
        "y": y,
        "r": r,
        "i1": i1,
        "i2": i2,
    }


def _unrotate(z: np.ndarray, norms, signs: np.ndarray, d: int) -> np.ndarray:
    """x_hat = RN16(n * diag(s) H z / sqrt(P)) (RN16(diag(s) H z / sqrt(P)) for norms=None),
    products and sums in float64, rounded once: z has P columns, x_hat the first d of the
    P reconstructed coordinates."""
    p = z.shape[1]
    H = _H(p)
    w = (z.astype(np.float64) @ H.T)[:, :d] / math.sqrt(p)
    s = np.asarray(signs, dtype=np.float64)
    u_hat = w * s[None, :]
    if norms is not None:
        u_hat = u_hat * np.asarray(norms, dtype=np.float32).astype(np.float64)[:, None]
    return u_hat.astype(np.float16)


def decode(packed1: np.ndarray, packed2: np.ndarray, norms, signs: np.ndarray, t: Tables) -> np.ndarray:
    """Decode [N, n_words] streams to float16 [N, D]; norms=None gives unit reconstructions."""
    i1 = packing.unpack(packed1, t.bits, t.p)
    i2 = packing.unpack(packed2, t.bits, t.p)
    z = (t.c1[i1] + t.c2[i2]).astype(np.float32)
    return _unrotate(z, norms, signs, t.d)


def encode_mse(x16: np.ndarray, signs: np.ndarray, t: Tables) -> dict:
    """Single-stage encode: normalize, rotate, nearest stage-1 (Gaussian Lloyd-Max)
    centroid, pack one stream.  ["turboquant" tag page, "Kernel 3": the rotation followed
    by the nearest-centroid quantize; the cache keeps the unit vector's codes and its norm
    as in the two-stage codec.]  Returns the packed stream, norms and intermediates."""
    x16 = np.asarray(x16, dtype=np.float16)
    if x16.ndim != 2 or x16.shape[1] != t.d:
        raise ValueError("x16 must be [N, D] with D matching the tables")
    norm, y = norms_and_rotation(x16, signs, t.p)
    i1 = np.empty(y.shape, dtype=np.uint8)
    for a in range(0, y.shape[0], CHUNK):
        i1[a:a + CHUNK] = nearest(y[a:a + CHUNK], t.c1)
    return {"packed": packing.pack(i1, t.bits), "norms": norm.astype(np.float32), "norm64": norm, "y": y, "i1": i1}


def decode_mse(packed: np.ndarray, norms, signs: np.ndarray, t: Tables) -> np.ndarray:
    """Single-stage decode: z = c1[i] ("turboquant" tag page, "Kernel 2": dequantize is a
    gather of the centroid), then the inverse rotation and the norm."""
    i1 = packing.unpack(packed, t.bits, t.p)
    return _unrotate(t.c1[i1].astype(np.float32), norms, signs, t.d)
