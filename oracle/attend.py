"""Softmax attention over a packed two-stage cache, written as plainly as possible (oracle
side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The definition followed ("turboquant" tag page, "Kernel 5": attention whose keys are the
dequantized cache entries c1[i1] + c2[i2], taken inside one softmax pass; here the values
come from a packed cache too): for every query vector q of query head h, with key/value
head g = h // (Hq / Hkv),

    khat_t = n_t diag(s_k) H z_t / sqrt(D),   z_t = c1[i1] + c2[i2]  (the key cache)
    vhat_t = the same for the value cache
    p      = softmax_t(scale * q . khat_t),   t in [0, S_kv)
    out    = RN16(sum_t p_t vhat_t)

khat and vhat are the unrounded reconstructions of the two-stage decode (float64; the
z tables are the float32 sums of the decode). Products, sums and the softmax are float64
with the maximum subtracted; the output is rounded to float16 once.
"""
from __future__ import annotations

import math

import numpy as np

from . import packing
from .codebooks import Tables
from .rvq import _H


def reconstruct(packed1: np.ndarray, packed2: np.ndarray, norms: np.ndarray, signs: np.ndarray,
                t: Tables) -> np.ndarray:
    """float64 [N, D] reconstructions n diag(s) H z / sqrt(D) of packed rows [N, n_words]."""
    d = t.d
    i1 = packing.unpack(packed1, t.bits, d)
    i2 = packing.unpack(packed2, t.bits, d)
    z = (t.c1[i1] + t.c2[i2]).astype(np.float32).astype(np.float64)
    w = (z @ _H(d).T) / math.sqrt(d)
    return w * np.asarray(signs, np.float64)[None, :] * np.asarray(norms, np.float64)[:, None]


def attend64(q16: np.ndarray, kcache, vcache, signs_k, signs_v, tk: Tables, tv: Tables, S_kv: int,
             scale: float) -> np.ndarray:
    """float64 attention outputs [B, Hq, Sq, D] before the final rounding.

    q16: float16 [B, Hq, Sq, D]; kcache, vcache: (packed1, packed2, norms) with shapes
    [B, Hkv, S_cap, n_words] and [B, Hkv, S_cap]."""
    B, Hq, Sq, d = q16.shape
    k1, k2, kn = kcache
    v1, v2, vn = vcache
    Hkv = k1.shape[1]
    group = Hq // Hkv
    out = np.zeros((B, Hq, Sq, d), np.float64)
    for b in range(B):
        for g in range(Hkv):
            K = reconstruct(k1[b, g, :S_kv], k2[b, g, :S_kv], kn[b, g, :S_kv], signs_k, tk)
            V = reconstruct(v1[b, g, :S_kv], v2[b, g, :S_kv], vn[b, g, :S_kv], signs_v, tv)
            for h in range(g * group, (g + 1) * group):
                qh = q16[b, h].astype(np.float64)               # [Sq, D]
                s = scale * (qh @ K.T)                           # [Sq, S_kv]
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                out[b, h] = p @ V
    return out


def attend(q16: np.ndarray, kcache, vcache, signs_k, signs_v, tk: Tables, tv: Tables, S_kv: int,
           scale: float) -> np.ndarray:
    """float16 [B, Hq, Sq, D] attention outputs (see the module docstring)."""
    return attend64(q16, kcache, vcache, signs_k, signs_v, tk, tv, S_kv, scale).astype(np.float16)
