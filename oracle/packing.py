"""LSB-first packing of b-bit codes into uint32 words (oracle side; test infrastructure).

Follows the VeloxQuant-MLX blog, "rvq" tag page, section "The kernel": a word holds
floor(32 / b) consecutive codes of one vector, code j of the word occupying bits
[j*b, j*b + b); codes past the end of the vector contribute nothing, so a partial last
word has zero padding. Each vector owns ceil(D / floor(32 / b)) words per stream
("The pipeline, as it actually runs" reshapes each stream to (B, H, S, n_words)).
"""
from __future__ import annotations

import numpy as np


def elems_per_word(bits: int) -> int:
    return 32 // bits


def n_words(d: int, bits: int) -> int:
    epw = elems_per_word(bits)
    return (d + epw - 1) // epw


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes: integer array [..., D] with values < 2**bits -> uint32 [..., n_words]."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    epw = elems_per_word(bits)
    nw = n_words(d, bits)
    mask = (1 << bits) - 1
    out = np.zeros(codes.shape[:-1] + (nw,), dtype=np.uint64)
    for j in range(d):
        w, k = divmod(j, epw)
        out[..., w] |= (codes[..., j].astype(np.uint64) & mask) << np.uint64(k * bits)
    return out.astype(np.uint32)


def unpack(words: np.ndarray, bits: int, d: int) -> np.ndarray:
    """uint32 [..., n_words] -> uint8 codes [..., d] (inverse of pack)."""
    words = np.asarray(words, dtype=np.uint32)
    epw = elems_per_word(bits)
    mask = (1 << bits) - 1
    out = np.zeros(words.shape[:-1] + (d,), dtype=np.uint8)
    for j in range(d):
        w, k = divmod(j, epw)
        out[..., j] = (words[..., w] >> np.uint32(k * bits)) & mask
    return out


def padding_mask(d: int, bits: int) -> np.ndarray:
    """uint32 [n_words]: the bits of each word that hold no code (must be zero)."""
    nw = n_words(d, bits)
    used = np.zeros(nw, dtype=np.uint64)
    epw = elems_per_word(bits)
    for j in range(d):
        w, k = divmod(j, epw)
        used[w] |= np.uint64(((1 << bits) - 1) << (k * bits))
    return (~used & np.uint64(0xFFFFFFFF)).astype(np.uint32)
