"""Philox4x32-10 and the stream layout of the sampler's random numbers (oracle side).

Generator: Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC'11), section 3 / table of Philox parameters: a 4-word
counter, a 2-word key, ten rounds, each round multiplying words 0 and 2 by fixed 32-bit
constants and mixing the high halves with the other words and the round key; the key is
advanced by the two Weyl constants between rounds.

The pages only ask for Gumbel noise (vLLM blog, sampler section) and uniform replacement
tokens (DiffusionGemma Explained, "Sampling": renoise with uniformly drawn tokens;
Technical Report sec. 2.1.1 eq. (1)), so the layout below is this library's own
definition, written separately on the HIP side:

  key                 = (seed & 0xffffffff, seed >> 32)
  Gumbel  (row r, vocab v, step s):   counter (v >> 2, r, s, 0x47554D42), word v & 3
  renoise (row r, step s):            counter (0, r, s, 0x52454E4F),      word 0
  q_sample(row r):                    counter (0, r, 0, 0x51534D50),      words 0 (keep), 1 (token)
  uniform in (0,1):   u = ((x >> 9) + 0.5) * 2**-23
  uniform token:      (x * V) >> 32   (multiply-shift; exact when V is a power of two)
"""
from __future__ import annotations

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)

TAG_GUMBEL = 0x47554D42
TAG_RENOISE = 0x52454E4F
TAG_QSAMPLE = 0x51534D50


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on broadcastable arrays of 32-bit words.  Returns 4 uint32 arrays."""
    c0, c1, c2, c3, k0, k1 = (np.asarray(x, dtype=np.uint64) & MASK32
                              for x in (c0, c1, c2, c3, k0, k1))
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(c0, c1, c2, c3, k0, k1)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + _W0) & MASK32
            k1 = (k1 + _W1) & MASK32
        p0 = _M0 * c0          # full 64-bit product of two 32-bit words
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def key_of(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def uniform01(x) -> np.ndarray:
    """u = ((x >> 9) + 0.5) / 2**23, exactly, in fp64; lies in [2**-24, 1 - 2**-24]."""
    x = np.asarray(x, dtype=np.uint32)
    return ((x >> np.uint32(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def uniform_token(x, V: int) -> np.ndarray:
    """floor(x * V / 2**32) for 32-bit words x."""
    x = np.asarray(x, dtype=np.uint64)
    return ((x * np.uint64(V)) >> np.uint64(32)).astype(np.int64)


def gumbel_words(row: int, V: int, seed: int, step: int) -> np.ndarray:
    """The V raw 32-bit words that drive the Gumbel noise of one row."""
    k0, k1 = key_of(seed)
    n = (V + 3) // 4
    j = np.arange(n, dtype=np.uint64)
    w = philox4x32_10(j, row, step, TAG_GUMBEL, k0, k1)
    return np.stack(w, axis=1).reshape(-1)[:V]


def gumbel_noise(row: int, V: int, seed: int, step: int) -> np.ndarray:
    """Standard Gumbel noise g_v = -ln(-ln u_v) for v = 0..V-1 of one row, fp64."""
    u = uniform01(gumbel_words(row, V, seed, step))
    return -np.log(-np.log(u))


def renoise_tokens(rows: np.ndarray, V: int, seed: int, step) -> np.ndarray:
    """Uniform replacement token of each row (step may be per row)."""
    k0, k1 = key_of(seed)
    w0, _, _, _ = philox4x32_10(0, np.asarray(rows, dtype=np.uint64), step, TAG_RENOISE, k0, k1)
    return uniform_token(w0, V)


def qsample_words(rows: np.ndarray, seed: int):
    k0, k1 = key_of(seed)
    w0, w1, _, _ = philox4x32_10(0, np.asarray(rows, dtype=np.uint64), 0, TAG_QSAMPLE, k0, k1)
    return w0, w1
