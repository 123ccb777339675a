"""Oracle for q_sample, the closed-form forward corruption.

Definition (Technical Report part 2/6, sec. 2.1.1 eq. (1)): given the clean canvas x0 and
the keep probability kappa_t, each position independently keeps its clean token with
probability kappa_t and otherwise takes a token drawn uniformly from the vocabulary, so
P(x_t = x0) = kappa_t + (1 - kappa_t) / V.  DiffusionGemma-Lite ("Forward process") draws it
in one shot, never by iterating the chain.  (That page's per-row table, clean token
weighted by alpha and every other by (1 - alpha)/V, does not sum to one; eq. (1) is used.)

Keep test on 24 bits: keep iff (w0 >> 8) < floor(kappa * 2**24), with kappa the fp32 value
the caller passed; the replacement token is the multiply-shift uniform token of w1.
"""
from __future__ import annotations

import math

import numpy as np

from . import philox


def keep_threshold(kappa_f32: float) -> int:
    return int(math.floor(float(np.float32(kappa_f32)) * 16777216.0))


def q_sample(x0: np.ndarray, n_canvas: int, C: int, V: int, kappa: np.ndarray,
             seed: int) -> np.ndarray:
    x0 = np.asarray(x0, dtype=np.int64)
    rows = np.arange(n_canvas * C, dtype=np.uint64)
    w0, w1 = philox.qsample_words(rows, seed)
    thr = np.array([keep_threshold(k) for k in np.asarray(kappa, dtype=np.float32)],
                   dtype=np.int64)
    thr_row = np.repeat(thr, C)
    keep = (w0.astype(np.int64) >> 8) < thr_row
    return np.where(keep, x0, philox.uniform_token(w1, V))
