"""Oracle for the self-conditioning consumer: the next decode step's input rows built from the
self-conditioning expectation and the renoised tokens.  Test infrastructure only (tests,
the smoke check and the bench's CPU baseline may use it; the product path never does).

Definitions followed (DiffusionGemma Explained, "Self-conditioning" and the model's decode
forward; the conditioning MLP of the "MLP and mixture-of-experts block" section, a gated
GELU MLP as in the "Mixture of Experts" section; RMSNorm as in the "RMSNorm" section;
Technical Report sec. 3.2 eq. (6), z = FFW(p_hat_0 E)):

  s      = sqrt(D)                                   (the embedding scale)
  cx     = sc * s                                    (sc = sum_v p_v E_v, [R, D])
  rms_w(x) = w * x * sqrt(D) / (||x||_2 + eps)       (norm over the row, eps added to the norm)
  x1     = rms_w(cx)              with w = the MLP's pre-norm weight
  y      = (x1 W_up^T) * GELU(x1 W_gate^T)           (GELU with the error function)
  res    = y W_down^T
  out    = rms_1(E[tok] * s + res)                   (no weight)

Precision: fp64 arithmetic, rounded to bf16 (round to nearest even) where the pages' code
holds the tensors that feed a matrix product, and at the output: x1, y and out.  cx and
res stay unrounded (plain reading: a fused implementation need not materialise them).

The first decode step has no previous prediction: sc = None gives res = 0, so
out = rms_1(E[tok] s) (the MLP maps zero to zero).
Rows of commit canvases are not computed (NaN), nor are rows whose token lies outside
[0, V) (the pages never index the embedding out of range; such a row is NaN).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (ties to even), returned as fp64; finite inputs.

    A bf16 number has 8 significant bits and the exponent range of fp32: below 2^-126 its
    quantum is 2^-133.  Rounding the significand scaled to 8 integer bits with rint (ties to
    even, exact in fp64) gives the nearest representable value."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # subnormal range: fixed quantum 2^-133
    q = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    return np.where(x == 0, x, q)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def gelu(x: np.ndarray) -> np.ndarray:
    """x Phi(x) with Phi the standard normal CDF, 0.5 (1 + erf(x / sqrt 2))."""
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * x * (1.0 + erf(np.asarray(x, np.float64) / math.sqrt(2.0)))


def rms(x: np.ndarray, w: Optional[np.ndarray], eps: float) -> np.ndarray:
    D = x.shape[-1]
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    y = x * math.sqrt(D) / (n + eps)
    return y if w is None else w * y


def selfcond_input(sc: Optional[np.ndarray], tokens: np.ndarray, E_bits: np.ndarray,
                   pre_norm_bits: np.ndarray, W_gate_bits: np.ndarray, W_up_bits: np.ndarray,
                   W_down_bits: np.ndarray, commit_row: Optional[np.ndarray] = None,
                   eps: float = 1e-6, rows=None) -> np.ndarray:
    """Next-step input rows (fp64 values of bf16 numbers, [n_rows, D]).

    sc        fp32/fp64 [R, D] expectation rows, or None for the first decode step
    tokens    int [R] renoised tokens of the canvas
    E_bits    bf16 bits [V, D]; pre_norm_bits bf16 [D]; W_gate/W_up bf16 [F, D];
              W_down bf16 [D, F]
    rows      the rows to compute (default all)."""
    R = tokens.shape[0]
    rows = np.arange(R) if rows is None else np.asarray(rows)
    V, D = E_bits.shape
    s = math.sqrt(D)
    cm = np.zeros(R, bool) if commit_row is None else np.asarray(commit_row, bool)
    out = np.full((rows.size, D), np.nan)
    tok_ok = (tokens >= 0) & (tokens < V)
    keep = ~cm[rows] & tok_ok[rows]
    rk = rows[keep]
    if rk.size == 0:
        return out
    emb = widen_bf16(E_bits[tokens[rk]]) * s
    if sc is None:
        res = np.zeros_like(emb)
    else:
        cx = np.asarray(sc, np.float64)[rk] * s
        x1 = round_bf16(rms(cx, widen_bf16(pre_norm_bits), eps))
        a = x1 @ widen_bf16(W_up_bits).T
        g = x1 @ widen_bf16(W_gate_bits).T
        y = round_bf16(a * gelu(g))
        res = y @ widen_bf16(W_down_bits).T
    out[keep] = round_bf16(rms(emb + res, None, eps))
    return out
