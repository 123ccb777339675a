"""Oracle for the FP8 embedding: E4M3 codes with one power-of-two scale per row.  Test
infrastructure only.

The vLLM page ships DiffusionGemma as an FP8 checkpoint with quantised weights and dynamic
activations (vLLM blog, quantised checkpoints); the pages print no scale scheme.  Reading
used here: the tied embedding is stored as OCP FP8 E4M3 (sign, 4 exponent bits with bias 7,
3 mantissa bits, no infinities, 0x7F / 0xFF NaN, largest finite 448) with one scale 2^k per
row, the row's largest |E| mapped to at most 448:

  k_v = the smallest integer with max_j |E_vj| <= 448 * 2^k_v, at least -117
        (a zero row gets -117; the floor keeps every nonzero dequantised value a normal
        fp32 / bf16 number, at least 2^-9 * 2^-117 = 2^-126)
  q_vj = E4M3 nearest to E_vj / 2^k_v (ties to the even code)
  E~_vj = 2^k_v * value(q_vj)

A power-of-two scale keeps E~ exact in bf16 (E4M3 has 4 significant bits, bf16 8) and
commutes with every rounding, so the FP8 pass is the bf16 pass on E~.

Dynamic activations (the same page: the FP8 checkpoint quantises activations at run time,
per token): reading used here, each row of the final hidden states h is quantised the same
way as an embedding row, with its own power-of-two scale chosen from that row alone when the
pass runs.  The FP8 x FP8 pass computes the logits of the dequantised rows h~ and E~,
S~ = h~ E~^T, i.e. the bf16 pass on (h~, E~): both are exact bf16 numbers, and so is every
product of two of them.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """Decode E4M3 codes (uint8) to fp64 (NaN for 0x7F and 0xFF)."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def _all_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_value(codes)
    keep = ~np.isnan(vals)
    return codes[keep], vals[keep]


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each finite |x| <= 448 (ties to the code with an even mantissa,
    i.e. an even code); +0 for zero."""
    x = np.asarray(x, np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("value beyond the E4M3 range")
    codes, vals = _all_codes()
    pos = vals >= 0
    pcodes, pvals = codes[pos & (codes < 0x80)], vals[pos & (codes < 0x80)]
    order = np.argsort(pvals)
    pcodes, pvals = pcodes[order], pvals[order]
    a = np.abs(x)
    i = np.clip(np.searchsorted(pvals, a), 1, len(pvals) - 1)
    lo, hi = pvals[i - 1], pvals[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & (pcodes[i] % 2 == 0))
    c = np.where(pick_hi, pcodes[i], pcodes[i - 1]).astype(np.uint8)
    c = np.where(a == 0, 0, c).astype(np.uint8)
    return np.where((x < 0) & (c != 0), c | 0x80, c).astype(np.uint8)


K_MIN = -117


def row_exponent(row_amax: np.ndarray) -> np.ndarray:
    """Smallest k >= K_MIN with amax <= 448 * 2^k."""
    out = np.empty(row_amax.shape, np.int64)
    for i, a in enumerate(np.asarray(row_amax, np.float64)):
        if a == 0:
            out[i] = K_MIN
            continue
        k = math.ceil(math.log2(a / E4M3_MAX))
        while a > E4M3_MAX * 2.0 ** k:        # guard the logarithm's rounding
            k += 1
        while a <= E4M3_MAX * 2.0 ** (k - 1):
            k -= 1
        out[i] = max(k, K_MIN)
    return out


def quantize_rows(E: np.ndarray):
    """fp64 values [V, d] -> (codes uint8 [V, d], exponents int [V])."""
    E = np.asarray(E, np.float64)
    k = row_exponent(np.max(np.abs(E), axis=1))
    return e4m3_round(E / np.exp2(k)[:, None]), k


def dequantize_rows(codes: np.ndarray, k: np.ndarray) -> np.ndarray:
    return e4m3_value(codes) * np.exp2(np.asarray(k, np.float64))[:, None]


def activation_rows(h_bits: np.ndarray):
    """Dynamic per-row quantisation of the final hidden states (bf16 bits [R, d]) for the
    FP8 x FP8 pass: (codes uint8 [R, d], exponents int [R], the dequantised rows h~ as bf16
    bits [R, d], exact)."""
    h = (np.asarray(h_bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, k = quantize_rows(h)
    hq = dequantize_rows(codes, k)
    bits = (hq.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64), hq)
    return codes, k, bits
