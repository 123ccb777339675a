"""Oracle for the vocab pass: per canvas position, everything the sampler needs from the
tied-unembedding logits, computed from the plain definitions in fp64.

Definitions followed (cited by page and section):

* logits  S_v = sum_k h_k E_{v,k} with the tied embedding E[V, d] used as the unembedding
  (DiffusionGemma Explained, "Tied embeddings" / final logits; Technical Report part 2/6,
  sec. 3.2 eq. (5)).
* tempered distribution  p = Softmax(S / T)  (Technical Report sec. 3.2 eq. (6);
  DiffusionGemma Explained, "Sampling" -> "Apply temperature").
* optional final-logit soft cap: S is replaced by c tanh(S / c) before the temperature
  (DiffusionGemma Explained, "Logit Softcapping" and the model's final-logits return); the
  argmax token stays that of S (tanh is increasing, so the capped logits have the same
  largest value at the same entries up to rounding; the plain reading keeps S's argmax).
* temperature schedule: decode pass i of N uses t_i = t_max + (i / N)(t_min - t_max)
  (DiffusionGemma Explained, "Sampling" -> "Apply temperature"; Technical Report sec. 3.3
  anneals from 0.8 to 0.4).
* lse = log sum_v exp(S_v / T); entropy H = -sum_v p_v log p_v = sum_v p_v (lse - z_v)
  (DiffusionGemma Explained, "Sampling" -> "Compute entropy").
* argmax token: the smallest v attaining max S (deterministic prediction used by the
  stability test; Technical Report sec. 3.3 "Adaptive stopping heuristic"; vLLM blog,
  convergence: committed tokens are the clean argmax).
* Gumbel-max sample: the smallest v attaining max (z'_v + g_v), g_v standard Gumbel noise
  from the Philox layout in ``oracle.philox`` (vLLM blog, sampler section: the candidate
  token is argmax(logits / T + Gumbel noise); DiffusionGemma Explained, "Sampling": accepted
  positions take a sample of their distribution).  z' = cap(S) / T_draw with the draw
  temperature T_draw, which is T unless the caller gives another one: the
  DiffusionGemma-Lite commit rule (section 4.2) reads its posterior p = softmax(logits)
  untempered and applies the annealed tau(k) to the x0-hat draw alone (item 4), so that
  sampler runs the statistics at T = 1 and the draw at T_draw = tau(k).
* confidence of a row: the probability of its argmax token under the distribution the
  statistics describe, p_{argmax} (the "conf" of the DiffusionGemma-Lite commit rule,
  section 4.2).
* self-conditioning expectation sc = sum_v p_v E_v = p_hat_0 E (Technical Report sec. 3.2
  eq. (6), the argument of FFW; DiffusionGemma Explained, "Self-conditioning").

Rows of commit canvases produce only the argmax token (vLLM blog: a converged canvas emits
its clean argmax and gets no further sampling or self-conditioning).

Decision margins (reported, used by the parity tests to exempt near-ties):
  mu_A = S_(1) - S_(2) and mu_G = y_(1) - y_(2) over distinct vocab indices, with
  y = z' + g the Gumbel keys: the distance from the decision to the nearest input that
  would change it (lowering the winner's key by more than the margin hands the decision to
  the runner-up).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from . import philox


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@dataclass
class RowResult:
    rows: np.ndarray        # global row ids
    lse: np.ndarray         # fp64, NaN for commit rows
    entropy: np.ndarray     # fp64, NaN for commit rows
    argmax: np.ndarray      # int64
    gumbel: np.ndarray      # int64, -1 for commit rows
    sc: Optional[np.ndarray]  # fp64 [n, d], NaN rows for commit rows
    mu_argmax: np.ndarray   # fp64 margins
    mu_gumbel: np.ndarray   # fp64 margins, inf for commit rows
    conf: Optional[np.ndarray] = None  # fp64 probability of the argmax token, NaN for commit rows
    argmax2: Optional[np.ndarray] = None  # runner-up of the argmax (-1 when V = 1)
    gumbel2: Optional[np.ndarray] = None  # runner-up of the Gumbel draw (-1: none)


def _top2_margin(x: np.ndarray) -> float:
    if x.shape[0] < 2:
        return np.inf
    i = int(np.argmax(x))
    best = x[i]
    rest = np.delete(x, i)
    return float(best - rest.max())


def _runner_up(x: np.ndarray) -> int:
    """The smallest index attaining the largest value among the indices other than the
    winner (the decision the margin separates the winner from); -1 for a single entry."""
    if x.shape[0] < 2:
        return -1
    i = int(np.argmax(x))
    y = x.copy()
    y[i] = -np.inf
    return int(np.argmax(y))


def vocab_pass_rows(E64: np.ndarray, h_bits: np.ndarray, rows: Sequence[int],
                    temperature_row: np.ndarray, commit_row: np.ndarray,
                    seed: int, step_row: np.ndarray, want_sc: bool = True,
                    row_block: int = 64, softcap: Optional[float] = None,
                    draw_temperature_row: Optional[np.ndarray] = None) -> RowResult:
    """Oracle results for the listed global rows.

    E64            fp64 [V, d] (the widened bf16 embedding)
    h_bits         bf16 bits [R, d] of the whole batch (only ``rows`` are read)
    temperature_row, commit_row, step_row: per global row (indexable by row id)
    softcap        None: z = S / T; c > 0: z = c tanh(S / c) / T
    draw_temperature_row: per global row, the temperature of the Gumbel-max draw alone
                   (None: the same as temperature_row)
    """
    if softcap is not None and not (softcap > 0 and math.isfinite(softcap)):
        raise ValueError("softcap must be finite and > 0")
    rows = np.asarray(rows, dtype=np.int64)
    V, d = E64.shape
    n = rows.shape[0]
    lse = np.full(n, np.nan)
    ent = np.full(n, np.nan)
    amax = np.zeros(n, dtype=np.int64)
    gtok = np.full(n, -1, dtype=np.int64)
    mu_a = np.zeros(n)
    mu_g = np.full(n, np.inf)
    conf = np.full(n, np.nan)
    am2 = np.full(n, -1, dtype=np.int64)
    gt2 = np.full(n, -1, dtype=np.int64)
    sc = np.full((n, d), np.nan) if want_sc else None
    for b0 in range(0, n, row_block):
        b1 = min(n, b0 + row_block)
        hb = widen_bf16(h_bits[rows[b0:b1]])
        S = hb @ E64.T                                   # [b, V] fp64 logits
        for j in range(b1 - b0):
            i = b0 + j
            r = int(rows[i])
            s = S[j]
            amax[i] = int(np.argmax(s))                  # first index attaining the max
            mu_a[i] = _top2_margin(s)
            am2[i] = _runner_up(s)
            if commit_row[r]:
                continue
            T = float(temperature_row[r])
            cs = s if softcap is None else softcap * np.tanh(s / softcap)
            z = cs / T
            Td = T if draw_temperature_row is None else float(draw_temperature_row[r])
            m = z.max()
            lse[i] = m + np.log(np.sum(np.exp(z - m)))
            p = np.exp(z - lse[i])
            ent[i] = float(np.sum(p * (lse[i] - z)))
            conf[i] = p[amax[i]]
            g = philox.gumbel_noise(r, V, seed, int(step_row[r]))
            y = cs / Td + g
            gtok[i] = int(np.argmax(y))
            mu_g[i] = _top2_margin(y)
            gt2[i] = _runner_up(y)
            if want_sc:
                sc[i] = p @ E64
    return RowResult(rows=rows, lse=lse, entropy=ent, argmax=amax, gumbel=gtok, sc=sc,
                     mu_argmax=mu_a, mu_gumbel=mu_g, conf=conf, argmax2=am2, gumbel2=gt2)


def temperature_schedule(i: int, N: int, t_max: float, t_min: float) -> float:
    """Temperature of decode pass i of N (i = 0 .. N - 1): linear from t_max toward t_min."""
    if not (N >= 1 and 0 <= i < N):
        raise ValueError("need 0 <= i < N")
    return t_max + (i / N) * (t_min - t_max)


def per_row(values_per_canvas: np.ndarray, C: int) -> np.ndarray:
    return np.repeat(np.asarray(values_per_canvas), C)
