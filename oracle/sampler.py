"""Oracle for the per-canvas accept / renoise / convergence step, in fp64.

Definitions followed:

* Entropy-bounded acceptance (Technical Report part 2/6, sec. 3.3 "Entropy-bounded token
  refinement"; DiffusionGemma Explained, "Sampling" -> "Keep a low-entropy prefix and
  renoise the rest"; vLLM blog, sampler section): order positions by entropy, lowest
  first, and accept the longest prefix of that order whose entropies *before* the
  position sum to at most the budget: position of rank k is accepted iff
  sum_{j<k} H_(j) <= budget.  Readings: the comparison is "<=" (the executable code on the
  DiffusionGemma Explained page); ties in entropy are ordered by position (stable sort).
* Accepted positions take their Gumbel-max sample; every other position is renoised with a
  uniform token drawn from the Philox renoise stream.
* Stability / convergence (Technical Report sec. 3.3 "Adaptive stopping heuristic";
  DiffusionGemma Explained, "Check for early stopping"; vLLM blog, convergence): the argmax
  canvas equals the previous step's argmax canvas at every position -> stable_count + 1,
  else 0; the canvas has converged when stable_count >= stability_threshold and the mean
  entropy is strictly below confidence_threshold.  prev_argmax = -1 marks "no previous
  canvas".
* Commit canvases (vLLM blog: a converged canvas is committed as its clean argmax): the
  next tokens are the argmax tokens, every position counts as accepted, the state resets
  (prev_argmax = -1, stable_count = 0) and converged = 0; mean entropy is not written.

Margins reported for the parity tests:
  mu_acc(i) = min(|P_rank(i) - budget|, min |H_i - H_j| over positions j with the other
  decision); mu_conv = |mean H - confidence_threshold|.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import philox


@dataclass
class SamplerResult:
    next_tokens: np.ndarray     # int64 [R]
    accept: np.ndarray          # uint8 [R]
    converged: np.ndarray       # uint8 [n]
    mean_entropy: np.ndarray    # fp64 [n], NaN for commit canvases
    prev_argmax: np.ndarray     # int64 [R] (updated state)
    stable_count: np.ndarray    # int64 [n] (updated state)
    mu_accept: np.ndarray       # fp64 [R], inf for commit canvases
    mu_conv: np.ndarray         # fp64 [n], inf for commit canvases


def accept_renoise(entropy, argmax_tok, gumbel_tok, commit, n_canvas: int, C: int, V: int,
                   budget: float, confidence: float, stability: int, seed: int, step,
                   prev_argmax, stable_count, canvas_ids=None) -> SamplerResult:
    """canvas_ids: the batch-wide indices of the n_canvas canvases given (default 0..n-1); the
    renoise counter of a position is its batch-wide row, canvas_id * C + position."""
    H = np.asarray(entropy, dtype=np.float64)
    am = np.asarray(argmax_tok, dtype=np.int64)
    gt = np.asarray(gumbel_tok, dtype=np.int64)
    prev = np.array(prev_argmax, dtype=np.int64, copy=True)
    cnt = np.array(stable_count, dtype=np.int64, copy=True)
    step = np.broadcast_to(np.asarray(step, dtype=np.int64), (n_canvas,))
    R = n_canvas * C
    nxt = np.zeros(R, dtype=np.int64)
    acc = np.zeros(R, dtype=np.uint8)
    conv = np.zeros(n_canvas, dtype=np.uint8)
    meanH = np.full(n_canvas, np.nan)
    mu_acc = np.full(R, np.inf)
    mu_conv = np.full(n_canvas, np.inf)
    for c in range(n_canvas):
        rows = np.arange(c * C, (c + 1) * C)
        if commit is not None and commit[c]:
            nxt[rows] = am[rows]
            acc[rows] = 1
            prev[rows] = -1
            cnt[c] = 0
            conv[c] = 0
            continue
        h = H[rows]
        order = sorted(range(C), key=lambda i: (h[i], i))
        before = 0.0
        prefix = np.zeros(C)
        for k, i in enumerate(order):
            prefix[i] = before
            before += h[i]
        a = prefix <= budget
        acc[rows] = a.astype(np.uint8)
        cid = c if canvas_ids is None else int(canvas_ids[c])
        ren = philox.renoise_tokens(np.arange(cid * C, (cid + 1) * C), V, seed, int(step[c]))
        nxt[rows] = np.where(a, gt[rows], ren)
        same = bool(np.all(am[rows] == prev[rows]))
        cnt[c] = cnt[c] + 1 if same else 0
        prev[rows] = am[rows]
        meanH[c] = math.fsum(h) / C
        conv[c] = 1 if (cnt[c] >= stability and meanH[c] < confidence) else 0
        # margins
        for i in range(C):
            m = abs(prefix[i] - budget)
            other = h[a != a[i]]
            if other.size:
                m = min(m, float(np.min(np.abs(other - h[i]))))
            mu_acc[rows[i]] = m
        mu_conv[c] = abs(meanH[c] - confidence)
    return SamplerResult(next_tokens=nxt, accept=acc, converged=conv, mean_entropy=meanH,
                         prev_argmax=prev, stable_count=cnt, mu_accept=mu_acc, mu_conv=mu_conv)


# ---------------------------------------------------------------------------------------
# The DiffusionGemma-Lite sampler (DiffusionGemma-Lite, section 4.2 "The commit rule" and
# section 4.4 "Entropy-bounded adaptive stopping"), a second sampler on the same vocabulary
# pass outputs.
#
#   commit    = (argmax == prev_argmax) | (conf >= prev_conf)     unchanged-or-stronger
#   new       = commit & ~committed                              frozen tokens stay
#   x         = new ? x0_draw : (committed ? x : uniform token)  uncommitted: redrawn
#   committed = committed | new;  prev_argmax = argmax;  prev_conf = conf
#   final     = committed ? x : x0_draw                          the returned canvas
#   adaptive stop: count = (mean H < threshold) ? count + 1 : 0, stopped when count >=
#   stability_steps; stability_steps = 0 turns it off (never stopped: the fixed schedule).
#
# Margins: the commit test compares two probabilities of the argmax token; conf >= prev_conf
# is ln conf >= ln prev_conf, a comparison of log-probabilities, i.e. of logits minus their
# log-partition, so its margin is taken on that scale (nats), like the argmax and Gumbel
# margins: mu_commit = |ln conf - ln prev_conf| (infinite where the argmax is unchanged and
# the rule commits regardless); the stop test's margin is |mean H - threshold| (nats).
#
# Readings: the posterior is p = softmax(logits), untempered (section 4.2 computes it so
# before the rule), so conf = max_v p_v is the probability of the argmax token under p and
# the stop test reads the mean entropy of p (section 4.4); only the x0-hat draw uses the
# annealed temperature tau(k) (section 4.2, item 4): x0_draw is the row's Gumbel-max sample
# of softmax(logits / tau(k)).  The vocabulary pass gives both at once when it runs its
# statistics at T = 1 and its draw at tau(k) (vocab_pass_rows' draw_temperature_row).  The
# uniform token comes from the same renoise stream as accept_renoise; the state starts at
# prev_argmax = -1, prev_conf = +inf, committed = 0 (no previous posterior: nothing commits
# at the first step).
# ---------------------------------------------------------------------------------------
@dataclass
class LiteResult:
    x: np.ndarray               # int64 [R] canvas after the step
    committed: np.ndarray       # uint8 [R]
    final: np.ndarray           # int64 [R]
    prev_argmax: np.ndarray     # int64 [R]
    prev_conf: np.ndarray       # fp64 [R]
    stable_count: np.ndarray    # int64 [n]
    converged: np.ndarray       # uint8 [n]
    mean_entropy: np.ndarray    # fp64 [n]
    mu_commit: np.ndarray       # fp64 [R]: |ln conf - ln prev_conf| where argmax changed, else inf
    mu_stop: np.ndarray         # fp64 [n]: |mean H - threshold|


def lite_step(entropy, argmax_tok, gumbel_tok, conf, n_canvas: int, C: int, V: int,
              threshold: float, stability_steps: int, seed: int, step, x, prev_argmax,
              prev_conf, committed, stable_count) -> LiteResult:
    H = np.asarray(entropy, np.float64)
    am = np.asarray(argmax_tok, np.int64)
    gt = np.asarray(gumbel_tok, np.int64)
    cf = np.asarray(conf, np.float64)
    x = np.array(x, np.int64, copy=True)
    pa = np.array(prev_argmax, np.int64, copy=True)
    pc = np.array(prev_conf, np.float64, copy=True)
    cm = np.array(committed, np.uint8, copy=True).astype(bool)
    cnt = np.array(stable_count, np.int64, copy=True)
    step = np.broadcast_to(np.asarray(step, np.int64), (n_canvas,))
    R = n_canvas * C
    final = np.zeros(R, np.int64)
    conv = np.zeros(n_canvas, np.uint8)
    meanH = np.zeros(n_canvas)
    mu_c = np.full(R, np.inf)
    mu_s = np.zeros(n_canvas)
    for c in range(n_canvas):
        rows = np.arange(c * C, (c + 1) * C)
        same = am[rows] == pa[rows]
        stronger = cf[rows] >= pc[rows]
        new = (same | stronger) & ~cm[rows]
        ren = philox.renoise_tokens(rows, V, seed, int(step[c]))
        x[rows] = np.where(new, gt[rows], np.where(cm[rows], x[rows], ren))
        cm[rows] |= new
        final[rows] = np.where(cm[rows], x[rows], gt[rows])
        with np.errstate(invalid="ignore", divide="ignore"):
            mu_c[rows] = np.where(same, np.inf, np.abs(np.log(cf[rows]) - np.log(pc[rows])))
        pa[rows] = am[rows]
        pc[rows] = cf[rows]
        meanH[c] = math.fsum(H[rows]) / C
        mu_s[c] = abs(meanH[c] - threshold)
        if stability_steps > 0:
            cnt[c] = cnt[c] + 1 if meanH[c] < threshold else 0
            conv[c] = 1 if cnt[c] >= stability_steps else 0
    return LiteResult(x=x, committed=cm.astype(np.uint8), final=final, prev_argmax=pa,
                      prev_conf=pc, stable_count=cnt, converged=conv, mean_entropy=meanH,
                      mu_commit=mu_c, mu_stop=mu_s)
