"""Seeded synthetic inputs for the denoise-step vocab pass, accept/renoise and q_sample.

This module only draws random inputs and rounds them to bf16.  It holds none of the
sampler's arithmetic (no logits, softmax, entropy, noise transforms or decisions), so
both the fp64 CPU oracle and the HIP path can be fed from it.

Workloads (DiffusionGemma Explained, "Sampling"; DiffusionGemma Technical Report part 2/6,
section 3.2 "The Denoising Framework at Inference"): a canvas holds C = 256 positions; the
final hidden state of each position is contracted with the tied embedding E[V, d].  The
synthetic hidden state of a position is ``scale * E[target] + N(0, 1)`` so that the target
token carries signal of tunable strength.

Every array is produced by numpy ``default_rng`` streams keyed by ``(seed, purpose)``, so a
piece (say E) is identical across workloads that share ``(V, d, seed)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

C_CANVAS = 256

# purposes of the independent random streams
_S_EMBED, _S_TARGET, _S_SCALE, _S_NOISE, _S_QS_X0, _S_QS_T, _S_FFW = 1, 2, 3, 4, 5, 6, 7


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_embedding(V: int, d: int, seed: int, chunk_rows: int = 16384) -> np.ndarray:
    """E ~ N(0, 1/d) as bf16 bits [V, d], generated in fixed row chunks."""
    rng = np.random.default_rng([seed, _S_EMBED, V, d])
    out = np.empty((V, d), dtype=np.uint16)
    s = np.float32(1.0 / math.sqrt(d))
    for r0 in range(0, V, chunk_rows):
        r1 = min(V, r0 + chunk_rows)
        blk = rng.standard_normal((r1 - r0, d), dtype=np.float32)
        blk *= s
        out[r0:r1] = round_to_bf16(blk)
    return out


def make_targets(R: int, V: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, _S_TARGET, R, V])
    return rng.integers(0, V, size=R, dtype=np.int64).astype(np.int32)


def make_hidden(E: np.ndarray, targets: np.ndarray, scale: np.ndarray, seed: int,
                step: int = 0, keep_signal: Optional[np.ndarray] = None) -> np.ndarray:
    """h[r] = scale[r] * E[target[r]] + N(0, 1), rounded to bf16 bits [R, d].

    ``keep_signal`` (bool [R]) zeroes the signal term where False (full-loop workload).
    ``step`` selects an independent noise stream per denoise step.
    """
    R = targets.shape[0]
    d = E.shape[1]
    rng = np.random.default_rng([seed, _S_NOISE, R, d, step])
    noise = rng.standard_normal((R, d), dtype=np.float32)
    sc = np.asarray(scale, dtype=np.float32).reshape(R, 1)
    if keep_signal is not None:
        sc = sc * np.asarray(keep_signal, dtype=np.float32).reshape(R, 1)
    sig = bf16_to_f32(E[targets]) * sc
    return round_to_bf16(sig + noise)


def make_ffw_weights(D: int, F: int, seed: int) -> Tuple[np.ndarray, ...]:
    """Random bf16 weights of the self-conditioning MLP: pre-norm weight 1 + 0.1 N(0, 1) [D],
    W_gate and W_up N(0, 1 / D) [F, D], W_down N(0, 1 / F) [D, F]."""
    rng = np.random.default_rng([seed, _S_FFW, D, F])
    pre = round_to_bf16((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    Wg = round_to_bf16((rng.standard_normal((F, D)) / math.sqrt(D)).astype(np.float32))
    Wu = round_to_bf16((rng.standard_normal((F, D)) / math.sqrt(D)).astype(np.float32))
    Wd = round_to_bf16((rng.standard_normal((D, F)) / math.sqrt(F)).astype(np.float32))
    return pre, Wg, Wu, Wd


def make_selfcond_rows(E: np.ndarray, R: int, seed: int, k: int = 4) -> np.ndarray:
    """Stand-ins for self-conditioning rows: random convex mixtures (Dirichlet(1) weights) of
    k random embedding rows, fp32 [R, d]; plus the tokens of the next canvas, uniform [R]."""
    V, d = E.shape
    rng = np.random.default_rng([seed, _S_FFW, R, V, d])
    idx = rng.integers(0, V, size=(R, k))
    wts = rng.dirichlet(np.ones(k), size=R).astype(np.float32)
    rows = np.einsum("rk,rkd->rd", wts, bf16_to_f32(E[idx])).astype(np.float32)
    return rows, rng.integers(0, V, size=R).astype(np.int32)


def cosine_kappa(t: np.ndarray, T: int) -> np.ndarray:
    """Keep probability of the cosine schedule, cos^2(pi/2 * t/T), in fp64 then fp32.

    This is an input of q_sample (the caller owns the schedule), computed once here.
    """
    return np.cos(0.5 * math.pi * np.asarray(t, dtype=np.float64) / T) ** 2


@dataclass
class VocabWorkload:
    """One batch of the vocab pass + accept/renoise."""
    name: str
    n_canvas: int
    V: int
    d: int
    temperature: np.ndarray          # fp32 [n]
    commit: np.ndarray               # u8 [n]
    budget: float
    confidence: float
    stability: int
    seed: int
    step: np.ndarray                 # int32 [n]
    E: np.ndarray                    # bf16 bits [V, d]
    h: np.ndarray                    # bf16 bits [R, d]
    targets: np.ndarray              # int32 [R]
    scale: np.ndarray                # fp32 [R]
    C: int = C_CANVAS
    extra: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return self.n_canvas * self.C


def _canvas_scales(n: int, lo: float, hi: float, seed: int, per_position: bool) -> np.ndarray:
    rng = np.random.default_rng([seed, _S_SCALE, n])
    if per_position:
        return rng.uniform(lo, hi, size=n * C_CANVAS).astype(np.float32)
    s = rng.uniform(lo, hi, size=n).astype(np.float32)
    return np.repeat(s, C_CANVAS)


def workload(name: str, seed: int = 0, V: Optional[int] = None, d: Optional[int] = None,
             n_canvas: Optional[int] = None, E: Optional[np.ndarray] = None) -> VocabWorkload:
    """Build one of the named workloads.  V, d, n_canvas override the sizes (smaller
    variants with the same recipe, for fast tests).

    tiny      : 1 x 256, V=4096,  d=256,  h = 3 E[t] + N(0,1), T=1.0
    lite      : 4 x 256, V=50257, d=1024, per-position scale U[0.5, 4], T=1.0
    large_v   : 1 x 256, V=262144, d=2816, scale 2, T=0.8
    batched   : 32 x 256, V=262144, d=2816, per-canvas scale U[0.3, 5], canvases c%4==3 commit
    full_loop : 8 x 256, V=262144, d=2816 (step 0 of the loop; later steps via loop_hidden)
    """
    presets = {
        "tiny": dict(n=1, V=4096, d=256, T=1.0),
        "lite": dict(n=4, V=50257, d=1024, T=1.0),
        "large_v": dict(n=1, V=262144, d=2816, T=0.8),
        "batched": dict(n=32, V=262144, d=2816, T=0.8),
        "full_loop": dict(n=8, V=262144, d=2816, T=0.8),
    }
    p = presets[name]
    n = n_canvas if n_canvas is not None else p["n"]
    V = V if V is not None else p["V"]
    d = d if d is not None else p["d"]
    R = n * C_CANVAS
    if E is None:
        E = make_embedding(V, d, seed)
    tg = make_targets(R, V, seed)
    if name == "tiny":
        scale = np.full(R, 3.0, dtype=np.float32)
    elif name == "lite":
        scale = _canvas_scales(n, 0.5, 4.0, seed, per_position=True)
    elif name == "large_v":
        scale = np.full(R, 2.0, dtype=np.float32)
    elif name == "batched":
        scale = _canvas_scales(n, 0.3, 5.0, seed, per_position=False)
    else:  # full_loop, step 0: s_0 = 0.5, every position keeps its signal
        scale = np.full(R, 0.5, dtype=np.float32)
    h = make_hidden(E, tg, scale, seed, step=0)
    commit = np.zeros(n, dtype=np.uint8)
    if name == "batched":
        commit[np.arange(n) % 4 == 3] = 1
    wl = VocabWorkload(
        name=name, n_canvas=n, V=V, d=d,
        temperature=np.full(n, p["T"], dtype=np.float32),
        commit=commit, budget=4.0,
        confidence=0.1 if name == "full_loop" else 0.005,
        stability=2 if name == "full_loop" else 1,
        seed=seed, step=np.zeros(n, dtype=np.int32),
        E=E, h=h, targets=tg, scale=scale)
    return wl


def loop_scale(k: int, signal=(0.5, 0.25)) -> float:
    """Signal strength of denoise step k in the full-loop workload: a + b k, (a, b) = (0.5,
    0.25) for the workload as specified (a test may ask for a faster-growing signal)."""
    return signal[0] + signal[1] * k


def loop_hidden(wl: VocabWorkload, k: int, accepted_prev: Optional[np.ndarray]) -> np.ndarray:
    """Hidden state of step k of the full-loop workload.  ``accepted_prev`` (bool [R]) is the
    previous step's accept mask (None at step 0: every position keeps its signal).  The signal
    schedule is wl.extra["signal"] if set, else (0.5, 0.25)."""
    scale = np.full(wl.R, loop_scale(k, wl.extra.get("signal", (0.5, 0.25))), dtype=np.float32)
    return make_hidden(wl.E, wl.targets, scale, wl.seed, step=k, keep_signal=accepted_prev)


@dataclass
class QSampleWorkload:
    n_canvas: int
    V: int
    x0: np.ndarray      # int32 [n*C]
    t: np.ndarray       # int32 [n]
    kappa: np.ndarray   # fp32 [n]
    seed: int
    C: int = C_CANVAS


def qsample_workload(n_canvas: int = 64, V: int = 50257, T_sched: int = 16,
                     seed: int = 0) -> QSampleWorkload:
    """Clean canvases and per-canvas times t ~ U{1..T}, keep probability from the cosine
    schedule (DiffusionGemma-Lite, "Forward process")."""
    r1 = np.random.default_rng([seed, _S_QS_X0, n_canvas, V])
    x0 = r1.integers(0, V, size=n_canvas * C_CANVAS, dtype=np.int64).astype(np.int32)
    r2 = np.random.default_rng([seed, _S_QS_T, n_canvas])
    t = r2.integers(1, T_sched + 1, size=n_canvas, dtype=np.int64).astype(np.int32)
    kappa = cosine_kappa(t, T_sched).astype(np.float32)
    return QSampleWorkload(n_canvas=n_canvas, V=V, x0=x0, t=t, kappa=kappa, seed=seed)
