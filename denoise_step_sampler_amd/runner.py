"""Device-side buffers and one-call wrappers around the C entry points.

Allocation of inputs, outputs, state and workspace with torch (device memory only); every
computation is a libdg.so call.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from . import binding as B


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) -> device int16 tensor holding the same bytes."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


@dataclass
class VocabBuffers:
    n_canvas: int
    V: int
    d: int
    E: torch.Tensor
    h: torch.Tensor
    temperature: torch.Tensor
    commit: Optional[torch.Tensor]
    step: torch.Tensor
    lse: torch.Tensor
    entropy: torch.Tensor
    argmax_tok: torch.Tensor
    gumbel_tok: torch.Tensor
    selfcond: Optional[torch.Tensor]
    workspace: torch.Tensor
    # sampler state and outputs
    prev_argmax: torch.Tensor
    stable_count: torch.Tensor
    next_tokens: torch.Tensor
    accept_mask: torch.Tensor
    converged: torch.Tensor
    mean_entropy: torch.Tensor
    C: int = B.DG_CANVAS
    extra: dict = field(default_factory=dict)
    # temperature of the Gumbel-max draw alone ([n_canvas] fp32), or None: the draw uses
    # `temperature` (the DiffusionGemma-Lite sampler: statistics at 1, the draw at tau(k))
    draw_temperature: Optional[torch.Tensor] = None
    # the prepared fp16 embedding (embedding_f16), or None: each pass builds it in
    # its workspace
    E16: Optional[torch.Tensor] = None

    @property
    def R(self) -> int:
        return self.n_canvas * self.C


def embedding_f16(E: torch.Tensor, V: int, d: int, stream=None) -> torch.Tensor:
    """The fp16 embedding the expectation multiplies (once per embedding)."""
    t = torch.empty(d * B.e16_rows(V), dtype=torch.int16, device=E.device)
    B.dg_embedding_f16(E, V, d, t, stream=stream)
    return t


def allocate(n_canvas: int, V: int, d: int, E: torch.Tensor, h: torch.Tensor,
             temperature, commit, step, want_selfcond: bool = True,
             sentinel: float = float("nan"), device="cuda",
             E16: Optional[torch.Tensor] = None) -> VocabBuffers:
    """E16: the prepared fp16 embedding, or None (each pass builds one)."""
    R = n_canvas * B.DG_CANVAS
    f32 = dict(dtype=torch.float32, device=device)
    i32 = dict(dtype=torch.int32, device=device)
    u8 = dict(dtype=torch.uint8, device=device)
    ws_bytes = B.dg_vocab_pass_ex_workspace_size(n_canvas, B.DG_CANVAS, V, d, E16 is not None)
    if ws_bytes == 0:
        raise ValueError(f"unsupported shape n={n_canvas} V={V} d={d}")
    return VocabBuffers(
        n_canvas=n_canvas, V=V, d=d, E=E, h=h,
        temperature=torch.as_tensor(np.asarray(temperature, np.float32)).to(device),
        commit=None if commit is None else torch.as_tensor(np.asarray(commit, np.uint8)).to(device),
        step=torch.as_tensor(np.asarray(step, np.int32)).to(device),
        lse=torch.full((R,), sentinel, **f32),
        entropy=torch.full((R,), sentinel, **f32),
        argmax_tok=torch.full((R,), -7, **i32),
        gumbel_tok=torch.full((R,), -7, **i32),
        selfcond=torch.full((R, d), sentinel, **f32) if want_selfcond else None,
        workspace=torch.empty(ws_bytes, **u8),
        prev_argmax=torch.full((R,), -1, **i32),
        stable_count=torch.zeros(n_canvas, **i32),
        next_tokens=torch.full((R,), -7, **i32),
        accept_mask=torch.full((R,), 7, **u8),
        converged=torch.full((n_canvas,), 7, **u8),
        mean_entropy=torch.full((n_canvas,), sentinel, **f32), E16=E16)


def from_workload(wl, want_selfcond: bool = True, device="cuda", E: Optional[torch.Tensor] = None,
                  commit_any: Optional[bool] = None,
                  E16: Optional[torch.Tensor] = None) -> VocabBuffers:
    E_t = bf16_tensor(wl.E, device) if E is None else E
    commit = wl.commit if (commit_any if commit_any is not None else bool(wl.commit.any())) else None
    return allocate(wl.n_canvas, wl.V, wl.d, E_t, bf16_tensor(wl.h, device), wl.temperature,
                    commit, wl.step, want_selfcond=want_selfcond, device=device, E16=E16)


def vocab_pass(b: VocabBuffers, seed: int, stream=None, softcap: Optional[float] = None) -> None:
    """softcap: None for the plain logits, c > 0 for c tanh(S / c) before the temperature.
    With b.draw_temperature the Gumbel-max draw takes that temperature, with b.E16 the
    expectation multiplies the prepared embedding (both through dg_vocab_pass_ex)."""
    if b.draw_temperature is not None or b.E16 is not None:
        B.dg_vocab_pass_ex(b.E, b.E16, b.h, b.n_canvas, b.C, b.V, b.d, b.temperature,
                           b.draw_temperature,
                           0.0 if softcap is None else float(softcap), b.commit, seed, b.step,
                           b.lse, b.entropy, b.argmax_tok, b.gumbel_tok, b.selfcond, b.workspace,
                           stream=stream)
        return
    args = (b.E, b.h, b.n_canvas, b.C, b.V, b.d, b.temperature, b.commit, seed, b.step, b.lse,
            b.entropy, b.argmax_tok, b.gumbel_tok, b.selfcond, b.workspace)
    if softcap is None:
        B.dg_vocab_pass(*args, stream=stream)
    else:
        B.dg_vocab_pass_softcap(*args, stream=stream, softcap=softcap)


@dataclass
class FfwWeights:
    """Device copies of the self-conditioning MLP (bf16 bits as int16)."""
    D: int
    F: int
    pre_norm: torch.Tensor
    W_gate: torch.Tensor
    W_up: torch.Tensor
    W_down: torch.Tensor
    eps: float = 1e-6


def ffw_weights(pre, Wg, Wu, Wd, eps: float = 1e-6, device="cuda") -> FfwWeights:
    D, F = Wd.shape
    return FfwWeights(D=D, F=F, pre_norm=bf16_tensor(pre, device), W_gate=bf16_tensor(Wg, device),
                      W_up=bf16_tensor(Wu, device), W_down=bf16_tensor(Wd, device), eps=eps)


def ffw_workspace(n_canvas: int, D: int, F: int, device="cuda") -> torch.Tensor:
    n = B.dg_selfcond_input_workspace_size(n_canvas, B.DG_CANVAS, D, F)
    if n == 0:
        raise ValueError(f"unsupported shape n={n_canvas} D={D} F={F}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def selfcond_input(b: VocabBuffers, W: FfwWeights, out: torch.Tensor, workspace: torch.Tensor,
                   first_step: bool = False, stream=None) -> None:
    """The next step's input rows from b.selfcond and b.next_tokens (first_step: no
    self-conditioning signal yet)."""
    B.dg_selfcond_input(None if first_step else b.selfcond, b.next_tokens, b.E, W.pre_norm,
                        W.W_gate, W.W_up, W.W_down, b.commit, b.n_canvas, b.C, b.V, b.d, W.F,
                        W.eps, out, workspace, stream=stream)


@dataclass
class LiteState:
    """State and outputs of the DiffusionGemma-Lite sampler for a batch of canvases."""
    x: torch.Tensor
    prev_argmax: torch.Tensor
    prev_conf: torch.Tensor
    committed: torch.Tensor
    stable_count: torch.Tensor
    conf: torch.Tensor
    final_tokens: torch.Tensor
    converged: torch.Tensor
    mean_entropy: torch.Tensor


def lite_state(n_canvas: int, device="cuda") -> LiteState:
    """The initial state: no previous posterior (prev_argmax -1, prev_conf +inf), nothing
    committed, canvas tokens 0 (every position is redrawn at the first step)."""
    R = n_canvas * B.DG_CANVAS
    i32 = dict(dtype=torch.int32, device=device)
    return LiteState(x=torch.zeros(R, **i32), prev_argmax=torch.full((R,), -1, **i32),
                     prev_conf=torch.full((R,), float("inf"), dtype=torch.float32, device=device),
                     committed=torch.zeros(R, dtype=torch.uint8, device=device),
                     stable_count=torch.zeros(n_canvas, **i32),
                     conf=torch.empty(R, dtype=torch.float32, device=device),
                     final_tokens=torch.empty(R, **i32),
                     converged=torch.zeros(n_canvas, dtype=torch.uint8, device=device),
                     mean_entropy=torch.empty(n_canvas, dtype=torch.float32, device=device))


def lite_step(b: VocabBuffers, s: LiteState, threshold: float, stability_steps: int, seed: int,
              softcap: Optional[float] = None, stream=None) -> None:
    """The Lite sampler on the outputs of the vocabulary pass in b."""
    B.dg_lite_step(b.h, b.E, b.temperature, b.lse, b.entropy, b.argmax_tok, b.gumbel_tok,
                   b.n_canvas, b.C, b.V, b.d, 0.0 if softcap is None else softcap, threshold,
                   stability_steps, seed, b.step, s.conf, s.x, s.prev_argmax, s.prev_conf,
                   s.committed, s.stable_count, s.final_tokens, s.converged, s.mean_entropy,
                   stream=stream)


@dataclass
class Fp8Embedding:
    """The FP8 form of an embedding on the device: E4M3 codes, per-row exponents, and the
    dequantised rows as fp16, which the expectation multiplies (or None: built per pass)."""
    codes: torch.Tensor
    E16: Optional[torch.Tensor]
    row_exp: torch.Tensor


def quantize_embedding_fp8(E: torch.Tensor, V: int, d: int, stream=None,
                           with_e16: bool = True) -> Fp8Embedding:
    f = Fp8Embedding(codes=torch.empty(V * d, dtype=torch.uint8, device=E.device),
                     E16=(torch.empty(d * B.e16_rows(V), dtype=torch.int16, device=E.device)
                           if with_e16 else None),
                     row_exp=torch.empty(V, dtype=torch.int32, device=E.device))
    B.dg_quantize_embedding_fp8(E, V, d, f.codes, f.E16, f.row_exp, stream=stream)
    return f


def fp8_workspace(n_canvas: int, V: int, d: int, device="cuda",
                  activations: bool = False) -> torch.Tensor:
    """Workspace of vocab_pass_fp8 (activations=True: of the FP8 x FP8 pass)."""
    f = B.dg_vocab_pass_fp8_dyn_workspace_size if activations else B.dg_vocab_pass_fp8_workspace_size
    n = f(n_canvas, B.DG_CANVAS, V, d)
    if n == 0:
        raise ValueError(f"unsupported shape n={n_canvas} V={V} d={d}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def vocab_pass_fp8(b: VocabBuffers, f: Fp8Embedding, workspace: torch.Tensor, seed: int,
                   stream=None, softcap: Optional[float] = None,
                   activations: bool = False) -> None:
    """The vocabulary pass on the FP8 embedding f (b.E is not read); activations=True
    quantises h per row too and multiplies FP8 by FP8 (workspace from
    fp8_workspace(..., activations=True))."""
    fn = B.dg_vocab_pass_fp8_dyn if activations else B.dg_vocab_pass_fp8
    fn(f.codes, f.E16, f.row_exp, b.h, b.n_canvas, b.C, b.V, b.d, b.temperature, b.commit, seed,
       b.step, b.lse, b.entropy, b.argmax_tok, b.gumbel_tok, b.selfcond, workspace,
       stream=stream, softcap=0.0 if softcap is None else softcap)


def temperature_schedule(i: int, N: int, t_max: float, t_min: float) -> float:
    """Temperature of decode pass i of N (0 <= i < N): linear from t_max toward t_min in steps
    of (t_min - t_max) / N (DiffusionGemma Explained, "Sampling" -> "Apply temperature")."""
    if not (N >= 1 and 0 <= i < N):
        raise ValueError(f"decode pass {i} outside [0, {N})")
    return t_max + (t_min - t_max) * (i / N)


def accept_renoise(b: VocabBuffers, budget: float, confidence: float, stability: int, seed: int,
                   stream=None) -> None:
    B.dg_accept_renoise(b.entropy, b.argmax_tok, b.gumbel_tok, b.commit, b.n_canvas, b.C, b.V,
                        budget, confidence, stability, seed, b.step, b.prev_argmax,
                        b.stable_count, b.next_tokens, b.accept_mask, b.converged,
                        b.mean_entropy, stream=stream)


def denoise_step(b: VocabBuffers, budget: float, confidence: float, stability: int, seed: int,
                 stream=None, softcap: Optional[float] = None) -> None:
    """One step of the hot path: vocabulary pass, then accept/renoise/convergence."""
    vocab_pass(b, seed, stream, softcap)
    accept_renoise(b, budget, confidence, stability, seed, stream)


@dataclass
class LoopResult:
    steps_run: int
    steps_to_converge: np.ndarray   # [n_canvas] step after which the canvas converged, -1 if never
    positions: int                  # sum over steps of active canvases x C
    step_ms: list                   # GPU time of each step (vocabulary pass + accept/renoise)

    @property
    def positions_per_s(self) -> float:
        return self.positions / (sum(self.step_ms) * 1e-3)


def run_loop(wl, seed: int, max_steps: int = 32, stream=None, on_step=None,
             E: Optional[torch.Tensor] = None, schedule: Optional[tuple] = None,
             softcap: Optional[float] = None) -> LoopResult:
    """The full denoise loop of the full_loop workload: at step k the hidden states come from
    synth.loop_hidden (signal 0.5 + 0.25 k, kept only at the positions accepted at step
    k - 1), then one vocabulary pass and accept/renoise run on the canvases that have not
    converged; a canvas leaves the batch once converged, and the loop ends when none is left
    or after max_steps.  Hidden-state synthesis and its upload are outside the timed region.

    on_step(k, b, canvases, state_in) is called after each step with the buffers, the
    original canvas ids in the batch and the host copies of the sampler state the step
    started from (prev_argmax, stable_count).
    schedule: None keeps each canvas's workload temperature; (t_max, t_min) gives every
    canvas temperature_schedule(k, max_steps, t_max, t_min) at step k.  softcap as in
    vocab_pass."""
    from . import synth
    stream = stream if stream is not None else torch.cuda.current_stream()
    n, C = wl.n_canvas, B.DG_CANVAS
    E_t = bf16_tensor(wl.E) if E is None else E
    active = np.arange(n)
    prev = np.full(n * C, -1, np.int32)        # sampler state of every canvas (host copy)
    cnt = np.zeros(n, np.int32)
    accepted_prev = None
    steps_to_converge = np.full(n, -1, np.int64)
    positions, step_ms, b = 0, [], None
    for k in range(max_steps):
        if active.size == 0:
            break
        h_all = synth.loop_hidden(wl, k, accepted_prev)
        rows = (active[:, None] * C + np.arange(C)[None, :]).reshape(-1)
        temp = (wl.temperature[active] if schedule is None else
                np.full(active.size, temperature_schedule(k, max_steps, *schedule), np.float32))
        if b is None or b.n_canvas != active.size:
            b = allocate(active.size, wl.V, wl.d, E_t, bf16_tensor(h_all[rows]), temp, None,
                         np.full(active.size, k, np.int32))
            b.prev_argmax.copy_(torch.from_numpy(prev[rows]))
            b.stable_count.copy_(torch.from_numpy(cnt[active]))
        else:
            b.h.copy_(bf16_tensor(h_all[rows]))
            b.step.fill_(k)
            b.temperature.copy_(torch.from_numpy(np.asarray(temp, np.float32)))
        state_in = (b.prev_argmax.cpu().numpy(), b.stable_count.cpu().numpy())
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        denoise_step(b, wl.budget, wl.confidence, wl.stability, seed, stream, softcap)
        t1.record(stream)
        t1.synchronize()
        step_ms.append(t0.elapsed_time(t1))
        positions += active.size * C
        if on_step is not None:
            on_step(k, b, active.copy(), state_in)
        acc = b.accept_mask.cpu().numpy().astype(bool)
        conv = b.converged.cpu().numpy().astype(bool)
        accepted_prev = np.zeros(n * C, bool) if accepted_prev is None else accepted_prev.copy()
        accepted_prev[rows] = acc
        prev[rows] = b.prev_argmax.cpu().numpy()
        cnt[active] = b.stable_count.cpu().numpy()
        steps_to_converge[active[conv]] = k
        active = active[~conv]
    return LoopResult(steps_run=len(step_ms), steps_to_converge=steps_to_converge,
                      positions=positions, step_ms=step_ms)


def run_loop_device(wl, seed: int, max_steps: int = 32, stream=None,
                    E: Optional[torch.Tensor] = None, E16: Optional[torch.Tensor] = None,
                    schedule: Optional[tuple] = None, softcap: Optional[float] = None,
                    noise_seed: int = 0) -> LoopResult:
    """The full-loop workload with no host round trip inside the loop: the hidden states of
    step k, s_k E[target] kept where step k - 1 accepted plus N(0, 1) noise, are synthesised on
    the device (torch's generator, seeded per step; the same recipe as synth.loop_hidden with
    another random stream), and a canvas that has converged stays in the batch as a commit
    canvas (its argmax only, as a converged canvas is committed) instead of leaving it.  Each
    step's GPU time is taken with events around the step alone (synthesis excluded)."""
    from . import synth
    stream = stream if stream is not None else torch.cuda.current_stream()
    n, C = wl.n_canvas, B.DG_CANVAS
    R, dev = n * C, "cuda"
    E_t = bf16_tensor(wl.E) if E is None else E
    tgt = torch.from_numpy(wl.targets.astype(np.int64)).to(dev)
    E_tgt = E_t.view(torch.bfloat16).reshape(wl.V, wl.d)[tgt].float()
    b = allocate(n, wl.V, wl.d, E_t, bf16_tensor(wl.h), wl.temperature, np.zeros(n, np.uint8),
                 np.zeros(n, np.int32), E16=E16)
    keep = torch.ones(R, dtype=torch.float32, device=dev)
    done = torch.zeros(n, dtype=torch.bool, device=dev)
    stc = torch.full((n,), -1, dtype=torch.int64, device=dev)
    active = torch.zeros(max_steps, dtype=torch.int64, device=dev)
    gen = torch.Generator(device=dev)
    events = []
    with torch.cuda.stream(stream):
        for k in range(max_steps):
            gen.manual_seed(noise_seed * 1000003 + k)
            noise = torch.randn((R, wl.d), generator=gen, device=dev, dtype=torch.float32)
            s_k = synth.loop_scale(k, wl.extra.get("signal", (0.5, 0.25)))
            h = E_tgt * (s_k * keep)[:, None] + noise
            b.h.copy_(h.to(torch.bfloat16).view(torch.int16))
            b.step.fill_(k)
            if schedule is not None:
                b.temperature.fill_(temperature_schedule(k, max_steps, *schedule))
            b.commit.copy_(done.to(torch.uint8))
            active[k] = (~done).sum()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            denoise_step(b, wl.budget, wl.confidence, wl.stability, seed, stream, softcap)
            t1.record(stream)
            events.append((t0, t1))
            keep = b.accept_mask.float()
            new = b.converged.bool() & ~done
            stc = torch.where(new, torch.full_like(stc, k), stc)
            done = done | new
    torch.cuda.synchronize()
    act = active.cpu().numpy()
    return LoopResult(steps_run=max_steps, steps_to_converge=stc.cpu().numpy(),
                      positions=int(act.sum()) * C,
                      step_ms=[a.elapsed_time(z) for a, z in events])
