"""Seeded fuzz of the vocabulary pass against the oracle, workspace poisoning, and invariance
of the results to how the batch is split across the GPU.

* Fuzz: random small shapes (V in [16, 5000], d a multiple of 128 up to 768, one or three
  canvases), temperatures from 0.3 to 50, commit flags, soft caps, separate draw temperatures
  and prepared fp16 embeddings, each case against the oracle at the bars
  of the hot-path contract; the loop stops at the first failing case and names it.
* Poisoned workspace: the workspace filled with 0xFF bytes (NaN floats, -1 integers) before
  the call gives bit-identical outputs to a zero-filled one, so every partial the kernels
  read was written by the same call.
* Split invariance: the pass distributes a canvas's vocabulary over a number of workgroups
  that depends on how many canvases share the call; a canvas computed alone and inside a
  batch of five must give the same argmax and the same statistics to fp32 rounding.
"""
import math
import sys

import numpy as np
import pytest

from denoise_step_sampler_amd import synth
from oracle import vocab_pass as ovp
from parity import VocabInputs, compare_vocab

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
C = 256


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from denoise_step_sampler_amd import binding
    binding.load()
    yield


def _host(b):
    return {"lse": b.lse.cpu().numpy(), "entropy": b.entropy.cpu().numpy(),
            "argmax": b.argmax_tok.cpu().numpy(), "gumbel": b.gumbel_tok.cpu().numpy(),
            "sc": None if b.selfcond is None else b.selfcond.cpu().numpy()}


def _case(i):
    rng = np.random.default_rng([2026, i])
    V = int(rng.integers(16, 5001))
    d = int(128 * rng.integers(1, 7))
    n = int(rng.choice([1, 3]))
    T = np.exp(rng.uniform(math.log(0.3), math.log(50.0), n)).astype(np.float32)
    commit = (rng.random(n) < 0.3).astype(np.uint8)
    commit[0] = 0
    softcap = float(rng.uniform(2.0, 40.0)) if rng.random() < 0.3 else None
    draw = (np.exp(rng.uniform(math.log(0.3), math.log(3.0), n)).astype(np.float32)
            if rng.random() < 0.3 else None)
    scale = float(rng.choice([0.5, 1.0, 3.0]))
    return dict(V=V, d=d, n=n, T=T, commit=commit, softcap=softcap, draw=draw, scale=scale,
                seed=int(rng.integers(0, 2 ** 63)), wseed=int(rng.integers(0, 1000)),
                want_sc=bool(rng.random() < 0.8), prepared=bool(rng.random() < 0.5))


def test_seeded_fuzz_against_the_oracle():
    from denoise_step_sampler_amd import runner
    n_cases = 24
    for i in range(n_cases):
        p = _case(i)
        label = (f"case {i}: V={p['V']} d={p['d']} n={p['n']} T={np.round(p['T'], 3).tolist()} "
                 f"commit={p['commit'].tolist()} softcap={p['softcap']} "
                 f"draw={None if p['draw'] is None else np.round(p['draw'], 3).tolist()} "
                 f"scale={p['scale']} sc={p['want_sc']} prepared={p['prepared']}")
        _say("[fuzz]", label)
        wl = synth.workload("lite", V=p["V"], d=p["d"], n_canvas=p["n"], seed=p["wseed"])
        wl.h = synth.round_to_bf16(synth.bf16_to_f32(wl.h) * np.float32(p["scale"]))
        wl.temperature = p["T"]
        wl.commit = p["commit"]
        wl.step = np.arange(p["n"], dtype=np.int32) * 3 + i
        E_t = runner.bf16_tensor(wl.E)
        b = runner.from_workload(wl, want_selfcond=p["want_sc"], commit_any=True, E=E_t,
                                 E16=runner.embedding_f16(E_t, wl.V, wl.d) if p["prepared"]
                                 else None)
        if p["draw"] is not None:
            b.draw_temperature = torch.as_tensor(p["draw"]).cuda()
        runner.vocab_pass(b, p["seed"], softcap=p["softcap"])
        torch.cuda.synchronize()
        E64 = ovp.widen_bf16(wl.E)
        Trow, st = np.repeat(wl.temperature, C), np.repeat(wl.step, C)
        draw_row = None if p["draw"] is None else np.repeat(p["draw"], C)
        cm = np.repeat(wl.commit.astype(bool), C)
        ref = ovp.vocab_pass_rows(E64, wl.h, np.arange(wl.R), Trow, cm, p["seed"], st,
                                  want_sc=p["want_sc"], softcap=p["softcap"],
                                  draw_temperature_row=draw_row)
        try:
            rep = compare_vocab(_host(b), ref, cm,
                                inputs=VocabInputs(E64, wl.h, Trow, st, p["seed"], p["softcap"],
                                                   draw_row))
        except AssertionError as e:
            raise AssertionError(f"{label}: {e}") from None
        _say("   ", rep)


@pytest.mark.parametrize("V,d,n,fp8", [(3000, 256, 3, False), (1000, 384, 2, False),
                                       (20000, 1024, 5, False), (2500, 256, 2, True)])
def test_poisoned_workspace_gives_identical_results(V, d, n, fp8):
    """Workspace bytes 0xFF (NaN / -1 everywhere) and 0x00 before the call: identical bits."""
    from denoise_step_sampler_amd import runner
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=12)
    wl.commit = (np.arange(n) % 3 == 1).astype(np.uint8)
    outs = []
    for fill in (0xFF, 0x00):
        b = runner.from_workload(wl, commit_any=True)
        if fp8:
            f = runner.quantize_embedding_fp8(b.E, V, d)
            ws = runner.fp8_workspace(n, V, d)
            ws.fill_(fill)
            runner.vocab_pass_fp8(b, f, ws, 4)
        else:
            b.workspace.fill_(fill)
            runner.vocab_pass(b, 4)
        torch.cuda.synchronize()
        outs.append(b)
    for k in ("lse", "entropy", "argmax_tok", "gumbel_tok", "selfcond"):
        x, y = getattr(outs[0], k).cpu().numpy(), getattr(outs[1], k).cpu().numpy()
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), k


def test_poisoned_selfcond_input_workspace():
    """The self-conditioning consumer's workspace poisoned the same way: identical bits."""
    from denoise_step_sampler_amd import runner
    n, V, D, F = 2, 1500, 256, 512
    E = synth.make_embedding(V, D, seed=3)
    pre, Wg, Wu, Wd = synth.make_ffw_weights(D, F, seed=3)
    W = runner.ffw_weights(pre, Wg, Wu, Wd)
    sc_rows, toks = synth.make_selfcond_rows(E, n * C, seed=3)
    wl = synth.workload("lite", V=V, d=D, n_canvas=n, seed=3, E=E)
    b = runner.from_workload(wl, commit_any=False)
    b.selfcond.copy_(torch.as_tensor(sc_rows))
    b.next_tokens.copy_(torch.as_tensor(toks))
    outs = []
    for fill in (0xFF, 0x00):
        ws = runner.ffw_workspace(n, D, F)
        ws.fill_(fill)
        out = torch.empty(n * C * D, dtype=torch.int16, device="cuda")
        runner.selfcond_input(b, W, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_split_invariance_canvas_alone_and_in_a_batch():
    """Five canvases in one call (rounds of 4 + 1, mixed lane counts, a commit canvas) against
    each non-commit canvas in a call of its own: the argmax tokens are equal except at the
    oracle's near-ties, lse and entropy agree to 1e-5 relative and the self-conditioning rows
    to 2e-5 (the merge order of the vocabulary partials differs, nothing else).  The Gumbel draw is
    not compared: its noise is keyed on the row within the call."""
    from denoise_step_sampler_amd import runner
    n, V, d = 5, 7000, 256
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=14)
    wl.commit = np.array([0, 0, 1, 0, 0], np.uint8)
    wl.temperature = np.linspace(0.6, 1.4, n).astype(np.float32)
    big = runner.from_workload(wl, commit_any=True)
    runner.vocab_pass(big, 9)
    torch.cuda.synchronize()
    E64 = ovp.widen_bf16(wl.E)
    for c in (0, 1, 3, 4):
        one = synth.workload("lite", V=V, d=d, n_canvas=1, seed=14, E=wl.E)
        one.h = wl.h[c * C:(c + 1) * C].copy()
        one.temperature = wl.temperature[c:c + 1].copy()
        one.step = wl.step[c:c + 1].copy()
        small = runner.from_workload(one, E=big.E)
        runner.vocab_pass(small, 9)
        torch.cuda.synchronize()
        rows = slice(c * C, (c + 1) * C)
        a1, a5 = small.argmax_tok.cpu().numpy(), big.argmax_tok.cpu().numpy()[rows]
        if not np.array_equal(a1, a5):
            ref = ovp.vocab_pass_rows(E64, one.h, np.arange(C), np.repeat(one.temperature, C),
                                      np.zeros(C, bool), 9, np.repeat(one.step, C),
                                      want_sc=False)
            assert np.all(ref.mu_argmax[a1 != a5] < 1e-4), c
        for k, tol in (("lse", 1e-5), ("entropy", 1e-5)):
            x = getattr(small, k).cpu().numpy().astype(np.float64)
            y = getattr(big, k).cpu().numpy()[rows].astype(np.float64)
            assert np.all(np.abs(x - y) <= tol * np.abs(y) + 1e-7), (c, k)
        x = small.selfcond.cpu().numpy().astype(np.float64)
        y = big.selfcond.cpu().numpy()[rows].astype(np.float64)
        rel = np.linalg.norm(x - y, axis=1) / np.linalg.norm(y, axis=1)
        assert rel.max() <= 2e-5, (c, rel.max())
        _say(f"    canvas {c}: max selfcond rel diff {rel.max():.2e}")
