"""The full denoise loop (8 canvases, signal 0.5 + 0.25 k kept only where the previous step
accepted) through the C ABI: every step's vocabulary-pass outputs and accept/renoise results
are checked against the oracle run on the same hidden states and the same incoming sampler
state, at the bars of the hot-path contract (margin-exempt decisions counted)."""
import sys

import numpy as np
import pytest

from denoise_step_sampler_amd import synth
from oracle import sampler as osm
from oracle import vocab_pass as ovp
from parity import MARGIN, VocabInputs, compare_sampler, compare_vocab

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


@pytest.mark.parametrize("schedule,softcap", [(None, None), ((0.8, 0.4), 30.0)])
def test_full_loop_reduced_every_step(schedule, softcap):
    """Per-canvas temperatures, or the linear anneal from 0.8 toward 0.4 over the loop's steps
    with the logits soft-capped at 30."""
    from denoise_step_sampler_amd import runner
    wl = synth.workload("full_loop", V=4096, d=256, seed=2)
    E64 = ovp.widen_bf16(wl.E)
    seed = 31
    reports = []

    def check(k, b, canv, state_in):
        prev_in, cnt_in = state_in
        n = canv.size
        rows = (canv[:, None] * C + np.arange(C)[None, :]).reshape(-1)
        h_bits = synth.loop_hidden(wl, k, check.acc_prev)[rows]
        step = np.full(n, k, np.int32)
        if schedule is None:
            T = np.repeat(wl.temperature[canv], C)
        else:
            T = np.full(n * C, ovp.temperature_schedule(k, 10, *schedule))
        ref = ovp.vocab_pass_rows(E64, h_bits, np.arange(n * C), T, np.zeros(n * C, bool),
                                  seed, np.repeat(step, C), want_sc=False, softcap=softcap)
        out = {"lse": b.lse.cpu().numpy(), "entropy": b.entropy.cpu().numpy(),
               "argmax": b.argmax_tok.cpu().numpy(), "gumbel": b.gumbel_tok.cpu().numpy()}
        rep = compare_vocab(out, ref, np.zeros(n * C, bool),
                            inputs=VocabInputs(E64, h_bits, T, np.repeat(step, C), seed, softcap))
        # the sampler on the oracle's fp64 entropies and tokens (argmax: the GPU's, equal to
        # the oracle's except at margin-exempt rows, so that the stability state is comparable)
        sref = osm.accept_renoise(ref.entropy, out["argmax"], ref.gumbel, None, n, C, wl.V,
                                  wl.budget, wl.confidence, wl.stability, seed, step,
                                  prev_in, cnt_in)
        acc = b.accept_mask.cpu().numpy()
        ex = sref.mu_accept < MARGIN
        assert not ((acc != sref.accept) & ~ex).any(), f"step {k}: accept mismatch"
        nxt = b.next_tokens.cpu().numpy()
        same = (acc == sref.accept) & (ref.mu_gumbel >= MARGIN)
        assert np.array_equal(nxt[same], sref.next_tokens[same]), f"step {k}: token mismatch"
        assert np.array_equal(b.prev_argmax.cpu().numpy(), sref.prev_argmax)
        assert np.array_equal(b.stable_count.cpu().numpy(), sref.stable_count)
        conv = b.converged.cpu().numpy()
        assert not ((conv != sref.converged) & (sref.mu_conv >= MARGIN)).any()
        rep.update(step=k, accepted=int(acc.sum()), accept_exempt=int(ex.sum()))
        reports.append(rep)
        a = np.zeros(wl.R, bool) if check.acc_prev is None else check.acc_prev.copy()
        a[rows] = acc.astype(bool)
        check.acc_prev = a

    check.acc_prev = None
    res = runner.run_loop(wl, seed, max_steps=10, on_step=check, schedule=schedule,
                          softcap=softcap)
    for r in reports:
        _say("   ", r)
    assert res.steps_run == 10 and len(reports) == 10
    if schedule is not None:
        return
    # near-maximal entropies: one accepted position per canvas and step, nothing converges
    assert all(r["accepted"] == 8 for r in reports)
    assert np.all(res.steps_to_converge == -1)
    assert res.positions == 10 * 8 * C


def _oracle_loop(wl, seed, max_steps):
    """The loop in the oracle alone: every step's pass on the active canvases, accept/renoise
    on its fp64 outputs, canvases leaving the batch once converged.  Returns the step after
    which each canvas converged (-1: never) and the smallest decision margin met."""
    E64 = ovp.widen_bf16(wl.E)
    n, V = wl.n_canvas, wl.V
    active = np.arange(n)
    prev = np.full(n * C, -1)
    cnt = np.zeros(n, np.int64)
    acc_prev, stc, mu = None, np.full(n, -1), np.inf
    for k in range(max_steps):
        if not active.size:
            break
        rows = (active[:, None] * C + np.arange(C)[None, :]).reshape(-1)
        na = active.size
        h = synth.loop_hidden(wl, k, acc_prev)[rows]
        ref = ovp.vocab_pass_rows(E64, h, np.arange(na * C), np.repeat(wl.temperature[active], C),
                                  np.zeros(na * C, bool), seed, np.full(na * C, k), want_sc=False)
        s = osm.accept_renoise(ref.entropy, ref.argmax, ref.gumbel, None, na, C, V, wl.budget,
                               wl.confidence, wl.stability, seed, np.full(na, k), prev[rows],
                               cnt[active])
        mu = min(mu, ref.mu_argmax.min(), s.mu_conv.min())
        a = np.zeros(n * C, bool) if acc_prev is None else acc_prev.copy()
        a[rows] = s.accept.astype(bool)
        acc_prev = a
        prev[rows] = s.prev_argmax
        cnt[active] = s.stable_count
        stc[active[s.converged == 1]] = k
        active = active[s.converged == 0]
    return stc, mu


def test_converging_loop_compacts_the_batch():
    """A loop whose canvases converge at different steps: every position accepted (budget
    1e6, so every position keeps its signal), the signal growing as 3 + 2 k and per-canvas
    temperatures 0.5 .. 1.2.  In the oracle the canvases converge after steps
    5, 4, 5, 5, 6, 7, 7, 8, so the batch shrinks 8 -> 7 -> 4 -> 3 -> 1 and the renoise and
    Gumbel counters follow the compacted rows.  Every step's pass (statistics, tokens and
    the self-conditioning rows) and accept/renoise state are checked against the oracle on
    the same compacted batch, and the steps to convergence must equal the oracle's."""
    from denoise_step_sampler_amd import runner
    wl = synth.workload("full_loop", V=4096, d=256, seed=2)
    wl.extra["signal"] = (3.0, 2.0)
    wl.budget = 1e6
    wl.temperature = np.linspace(0.5, 1.2, 8).astype(np.float32)
    E64 = ovp.widen_bf16(wl.E)
    seed = 31
    want, mu = _oracle_loop(wl, seed, 12)
    assert mu >= MARGIN, "pick a loop without near-tie decisions"
    assert list(want) == [5, 4, 5, 5, 6, 7, 7, 8]
    sizes = []

    def check(k, b, canv, state_in):
        prev_in, cnt_in = state_in
        n = canv.size
        sizes.append(n)
        rows = (canv[:, None] * C + np.arange(C)[None, :]).reshape(-1)
        h_bits = synth.loop_hidden(wl, k, check.acc_prev)[rows]
        T = np.repeat(wl.temperature[canv], C)
        st = np.full(n * C, k)
        ref = ovp.vocab_pass_rows(E64, h_bits, np.arange(n * C), T, np.zeros(n * C, bool), seed,
                                  st)
        out = {"lse": b.lse.cpu().numpy(), "entropy": b.entropy.cpu().numpy(),
               "argmax": b.argmax_tok.cpu().numpy(), "gumbel": b.gumbel_tok.cpu().numpy(),
               "sc": b.selfcond.cpu().numpy()}
        rep = compare_vocab(out, ref, np.zeros(n * C, bool),
                            inputs=VocabInputs(E64, h_bits, T, st, seed))
        sref = osm.accept_renoise(ref.entropy, ref.argmax, ref.gumbel, None, n, C, wl.V,
                                  wl.budget, wl.confidence, wl.stability, seed, np.full(n, k),
                                  prev_in, cnt_in)
        got = {"next_tokens": b.next_tokens.cpu().numpy(), "accept": b.accept_mask.cpu().numpy(),
               "converged": b.converged.cpu().numpy(),
               "mean_entropy": b.mean_entropy.cpu().numpy(),
               "prev_argmax": b.prev_argmax.cpu().numpy(),
               "stable_count": b.stable_count.cpu().numpy()}
        rep.update(compare_sampler(got, sref, None, C, H=ref.entropy, budget=wl.budget))
        _say(f"    step {k}: {n} canvases", rep)
        a = np.zeros(wl.R, bool) if check.acc_prev is None else check.acc_prev.copy()
        a[rows] = got["accept"].astype(bool)
        check.acc_prev = a

    check.acc_prev = None
    res = runner.run_loop(wl, seed, max_steps=12, on_step=check)
    assert list(res.steps_to_converge) == list(want)
    assert sizes == [8, 8, 8, 8, 8, 7, 4, 3, 1]
    assert res.positions == sum(sizes) * C


def test_full_loop_full_shape_two_steps():
    """The full denoise loop at its real shape (8 canvases x 256, V = 262144, d = 2816, the
    self-conditioning expectation on): two steps.  Sampled rows of every canvas (statistics,
    tokens, self-conditioning rows) against the oracle, and every accept/renoise output and
    state against the oracle's sampler on the pass's own entropies and tokens."""
    from denoise_step_sampler_amd import runner
    _say("[full_loop] generating V=262144 d=2816 embedding")
    wl = synth.workload("full_loop")
    E64 = ovp.widen_bf16(wl.E)
    seed = 19
    rng = np.random.default_rng(7)
    reports = []

    def check(k, b, canv, state_in):
        prev_in, cnt_in = state_in
        n = canv.size
        rows = (canv[:, None] * C + np.arange(C)[None, :]).reshape(-1)
        h_bits = synth.loop_hidden(wl, k, check.acc_prev)[rows]
        T = np.repeat(wl.temperature[canv], C)
        st = np.full(n * C, k)
        pick = np.sort(np.concatenate([c * C + rng.choice(C, 2, replace=False) for c in range(n)]))
        ref = ovp.vocab_pass_rows(E64, h_bits, pick, T, np.zeros(n * C, bool), seed, st)
        out = {"lse": b.lse.cpu().numpy()[pick], "entropy": b.entropy.cpu().numpy()[pick],
               "argmax": b.argmax_tok.cpu().numpy()[pick],
               "gumbel": b.gumbel_tok.cpu().numpy()[pick], "sc": b.selfcond.cpu().numpy()[pick]}
        rep = compare_vocab(out, ref, np.zeros(n * C, bool),
                            inputs=VocabInputs(E64, h_bits, T, st, seed))
        H = b.entropy.cpu().numpy().astype(np.float64)
        am, gm = b.argmax_tok.cpu().numpy(), b.gumbel_tok.cpu().numpy()
        sref = osm.accept_renoise(H, am, gm, None, n, C, wl.V, wl.budget, wl.confidence,
                                  wl.stability, seed, np.full(n, k), prev_in, cnt_in)
        got = {"next_tokens": b.next_tokens.cpu().numpy(), "accept": b.accept_mask.cpu().numpy(),
               "converged": b.converged.cpu().numpy(),
               "mean_entropy": b.mean_entropy.cpu().numpy(),
               "prev_argmax": b.prev_argmax.cpu().numpy(),
               "stable_count": b.stable_count.cpu().numpy()}
        rep.update(compare_sampler(got, sref, None, C, H=H, budget=wl.budget))
        rep.update(step=k, accepted=int(got["accept"].sum()))
        _say("   ", rep)
        reports.append(rep)
        a = np.zeros(wl.R, bool) if check.acc_prev is None else check.acc_prev.copy()
        a[rows] = got["accept"].astype(bool)
        check.acc_prev = a

    check.acc_prev = None
    res = runner.run_loop(wl, seed, max_steps=2, on_step=check)
    assert res.steps_run == 2 and len(reports) == 2
    # near-maximal entropies: one accepted position per canvas and step
    assert all(r["accepted"] == 8 for r in reports)
