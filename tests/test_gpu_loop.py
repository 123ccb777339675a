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
from parity import MARGIN, compare_vocab

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
        rep = compare_vocab(out, ref, np.zeros(n * C, bool))
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
