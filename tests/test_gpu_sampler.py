"""Parity of dg_accept_renoise and dg_q_sample (through the C ABI) with the oracle, and of one
whole denoising step (vocabulary pass + accept/renoise) on the tiny workload."""
import math
import os
import sys

import numpy as np
import pytest

from denoise_step_sampler_amd import synth
from oracle import q_sample as oqs
from oracle import sampler as osm
from oracle import vocab_pass as ovp
from parity import compare_sampler

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
C = 256
HERE = os.path.dirname(os.path.abspath(__file__))


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


def _dev(x, dt):
    return torch.as_tensor(np.ascontiguousarray(x)).to(dtype=dt, device="cuda")


def _gpu_accept(H, am, gm, commit, n, V, budget, conf, thr, seed, step, prev, cnt):
    from denoise_step_sampler_amd import binding as B
    R = n * C
    t = dict(H=_dev(H.astype(np.float32), torch.float32), am=_dev(am, torch.int32),
             gm=_dev(gm, torch.int32),
             commit=None if commit is None else _dev(commit, torch.uint8),
             step=_dev(step, torch.int32), prev=_dev(prev, torch.int32),
             cnt=_dev(cnt, torch.int32))
    nxt = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    acc = torch.full((R,), 7, dtype=torch.uint8, device="cuda")
    conv = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    mean = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    B.dg_accept_renoise(t["H"], t["am"], t["gm"], t["commit"], n, C, V, budget, conf, thr, seed,
                        t["step"], t["prev"], t["cnt"], nxt, acc, conv, mean)
    torch.cuda.synchronize()
    return {"next_tokens": nxt.cpu().numpy(), "accept": acc.cpu().numpy(),
            "converged": conv.cpu().numpy(), "mean_entropy": mean.cpu().numpy(),
            "prev_argmax": t["prev"].cpu().numpy(), "stable_count": t["cnt"].cpu().numpy()}


def _both(H, am, gm, commit, n, V, budget, conf, thr, seed, step, prev, cnt, label="",
          max_exempt=None):
    _say(f"[accept_renoise] {label} n={n} V={V} budget={budget}")
    H32 = np.asarray(H, np.float32)
    got = _gpu_accept(H32, am, gm, commit, n, V, budget, conf, thr, seed, step, prev, cnt)
    b32 = float(np.float32(budget))
    ref = osm.accept_renoise(H32.astype(np.float64), am, gm, commit, n, C, V, b32,
                             float(np.float32(conf)), thr, seed, step, prev, cnt)
    rep = compare_sampler(got, ref, commit, C, H=H32.astype(np.float64), budget=b32,
                          max_exempt=max_exempt)
    _say("   ", rep)
    return got, ref


def test_random_entropies_mixed_commit():
    rng = np.random.default_rng(0)
    n, V = 6, 50257
    H = rng.uniform(0, 0.2, size=n * C)
    H[C:2 * C] = rng.exponential(0.05, C)
    H[2 * C:3 * C] = 11.0 + rng.uniform(0, 0.5, C)       # near-maximal entropies
    H[3 * C:3 * C + 40] = 0.0                              # ties at zero
    am = rng.integers(0, V, n * C)
    gm = rng.integers(0, V, n * C)
    commit = np.array([0, 0, 0, 1, 0, 1], np.uint8)
    prev = np.where(rng.random(n * C) < 0.5, am, -1)
    prev[4 * C:5 * C] = am[4 * C:5 * C]                    # canvas 4 stable and confident
    H[4 * C:5 * C] = rng.uniform(0, 0.05, C)
    cnt = np.array([0, 3, 1, 2, 5, 9])
    step = np.arange(n) * 7
    got, ref = _both(H, am, gm, commit, n, V, 4.0, 0.1, 2, 42, step, prev, cnt, "random")
    assert got["accept"][2 * C:3 * C].sum() == 1
    assert got["converged"][4] == 1 and got["stable_count"][4] == 6


def test_equal_entropies_order_by_position():
    """Every entropy equal: each position has an equal entropy with the other decision, so all
    are exempt by construction; the stable order still fixes which two are accepted."""
    n, V = 1, 1000
    H = np.full(C, math.log(16), dtype=np.float64)
    am = np.arange(C)
    got, _ = _both(H, am, am + 1, None, n, V, 4.0, 0.1, 1, 5, np.zeros(1), np.full(C, -1),
                   np.zeros(1), "ties", max_exempt=C)
    assert list(np.nonzero(got["accept"])[0]) == [0, 1]


def _golden():
    out = []
    with open(os.path.join(HERE, "golden", "accept_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            b, H, a = line.split("|")
            out.append((float(b), [float(x) for x in H.split()], [int(x) for x in a.split()]))
    return out


@pytest.mark.parametrize("case", range(5))
def test_hand_worked_cases_embedded(case):
    """The hand-worked cases in the first positions of a canvas; the other positions carry a
    large entropy, so they rank last and are renoised without changing the worked decisions."""
    budget, Hc, expect = _golden()[case]
    H = np.full(C, 100.0)
    H[:len(Hc)] = Hc
    am = np.arange(C)
    # the worked cases include equal entropies and a prefix exactly at the budget (exempt by
    # construction); their decisions are checked against the worked values below
    got, _ = _both(H, am, am + 3, None, 1, 4096, budget, 0.1, 1, 0, np.zeros(1),
                   np.full(C, -1), np.zeros(1), f"golden{case}", max_exempt=C)
    assert list(got["accept"][:len(Hc)]) == expect
    assert got["accept"][len(Hc):].sum() == 0


def test_stability_counter_over_steps():
    n, V = 2, 300
    rng = np.random.default_rng(5)
    H = np.full(n * C, 0.001)
    am = rng.integers(0, V, n * C)
    prev = np.full(n * C, -1)
    cnt = np.zeros(n)
    for k in range(4):
        got, ref = _both(H, am, am, None, n, V, 4.0, 0.1, 2, 3, np.full(n, k), prev, cnt,
                         f"step{k}")
        prev, cnt = got["prev_argmax"], got["stable_count"]
        assert list(cnt) == [k, k]
        assert list(got["converged"]) == ([1, 1] if k >= 2 else [0, 0])


def test_q_sample_matches_oracle():
    from denoise_step_sampler_amd import binding as B
    wl = synth.qsample_workload(n_canvas=64, V=50257, seed=0)
    for kappa, V, label in ((wl.kappa, wl.V, "cosine"), (np.zeros(64, np.float32), wl.V, "k=0"),
                            (np.ones(64, np.float32), wl.V, "k=1"), (wl.kappa, 1, "V=1")):
        _say(f"[q_sample] {label}")
        x0 = wl.x0 if V > 1 else np.zeros_like(wl.x0)
        xt = torch.full((x0.size,), -7, dtype=torch.int32, device="cuda")
        B.dg_q_sample(_dev(x0, torch.int32), 64, C, V, _dev(kappa, torch.float32), 1234, xt)
        torch.cuda.synchronize()
        ref = oqs.q_sample(x0, 64, C, V, kappa, 1234)
        assert np.array_equal(xt.cpu().numpy(), ref)


def test_whole_step_tiny_workload():
    """Vocabulary pass + accept/renoise on the tiny workload against the oracle run end to end
    on its own fp64 outputs; positions whose accept or Gumbel decision margin is below 1e-4
    are exempt."""
    from denoise_step_sampler_amd import runner
    wl = synth.workload("tiny")
    b = runner.from_workload(wl)
    runner.denoise_step(b, wl.budget, wl.confidence, wl.stability, seed=0)
    torch.cuda.synchronize()
    ref_v = ovp.vocab_pass_rows(ovp.widen_bf16(wl.E), wl.h, np.arange(wl.R),
                                np.repeat(wl.temperature, C), np.zeros(wl.R, bool), 0,
                                np.repeat(wl.step, C))
    ref = osm.accept_renoise(ref_v.entropy, ref_v.argmax, ref_v.gumbel, None, 1, C, wl.V,
                             wl.budget, wl.confidence, wl.stability, 0, wl.step,
                             np.full(wl.R, -1), np.zeros(1))
    acc = b.accept_mask.cpu().numpy()
    ex = (ref.mu_accept < 1e-4)
    assert ex.sum() <= 2 and (ref_v.mu_gumbel < 1e-4).sum() <= 2   # near-ties are rare
    assert not ((acc != ref.accept) & ~ex).any()
    nxt = b.next_tokens.cpu().numpy()
    ok_g = ref_v.mu_gumbel >= 1e-4
    same = (acc == ref.accept) & ok_g
    assert np.array_equal(nxt[same], ref.next_tokens[same])
    _say("   accepted:", int(acc.sum()), "exempt:", int(ex.sum()))
    assert acc.sum() == 1


def test_step_captured_in_a_hip_graph():
    """The vocabulary pass and accept/renoise queue only kernels on the caller's stream (no
    allocation, memset or synchronisation), so a step can be captured in a HIP graph: three
    replays, with eager state resets between them, reproduce the eager step bit for bit."""
    from denoise_step_sampler_amd import runner
    wl = synth.workload("lite", V=5000, d=256, n_canvas=3, seed=2)
    wl.commit = np.array([0, 1, 0], np.uint8)
    b = runner.from_workload(wl)
    keys = ("lse", "entropy", "argmax_tok", "gumbel_tok", "selfcond", "next_tokens",
            "accept_mask", "converged", "prev_argmax", "stable_count", "mean_entropy")

    def reset():
        b.prev_argmax.fill_(-1)
        b.stable_count.zero_()

    def step():
        runner.denoise_step(b, wl.budget, wl.confidence, wl.stability, 5,
                            stream=torch.cuda.current_stream())

    reset()
    step()
    torch.cuda.synchronize()
    ref = {k: getattr(b, k).clone() for k in keys}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        reset()
        for k in ("lse", "entropy", "selfcond", "mean_entropy"):
            getattr(b, k).fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in keys:
            x, y = getattr(b, k).cpu().numpy(), ref[k].cpu().numpy()
            if x.dtype == np.float32:
                x, y = x.view(np.uint32), y.view(np.uint32)
            assert np.array_equal(x, y), k
