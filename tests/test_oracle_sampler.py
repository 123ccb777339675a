"""Pins of the accept/renoise/convergence oracle: hand-worked cases (golden file), scripted
stability sequences and the renoise stream."""
import math
import os

import numpy as np
import pytest

from oracle import philox, sampler

HERE = os.path.dirname(os.path.abspath(__file__))


def _cases():
    out = []
    with open(os.path.join(HERE, "golden", "accept_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            b, H, a = line.split("|")
            out.append((float(b), [float(x) for x in H.split()], [int(x) for x in a.split()]))
    return out


def _one_canvas(H, budget, C=None, gum=None, am=None, prev=None, cnt=0, conf=0.1, thr=1,
                step=0, seed=0, V=1000):
    C = C or len(H)
    gum = np.arange(C) + 500 if gum is None else gum
    am = np.arange(C) + 100 if am is None else am
    prev = np.full(C, -1) if prev is None else prev
    return sampler.accept_renoise(np.array(H), am, gum, np.zeros(1, np.uint8), 1, C, V,
                                  budget, conf, thr, seed, np.array([step]), prev,
                                  np.array([cnt]))


@pytest.mark.parametrize("case", range(5))
def test_hand_worked_acceptances(case):
    budget, H, expect = _cases()[case]
    r = _one_canvas(H, budget)
    assert list(r.accept) == expect
    gum = np.arange(len(H)) + 500
    ren = philox.renoise_tokens(np.arange(len(H)), 1000, 0, 0)
    assert np.array_equal(r.next_tokens, np.where(np.array(expect) == 1, gum, ren))


def test_at_least_one_accepted_and_budget_monotone():
    rng = np.random.default_rng(0)
    for _ in range(50):
        H = rng.uniform(0, 3, size=256)
        prev_count = 0
        for b in (0.0, 0.5, 1.0, 4.0, 20.0, 1e9):
            r = _one_canvas(H, b)
            n = int(r.accept.sum())
            assert n >= 1 and n >= prev_count
            prev_count = n
        assert n == 256
        # accepted set is a prefix of the entropy order
        r = _one_canvas(H, 4.0)
        order = np.lexsort((np.arange(256), H))
        acc = r.accept[order]
        k = int(acc.sum())
        assert np.all(acc[:k] == 1) and np.all(acc[k:] == 0)
        assert H[order[:k - 1]].sum() <= 4.0 < H[order[:k]].sum() or k == 256


def test_near_maximal_entropy_accepts_exactly_one():
    """Entropies near ln V (> budget) accept only the lowest-entropy position."""
    H = np.full(256, math.log(262144) - 0.8) + np.linspace(0, 0.01, 256)[::-1]
    r = _one_canvas(H, 4.0)
    assert r.accept.sum() == 1 and r.accept[255] == 1


def test_stability_counter_and_convergence_script():
    C = 4
    H = np.full(C, 0.01)
    am1 = np.array([1, 2, 3, 4])
    am2 = np.array([1, 2, 3, 5])
    prev = np.full(C, -1)
    cnt = 0
    # step 0: no previous canvas -> count 0, not converged
    r = _one_canvas(H, 4.0, am=am1, prev=prev, cnt=cnt, thr=2)
    assert r.stable_count[0] == 0 and r.converged[0] == 0
    assert np.array_equal(r.prev_argmax, am1)
    # step 1: same argmax -> 1 (threshold 2 not reached)
    r = _one_canvas(H, 4.0, am=am1, prev=r.prev_argmax, cnt=r.stable_count[0], thr=2)
    assert r.stable_count[0] == 1 and r.converged[0] == 0
    # step 2: same -> 2, mean H 0.01 < 0.1 -> converged
    r = _one_canvas(H, 4.0, am=am1, prev=r.prev_argmax, cnt=r.stable_count[0], thr=2)
    assert r.stable_count[0] == 2 and r.converged[0] == 1
    # step 3: one position changes -> reset
    r = _one_canvas(H, 4.0, am=am2, prev=r.prev_argmax, cnt=r.stable_count[0], thr=2)
    assert r.stable_count[0] == 0 and r.converged[0] == 0
    # stable but too uncertain (mean entropy not strictly below the threshold)
    r = _one_canvas(np.full(C, 0.1), 4.0, am=am2, prev=am2, cnt=5, thr=2, conf=0.1)
    assert r.stable_count[0] == 6 and r.converged[0] == 0
    assert r.mu_conv[0] == 0.0


def test_commit_canvas_resets_state():
    C = 3
    H = np.array([0.1, 0.2, 0.3, 5.0, 5.0, 5.0])
    am = np.array([7, 8, 9, 10, 11, 12])
    gum = np.array([1, 2, 3, 4, 5, 6])
    prev = np.array([7, 8, 9, 10, 11, 12])
    r = sampler.accept_renoise(H, am, gum, np.array([1, 0], np.uint8), 2, C, 100, 1.0, 0.5, 1,
                               0, np.array([0, 0]), prev, np.array([4, 4]))
    assert list(r.next_tokens[:3]) == [7, 8, 9] and list(r.accept[:3]) == [1, 1, 1]
    assert list(r.prev_argmax[:3]) == [-1, -1, -1] and r.stable_count[0] == 0
    assert r.converged[0] == 0 and math.isnan(r.mean_entropy[0])
    # canvas 1: stable, mean 5.0 not < 0.5
    assert r.stable_count[1] == 5 and r.converged[1] == 0
    assert r.accept[3:].sum() == 1


def test_renoise_stream_depends_on_row_step_seed():
    H = np.full(8, 9.0)
    a = _one_canvas(H, 1.0, step=0).next_tokens
    b = _one_canvas(H, 1.0, step=1).next_tokens
    c = _one_canvas(H, 1.0, step=0, seed=1).next_tokens
    assert not np.array_equal(a[1:], b[1:]) and not np.array_equal(a[1:], c[1:])
    assert np.all((a >= 0) & (a < 1000))


def test_accept_margins():
    r = _one_canvas([0.5, 3.0, 0.2, 5.0, 1.0], 4.0)
    # position 3 (rank 4, prefix 4.7): margin min(0.7, |5 - 3|, ...) = 0.7
    assert abs(r.mu_accept[3] - 0.7) < 1e-12
    r = _one_canvas([2.5, 2.0, 0.0], 2.0)
    assert r.mu_accept[0] == 0.0
