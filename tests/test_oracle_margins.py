"""Pins of the oracle's decision margins, the quantities the parity tests use to exempt
near-ties from the bit-exact comparisons.

A margin is the distance from a decision to the nearest input that changes it.  The pins
check that meaning directly: they move the winner's key by slightly less and slightly more
than the reported margin (through the embedding row of the winning token, so the oracle
recomputes everything from its inputs) and require the decision to hold, then to change.
Hand-worked cases give nonzero values for every margin, and mutation checks plant plausible
mistakes in a copy of the oracle (a margin taken on the untempered or noise-free logits, a
dropped term) and require the pins to catch each of them.
"""
import math
import types

import numpy as np
import pytest

from denoise_step_sampler_amd import synth
from oracle import sampler as osm
from oracle import vocab_pass as ovp


# --- the top-2 gap itself ------------------------------------------------------------------

@pytest.mark.parametrize("x,want", [([1.0, 5.0, 3.0, 4.5], 0.5), ([-2.0, -7.0], 5.0),
                                    ([1.0, 5.0, 3.0, 5.0], 0.0), ([3.0], math.inf),
                                    ([0.25, -1.0, 0.25 - 2.0 ** -20], 2.0 ** -20),
                                    ([10.0, 9.0, 9.0, 9.0], 1.0)])
def test_top2_gap_hand_worked(x, want):
    """Largest minus the largest of the other indices (a tied maximum gives 0)."""
    assert ovp._top2_margin(np.array(x)) == want


# --- margins of the vocabulary pass as distances to the decision boundary -------------------

def _case(V=40, d=16, R=6, seed=3, scale=1.5):
    rng = np.random.default_rng(seed)
    E = rng.standard_normal((V, d)) / math.sqrt(d)
    h = synth.round_to_bf16((scale * rng.standard_normal((R, d))).astype(np.float32))
    return E, h


def _one(vp, E64, h, r, T, Td=None, seed=5, step=2, softcap=None):
    R = h.shape[0]
    return vp.vocab_pass_rows(E64, h, [r], np.full(R, T), np.zeros(R, bool), seed,
                              np.full(R, step), want_sc=False, softcap=softcap,
                              draw_temperature_row=None if Td is None else np.full(R, Td))


def _lowered(E64, h, r, v, delta):
    """E with row v moved so that S_v of row r drops by exactly delta (up to fp64 rounding)."""
    hb = ovp.widen_bf16(h[r])
    E2 = E64.copy()
    E2[v] = E2[v] - delta * hb / float(hb @ hb)
    return E2


def boundary_violations(vp, T=0.7, Td=None, eps=1e-7):
    """Rows whose argmax or Gumbel margin does not match the decision boundary: lowering the
    winner's key by (1 - eps) * margin must keep the decision, by (1 + eps) * margin must
    change it.  Returns a list of (kind, row) failures."""
    E64, h = _case()
    bad = []
    for r in range(h.shape[0]):
        base = _one(vp, E64, h, r, T, Td)
        am, ma = int(base.argmax[0]), float(base.mu_argmax[0])
        gt, mg = int(base.gumbel[0]), float(base.mu_gumbel[0])
        assert ma > 0 and mg > 0, "pick a case without ties"
        # argmax: S itself moves by delta
        lo = _one(vp, _lowered(E64, h, r, am, (1 - eps) * ma), h, r, T, Td)
        hi = _one(vp, _lowered(E64, h, r, am, (1 + eps) * ma), h, r, T, Td)
        if int(lo.argmax[0]) != am or int(hi.argmax[0]) == am:
            bad.append(("argmax", r))
        # Gumbel: the key y = S / T_draw + g moves by delta / T_draw
        tdraw = T if Td is None else Td
        lo = _one(vp, _lowered(E64, h, r, gt, (1 - eps) * mg * tdraw), h, r, T, Td)
        hi = _one(vp, _lowered(E64, h, r, gt, (1 + eps) * mg * tdraw), h, r, T, Td)
        if int(lo.gumbel[0]) != gt or int(hi.gumbel[0]) == gt:
            bad.append(("gumbel", r))
    return bad


@pytest.mark.parametrize("T,Td", [(0.7, None), (1.0, 0.35), (2.5, None)])
def test_margins_are_distances_to_the_decision(T, Td):
    assert boundary_violations(ovp, T, Td) == []


def test_gumbel_margin_hand_worked():
    """V = 2, T = 1, logits 0 and 50: the keys are g_0 and 50 + g_1, so the margin is
    50 + g_1 - g_0 with the two noise values of the row; it is not 50 (the gap of the
    noise-free logits), and the token is 1."""
    from oracle import philox
    E64 = np.array([[0.0], [1.0]])
    h = synth.round_to_bf16(np.array([[50.0]], np.float32))
    r = _one(ovp, E64, h, 0, 1.0, seed=7, step=3)
    g = philox.gumbel_noise(0, 2, 7, 3)
    assert int(r.gumbel[0]) == 1 and int(r.argmax[0]) == 1
    assert r.mu_argmax[0] == 50.0
    assert abs(r.mu_gumbel[0] - (50.0 + g[1] - g[0])) < 1e-12
    assert abs(r.mu_gumbel[0] - 50.0) > 1e-3


def test_argmax_margin_hand_worked():
    """d = 2, rows of E (1, 0), (0, 1), (1, 1), (-1, 0), h = (2, 0.5): S = (2, 0.5, 2.5, -2),
    argmax 2 with margin 0.5."""
    E64 = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-1.0, 0.0]])
    h = synth.round_to_bf16(np.array([[2.0, 0.5]], np.float32))
    r = _one(ovp, E64, h, 0, 1.0)
    assert int(r.argmax[0]) == 2 and r.mu_argmax[0] == 0.5


# --- margins of the samplers --------------------------------------------------------------

def test_accept_margins_hand_worked():
    """Budget 4, H = (0.5, 3.0, 0.2, 5.0, 1.0): order 2, 0, 4, 1, 3 with exclusive prefixes
    0, 0.2, 0.7, 1.7, 4.7; positions 0, 1, 2, 4 accepted, 3 rejected.  Margins: distance of the
    position's prefix to the budget, or to the nearest entropy with the other decision:
    (min(3.8, 4.5), min(2.3, 2.0), min(4.0, 4.8), min(0.7, 2.0), min(3.3, 4.0))."""
    H = np.array([0.5, 3.0, 0.2, 5.0, 1.0])
    C = 5
    r = osm.accept_renoise(H, np.zeros(C, np.int64), np.arange(C), None, 1, C, 100, 4.0, 0.5, 1,
                           0, 0, np.full(C, -1), np.zeros(1))
    assert list(r.accept) == [1, 1, 1, 0, 1]
    assert np.allclose(r.mu_accept, [3.8, 2.0, 4.0, 0.7, 3.3], atol=1e-12, rtol=0)
    # mean H = 1.94: convergence margin against a threshold of 0.5 is 1.44
    assert abs(r.mu_conv[0] - 1.44) < 1e-12


def test_accept_margin_all_accepted():
    """With every position accepted there is no opposite decision: the margin is the budget
    distance alone (budget 10, H = (1, 2, 3): prefixes 0, 1, 3 -> margins 10, 9, 7)."""
    H = np.array([1.0, 2.0, 3.0])
    r = osm.accept_renoise(H, np.zeros(3, np.int64), np.arange(3), None, 1, 3, 100, 10.0, 0.5, 1,
                           0, 0, np.full(3, -1), np.zeros(1))
    assert list(r.accept) == [1, 1, 1]
    assert np.allclose(r.mu_accept, [10.0, 9.0, 7.0], atol=1e-12, rtol=0)


def _lite(conf, prev_conf, am, prev_am, H, threshold=0.25):
    C = len(conf)
    return osm.lite_step(np.asarray(H, float), np.asarray(am), np.arange(C), np.asarray(conf, float),
                         1, C, 50, threshold, 2, 0, 0, np.zeros(C, np.int64), np.asarray(prev_am),
                         np.asarray(prev_conf, float), np.zeros(C, np.uint8), np.zeros(1))


def test_lite_commit_margin_hand_worked():
    """Changed argmax: the commit decision is conf >= prev_conf, margin |ln conf - ln prev_conf|
    (ln 1.2 = 0.18232 and ln 1.5 = 0.40547); unchanged argmax commits whatever the confidences
    (margin infinite)."""
    r = _lite([0.30, 0.20, 0.9], [0.25, 0.30, 0.1], [4, 4, 7], [3, 5, 7], [0.1, 0.2, 0.3])
    assert list(r.committed) == [1, 0, 1]
    assert np.allclose(r.mu_commit[:2], [0.1823215567939546, 0.4054651081081644], atol=1e-14,
                       rtol=0)
    assert r.mu_commit[2] == np.inf


def test_lite_stop_margin_hand_worked():
    """Mean entropy 0.2 against a threshold of 0.25: margin 0.05 (and below the threshold, so
    the stop counter advances)."""
    r = _lite([0.5, 0.5], [1.0, 1.0], [1, 2], [1, 2], [0.1, 0.3])
    assert abs(r.mu_stop[0] - 0.05) < 1e-15
    assert r.stable_count[0] == 1


def commit_margin_violations(sampler, eps=1e-7):
    """The Lite commit margin as a boundary: moving ln prev_conf toward ln conf by (1 + eps)
    margin flips the decision of a changed-argmax position, by (1 - eps) margin does not."""
    rng = np.random.default_rng(4)
    C = 16
    conf = rng.uniform(0.1, 0.9, C)
    prev = rng.uniform(0.1, 0.9, C)
    am, pam = np.arange(C), np.arange(C) + 1
    H = rng.uniform(0, 1, C)
    base = sampler.lite_step(H, am, am, conf, 1, C, 50, 0.3, 2, 0, 0, np.zeros(C, np.int64), pam,
                             prev, np.zeros(C, np.uint8), np.zeros(1))
    bad = []
    for i in range(C):
        m = base.mu_commit[i]
        sgn = 1.0 if base.committed[i] else -1.0   # committed: prev <= conf; move prev up
        for f, flips in ((1 - eps, False), (1 + eps, True)):
            p2 = prev.copy()
            p2[i] = prev[i] * np.exp(sgn * f * m)
            r = sampler.lite_step(H, am, am, conf, 1, C, 50, 0.3, 2, 0, 0, np.zeros(C, np.int64),
                                  pam, p2, np.zeros(C, np.uint8), np.zeros(1))
            if (r.committed[i] != base.committed[i]) != flips:
                bad.append(i)
    return bad


def test_lite_commit_margin_is_the_boundary():
    assert commit_margin_violations(osm) == []


# --- mutation checks: the pins above catch planted margin mistakes ------------------------

def _mutant(module, old: str, new: str):
    """A copy of an oracle module with one source fragment replaced (the planted mistake)."""
    import inspect
    src = inspect.getsource(module)
    assert old in src, old
    m = types.ModuleType(module.__name__ + "_mutant")
    m.__dict__["__package__"] = "oracle"
    m.__dict__["__spec__"] = None
    import sys
    sys.modules[m.__name__] = m   # dataclasses look their module up by name
    exec(compile(src.replace(old, new), module.__file__ + ":mutant", "exec"), m.__dict__)
    return m


@pytest.mark.parametrize("old,new,T,Td,label", [
    ("mu_g[i] = _top2_margin(y)", "mu_g[i] = _top2_margin(z)", 0.7, None,
     "Gumbel margin on the noise-free logits"),
    ("mu_g[i] = _top2_margin(y)", "mu_g[i] = _top2_margin(z + g)", 1.0, 0.35,
     "Gumbel margin at the statistics' temperature instead of the draw's"),
    ("mu_a[i] = _top2_margin(s)", "mu_a[i] = _top2_margin(s / float(temperature_row[r]))", 2.5, None,
     "argmax margin on the tempered logits"),
    ("rest = np.delete(x, i)", "rest = x", 0.7, None, "runner-up taken over every index (margin 0)"),
    ("return float(best - rest.max())", "return float(best - rest.min())", 0.7, None,
     "margin to the smallest instead of the runner-up"),
])
def test_vocab_margin_mutations_are_caught(old, new, T, Td, label):
    m = _mutant(ovp, old, new)
    try:
        bad = boundary_violations(m, T, Td)
    except AssertionError:   # the planted mistake makes every margin 0
        bad = ["zero margins"]
    assert bad, f"planted mistake not caught: {label}"


@pytest.mark.parametrize("old,new,label", [
    ("np.abs(np.log(cf[rows]) - np.log(pc[rows]))", "np.abs(np.log(cf[rows]))",
     "commit margin drops prev_conf"),
    ("np.abs(np.log(cf[rows]) - np.log(pc[rows]))", "2 * np.abs(np.log(cf[rows]) - np.log(pc[rows]))",
     "commit margin doubled"),
    ("np.abs(np.log(cf[rows]) - np.log(pc[rows]))", "np.abs(cf[rows] - pc[rows])",
     "commit margin on the probabilities instead of their logarithms"),
])
def test_lite_margin_mutations_are_caught(old, new, label):
    m = _mutant(osm, old, new)
    assert commit_margin_violations(m), f"planted mistake not caught: {label}"


def test_accept_margin_mutations_are_caught():
    """Dropping either term of the accept margin changes a hand-worked value."""
    H = np.array([0.5, 3.0, 0.2, 5.0, 1.0])
    for old, new in (("m = min(m, float(np.min(np.abs(other - h[i]))))", "m = m"),
                     ("m = abs(prefix[i] - budget)", "m = np.inf")):
        mm = _mutant(osm, old, new)
        r = mm.accept_renoise(H, np.zeros(5, np.int64), np.arange(5), None, 1, 5, 100, 4.0, 0.5, 1,
                              0, 0, np.full(5, -1), np.zeros(1))
        assert not np.allclose(r.mu_accept, [3.8, 2.0, 4.0, 0.7, 3.3], atol=1e-12, rtol=0), old
