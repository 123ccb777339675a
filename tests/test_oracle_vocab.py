"""Pins of the vocab-pass oracle against closed forms, identities between its outputs that
it does not use itself (derivatives of lse), and sampling statistics."""
import math

import mpmath
import numpy as np
import pytest
from scipy import stats

from denoise_step_sampler_amd import synth
from oracle import vocab_pass as vp


def _run(E_bits, h_bits, T=1.0, commit=False, seed=0, step=0, want_sc=True):
    R = h_bits.shape[0]
    return vp.vocab_pass_rows(vp.widen_bf16(E_bits), h_bits, np.arange(R),
                              np.full(R, T), np.full(R, commit), seed, np.full(R, step),
                              want_sc=want_sc)


def test_widen_bf16_exact():
    vals = np.array([1.0, -2.5, 3.140625, 0.0, 1e-3], dtype=np.float32)
    b = synth.round_to_bf16(vals)
    w = vp.widen_bf16(b)
    assert w[0] == 1.0 and w[1] == -2.5 and w[2] == 3.140625 and w[3] == 0.0
    assert abs(w[4] - 1e-3) < 1e-3 * 2 ** -8


@pytest.mark.parametrize("T", [0.4, 0.8, 1.0, 2.0])
def test_uniform_logits_closed_form(T):
    """h = 0 gives equal logits: lse = H = ln V at any temperature, sc = mean_v E_v, argmax 0
    (the uniform initial distribution of DiffusionGemma Explained, "Lazy Sampling")."""
    V, d = 1000, 64
    E = synth.make_embedding(V, d, seed=1)
    h = np.zeros((3, d), dtype=np.uint16)
    r = _run(E, h, T=T)
    assert np.allclose(r.lse, math.log(V), atol=1e-12, rtol=0)
    assert np.allclose(r.entropy, math.log(V), atol=1e-12, rtol=0)
    mean_e = synth.bf16_to_f32(E).astype(np.float64).mean(axis=0)
    assert np.allclose(r.sc, mean_e[None, :], atol=1e-14, rtol=1e-12)
    assert np.all(r.argmax == 0)
    assert np.all(r.mu_argmax == 0.0)


def test_peaked_logits():
    """h = 100 * E[t] concentrates the distribution on t: H ~ 0, sc ~ E[t], argmax = t,
    Gumbel sample = t."""
    V, d = 2048, 128
    E = synth.make_embedding(V, d, seed=2)
    t = np.array([5, 77, 2047])
    h = synth.round_to_bf16(100.0 * synth.bf16_to_f32(E[t]))
    r = _run(E, h)
    assert np.array_equal(r.argmax, t)
    assert np.array_equal(r.gumbel, t)
    assert np.all(r.entropy < 1e-6)
    assert np.allclose(r.sc, synth.bf16_to_f32(E[t]), atol=1e-6)


def _two_level(V, k, a, b):
    """E and h (d = 2) whose logits are a on tokens [0, k) and b on the rest."""
    E = np.zeros((V, 2), dtype=np.float32)
    E[:k, 0] = 1.0
    E[k:, 1] = 1.0
    h = np.array([[a, b]], dtype=np.float32)
    return synth.round_to_bf16(E), synth.round_to_bf16(h)


@pytest.mark.parametrize("V,k,a,b,T", [(64, 3, 2.0, -1.0, 1.0), (5000, 17, 6.5, 0.25, 0.8),
                                       (16, 1, 0.0, 0.0, 1.0), (300, 299, -3.0, 4.0, 0.4)])
def test_two_level_closed_form(V, k, a, b, T):
    Eb, hb = _two_level(V, k, a, b)
    r = _run(Eb, hb, T=T)
    Z = k * math.exp(a / T) + (V - k) * math.exp(b / T)
    pa, pb = math.exp(a / T) / Z, math.exp(b / T) / Z
    H = -(k * pa * math.log(pa) + (V - k) * pb * math.log(pb))
    assert abs(r.lse[0] - math.log(Z)) < 1e-12 * max(1, abs(math.log(Z)))
    assert abs(r.entropy[0] - H) < 1e-12
    assert np.allclose(r.sc[0], [k * pa, (V - k) * pb], atol=1e-14)
    assert r.argmax[0] == (0 if a >= b else k)


def test_entropy_is_legendre_identity_of_lse():
    """H = lse - beta * d lse / d beta with beta = 1/T: checked by finite differences of the
    oracle's own lse at neighbouring temperatures (H is not computed that way)."""
    wl = synth.workload("tiny", V=512, d=64)
    E, h = wl.E, wl.h[:8]
    T, eps = 0.9, 1e-5
    lo = _run(E, h, T=1.0 / (1.0 / T - eps), want_sc=False).lse
    hi = _run(E, h, T=1.0 / (1.0 / T + eps), want_sc=False).lse
    mid = _run(E, h, T=T, want_sc=False)
    dlse = (hi - lo) / (2 * eps)
    H_fd = mid.lse - dlse / T
    assert np.allclose(mid.entropy, H_fd, atol=1e-7)


def test_selfcond_is_temperature_times_gradient_of_lse():
    """sc = sum_v p_v E_v = T * d lse / d h: central differences over each hidden coordinate."""
    V, d = 300, 6
    rng = np.random.default_rng(4)
    E = synth.round_to_bf16(rng.standard_normal((V, d)).astype(np.float32))
    E64 = vp.widen_bf16(E)
    h = rng.standard_normal(d)
    T = 0.7

    def lse_of(hv):
        z = (E64 @ hv) / T
        return float(mpmath.log(mpmath.fsum(mpmath.exp(mpmath.mpf(x)) for x in z)))

    # the oracle needs bf16 hidden states: use an exactly representable h
    hb = synth.round_to_bf16(h.astype(np.float32))
    h64 = vp.widen_bf16(hb)
    r = vp.vocab_pass_rows(E64, hb[None, :], [0], np.array([T]), np.array([False]), 0,
                           np.array([0]))
    eps = 1e-6
    grad = np.zeros(d)
    for i in range(d):
        e = np.zeros(d)
        e[i] = eps
        grad[i] = (lse_of(h64 + e) - lse_of(h64 - e)) / (2 * eps)
    assert np.allclose(r.sc[0], T * grad, atol=1e-8)


def test_entropy_increases_with_temperature():
    wl = synth.workload("tiny", V=777, d=32)
    Hs = [_run(wl.E, wl.h[:4], T=T, want_sc=False).entropy for T in (0.3, 0.5, 0.8, 1.0, 1.5, 3.0)]
    for a, b in zip(Hs, Hs[1:]):
        assert np.all(b > a)
    assert np.all(Hs[-1] < math.log(777))


def test_brute_force_v16_high_precision():
    """V = 16: lse, H and sc against 40-digit sums taken straight from -sum p log p and
    sum p E (mpmath), argmax by exhaustive comparison."""
    V, d = 16, 8
    rng = np.random.default_rng(7)
    E = synth.round_to_bf16(rng.standard_normal((V, d)).astype(np.float32))
    h = synth.round_to_bf16(rng.standard_normal((4, d)).astype(np.float32) * 2)
    T = 0.8
    r = _run(E, h, T=T)
    mpmath.mp.dps = 40
    E64, h64 = vp.widen_bf16(E), vp.widen_bf16(h)
    for i in range(4):
        logits = [mpmath.fsum(mpmath.mpf(h64[i, k]) * mpmath.mpf(E64[v, k]) for k in range(d))
                  for v in range(V)]
        w = [mpmath.exp(x / T) for x in logits]
        Z = mpmath.fsum(w)
        p = [x / Z for x in w]
        H = -mpmath.fsum(q * mpmath.log(q) for q in p)
        assert abs(float(mpmath.log(Z)) - r.lse[i]) < 1e-12
        assert abs(float(H) - r.entropy[i]) < 1e-12
        for k in range(d):
            s = mpmath.fsum(p[v] * mpmath.mpf(E64[v, k]) for v in range(V))
            assert abs(float(s) - r.sc[i, k]) < 1e-13
        best = max(range(V), key=lambda v: (logits[v], -v))
        assert r.argmax[i] == best


def test_gumbel_max_samples_the_tempered_distribution():
    """Across rows (independent noise counters) with identical logits, Gumbel-max token
    frequencies match softmax(S/T): chi-square test at V = 16."""
    V, d, n = 16, 4, 20000
    rng = np.random.default_rng(3)
    E = synth.round_to_bf16(rng.standard_normal((V, d)).astype(np.float32))
    h1 = synth.round_to_bf16(rng.standard_normal((1, d)).astype(np.float32))
    h = np.repeat(h1, n, axis=0)
    T = 0.8
    r = _run(E, h, T=T, want_sc=False, seed=12345, step=2)
    z = (vp.widen_bf16(E) @ vp.widen_bf16(h1)[0]) / T
    p = np.exp(z - z.max())
    p /= p.sum()
    counts = np.bincount(r.gumbel, minlength=V)
    keep = p * n >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    exp = np.append(p[keep] * n, p[~keep].sum() * n)
    assert stats.chisquare(obs, exp).pvalue > 1e-4
    # the noise differs between steps and seeds
    r2 = _run(E, h[:200], T=T, want_sc=False, seed=12345, step=3)
    assert not np.array_equal(r.gumbel[:200], r2.gumbel)


def test_commit_rows_only_argmax():
    wl = synth.workload("tiny", V=256, d=32)
    r = _run(wl.E, wl.h[:4], commit=True)
    assert np.all(np.isnan(r.entropy)) and np.all(r.gumbel == -1) and np.all(np.isnan(r.sc))
    r2 = _run(wl.E, wl.h[:4], commit=False)
    assert np.array_equal(r.argmax, r2.argmax)


def test_argmax_tie_lowest_index():
    V, d = 8, 2
    E = np.zeros((V, d), dtype=np.float32)
    E[3] = [1, 0]
    E[6] = [1, 0]
    E[1] = [0.5, 0]
    h = np.array([[2.0, 0.0]], dtype=np.float32)
    r = _run(synth.round_to_bf16(E), synth.round_to_bf16(h))
    assert r.argmax[0] == 3 and r.mu_argmax[0] == 0.0


# --- final-logit soft cap and temperature schedule ---------------------------------------

def _run_cap(E_bits, h_bits, c, T=1.0, seed=0, step=0, want_sc=True):
    R = h_bits.shape[0]
    return vp.vocab_pass_rows(vp.widen_bf16(E_bits), h_bits, np.arange(R), np.full(R, T),
                              np.zeros(R, bool), seed, np.full(R, step), want_sc=want_sc,
                              softcap=c)


def test_softcap_large_cap_is_no_cap():
    """c tanh(S / c) -> S as c grows: a cap far above every logit leaves all outputs."""
    wl = synth.workload("tiny", V=700, d=64)
    h = wl.h[:6]
    a = _run(wl.E, h, T=0.8, seed=3, step=2)
    b = _run_cap(wl.E, h, 1e7, T=0.8, seed=3, step=2)
    assert np.allclose(a.lse, b.lse, atol=1e-9, rtol=0)
    assert np.allclose(a.entropy, b.entropy, atol=1e-9, rtol=0)
    assert np.allclose(a.sc, b.sc, atol=1e-9, rtol=0)
    assert np.array_equal(a.argmax, b.argmax) and np.array_equal(a.gumbel, b.gumbel)


@pytest.mark.parametrize("V,k,a,b,c,T", [(64, 3, 2.0, -1.0, 1.5, 1.0),
                                         (5000, 17, 6.5, 0.25, 4.0, 0.8),
                                         (300, 299, -3.0, 4.0, 30.0, 0.4)])
def test_softcap_two_level_closed_form(V, k, a, b, c, T):
    """Two logit levels, capped then tempered: z = c tanh(level / c) / T (tanh from mpmath)."""
    Eb, hb = _two_level(V, k, a, b)
    r = _run_cap(Eb, hb, c, T=T)
    za = float(c * mpmath.tanh(mpmath.mpf(a) / c) / T)
    zb = float(c * mpmath.tanh(mpmath.mpf(b) / c) / T)
    Z = k * math.exp(za) + (V - k) * math.exp(zb)
    pa, pb = math.exp(za) / Z, math.exp(zb) / Z
    H = -(k * pa * math.log(pa) + (V - k) * pb * math.log(pb))
    assert abs(r.lse[0] - math.log(Z)) < 1e-12 * max(1, abs(math.log(Z)))
    assert abs(r.entropy[0] - H) < 1e-12
    assert np.allclose(r.sc[0], [k * pa, (V - k) * pb], atol=1e-14)
    assert r.argmax[0] == (0 if a >= b else k)


def test_softcap_saturation_limit():
    """Logits far beyond the cap saturate at +-c: the distribution becomes two-level, c / T on
    the n+ tokens with S > 0 and -c / T on the rest, whatever S's magnitudes."""
    V, c, T = 4000, 2.0, 0.7
    rng = np.random.default_rng(11)
    E = np.stack([rng.choice([-1.0, 1.0], V), rng.standard_normal(V)], axis=1)
    E = synth.round_to_bf16(E.astype(np.float32))
    h = synth.round_to_bf16(np.array([[4096.0, 1.0], [-2048.0, 3.0], [1024.0, -7.0]],
                                     np.float32))
    r = _run_cap(E, h, c, T=T)
    S = vp.widen_bf16(h) @ vp.widen_bf16(E).T
    assert np.abs(S).min() > 200 * c  # tanh(200) == 1 in fp64
    for i in range(3):
        npos = int(np.sum(S[i] > 0))
        Z = npos * math.exp(c / T) + (V - npos) * math.exp(-c / T)
        assert abs(r.lse[i] - math.log(Z)) < 1e-12 * abs(math.log(Z))
        assert r.argmax[i] == int(np.argmax(S[i]))


def test_softcap_bounds_lse_and_entropy():
    """|z| <= c / T: ln V - c / T <= lse <= ln V + c / T, and H <= ln V; the argmax token is
    S's argmax whatever the cap."""
    wl = synth.workload("tiny", V=900, d=64)
    h = synth.round_to_bf16(synth.bf16_to_f32(wl.h[:8]) * 50.0)
    for c in (0.5, 3.0, 20.0):
        r = _run_cap(wl.E, h, c, T=0.6)
        lnV = math.log(900)
        assert np.all(r.lse <= lnV + c / 0.6 + 1e-12)
        assert np.all(r.lse >= lnV - c / 0.6 - 1e-12)
        assert np.all(r.entropy <= lnV + 1e-12)
        S = vp.widen_bf16(h) @ vp.widen_bf16(wl.E).T
        assert np.array_equal(r.argmax, np.argmax(S, axis=1))


def test_softcap_rejects_bad_values():
    wl = synth.workload("tiny", V=64, d=16)
    for c in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            _run_cap(wl.E, wl.h[:1], c)


def test_temperature_schedule_endpoints():
    """t_0 = t_max, linear steps of (t_min - t_max) / N, never reaching t_min; the default
    anneal of the technical report runs from 0.8 toward 0.4."""
    N = 32
    ts = [vp.temperature_schedule(i, N, 0.8, 0.4) for i in range(N)]
    assert ts[0] == 0.8
    assert abs(ts[16] - 0.6) < 1e-15
    assert abs(ts[-1] - (0.4 + 0.4 / N)) < 1e-15
    assert all(b < a for a, b in zip(ts, ts[1:]))
    assert np.allclose(np.diff(ts), -0.4 / N, atol=1e-15)
    with pytest.raises(ValueError):
        vp.temperature_schedule(N, N, 0.8, 0.4)


def test_confidence_closed_forms():
    """conf = p of the argmax token: 1 / V for equal logits, the top level's probability for
    two-level logits."""
    wl = synth.workload("tiny", V=500, d=32)
    r = _run(wl.E, np.zeros((2, 32), np.uint16), T=0.7)
    assert np.allclose(r.conf, 1.0 / 500, rtol=1e-12)
    V, k, a, b, T = 400, 3, 3.0, 0.5, 0.8
    Eb, hb = _two_level(V, k, a, b)
    r = _run(Eb, hb, T=T)
    Z = k * math.exp(a / T) + (V - k) * math.exp(b / T)
    assert abs(r.conf[0] - math.exp(a / T) / Z) < 1e-14
