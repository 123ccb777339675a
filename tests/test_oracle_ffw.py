"""Pins of the self-conditioning consumer oracle: bf16 rounding against an independent bit-level
rounding, GELU at values of the normal CDF and its odd-part identity, permutation weights
(whose result is known entry by entry and catches a transposed operand), the zero-input
identity of the first decode step, scale invariance of the pre-norm, the norm of the output
and the placement of eps."""
import math

import numpy as np

from denoise_step_sampler_amd import synth
from oracle import selfcond_ffw as of


def test_round_bf16_matches_bit_rounding():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([1e-39, -3e-40, 2.0 ** -130, 0.0, 65504.0, -1.0])])
    x32 = x.astype(np.float32)
    got = of.round_bf16(x32.astype(np.float64))
    want = synth.bf16_to_f32(synth.round_to_bf16(x32)).astype(np.float64)
    assert np.array_equal(got, want)


def test_round_bf16_ties_to_even():
    one = 1.0
    assert of.round_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0            # tie -> even (1)
    assert of.round_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6
    assert of.round_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -30]))[0] == one + 2.0 ** -7


def test_gelu_values_and_odd_identity():
    # Phi(1) and Phi(-1) of the standard normal distribution
    assert abs(of.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    assert abs(of.gelu(np.array([-1.0]))[0] + 0.15865525393145707) < 1e-15
    assert of.gelu(np.array([0.0]))[0] == 0.0
    x = np.linspace(-6, 6, 101)
    assert np.allclose(of.gelu(x) - of.gelu(-x), x, atol=1e-14)   # Phi(x) + Phi(-x) = 1
    assert np.allclose(of.gelu(np.array([40.0, -40.0])), [40.0, 0.0])


def _weights(D, F, seed):
    rng = np.random.default_rng(seed)
    mk = lambda *s: synth.round_to_bf16((rng.standard_normal(s) / math.sqrt(s[-1])).astype(np.float32))
    pre = synth.round_to_bf16((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    return pre, mk(F, D), mk(F, D), mk(D, F)


def test_first_step_zero_input_is_plain_embedding():
    V, D, F, R = 50, 16, 24, 6
    E = synth.make_embedding(V, D, seed=3)
    tok = np.arange(R) * 7 % V
    pre, Wg, Wu, Wd = _weights(D, F, 1)
    a = of.selfcond_input(None, tok, E, pre, Wg, Wu, Wd)
    b = of.selfcond_input(np.zeros((R, D)), tok, E, pre, Wg, Wu, Wd)
    assert np.array_equal(a, b)
    e = synth.bf16_to_f32(E[tok]).astype(np.float64)
    want = of.round_bf16(e * math.sqrt(D) / (np.linalg.norm(e, axis=1, keepdims=True) + 1e-6 / math.sqrt(D)) )
    assert np.allclose(a, want, rtol=2.0 ** -7, atol=0)


def test_permutation_weights_entrywise():
    """W_gate, W_up, W_down permutation matrices: y_j = x1[pi(j)] GELU(x1[sigma(j)]) and
    res_i = y[rho(i)], with x1 = the pre-normed row (pre-norm weights powers of two)."""
    V, D, R = 40, 8, 5
    F = D
    rng = np.random.default_rng(9)
    E = synth.make_embedding(V, D, seed=4)
    tok = rng.integers(0, V, R)
    sc = rng.standard_normal((R, D))
    pi, sigma, rho = rng.permutation(D), rng.permutation(D), rng.permutation(D)
    for p in (pi, sigma, rho):
        assert not np.array_equal(np.argsort(p), p)   # not an involution
    perm = lambda q: synth.round_to_bf16(np.eye(D, dtype=np.float32)[q])  # row j = e_q[j]
    w = 2.0 ** rng.integers(-1, 2, D)
    pre = synth.round_to_bf16(w.astype(np.float32))
    eps = 1e-6
    got = of.selfcond_input(sc, tok, E, pre, perm(sigma), perm(pi), perm(rho), eps=eps)
    s = math.sqrt(D)
    for r in range(R):
        cx = sc[r] * s
        x1 = of.round_bf16(w * cx * s / (math.sqrt(sum(v * v for v in cx)) + eps))
        y = np.array([of.round_bf16(np.array([x1[pi[j]] * 0.5 * x1[sigma[j]] *
                                             (1 + math.erf(x1[sigma[j]] / math.sqrt(2)))]))[0]
                      for j in range(F)])
        res = np.array([y[rho[i]] for i in range(D)])
        x = synth.bf16_to_f32(E[tok[r]]).astype(np.float64) * s + res
        want = of.round_bf16(x * s / (math.sqrt(sum(v * v for v in x)) + eps))
        assert np.array_equal(got[r], want), r


def test_prenorm_scale_invariance_and_output_norm():
    V, D, F, R = 300, 64, 96, 8
    rng = np.random.default_rng(2)
    E = synth.make_embedding(V, D, seed=5)
    tok = rng.integers(0, V, R)
    sc = rng.standard_normal((R, D)) * 0.05
    pre, Wg, Wu, Wd = _weights(D, F, 3)
    a = of.selfcond_input(sc, tok, E, pre, Wg, Wu, Wd, eps=0.0)
    b = of.selfcond_input(2.0 * sc, tok, E, pre, Wg, Wu, Wd, eps=0.0)
    assert np.array_equal(a, b)
    c = of.selfcond_input(sc, tok, E, pre, Wg, Wu, Wd)
    n = np.linalg.norm(c, axis=1)
    assert np.all(np.abs(n / math.sqrt(D) - 1.0) < 2.0 ** -8)


def test_eps_is_added_to_the_norm():
    """Embedding row (1, 0, 0, 0), D = 4, eps = 2, first step: x = E[tok] sqrt(D) = (2, 0, 0, 0)
    has norm 2 = eps, so the first entry is 2 sqrt(D) / (2 + eps) = 1 exactly (eps inside a
    square root, or added to the mean square, would give another value)."""
    D = 4
    E = synth.round_to_bf16(np.array([[1.0, 0.0, 0.0, 0.0]], np.float32))
    pre, Wg, Wu, Wd = _weights(D, 4, 0)
    out = of.selfcond_input(None, np.array([0]), E, pre, Wg, Wu, Wd, eps=2.0)
    assert out[0, 0] == 1.0 and np.all(out[0, 1:] == 0.0)


def test_commit_rows_untouched():
    V, D, F, R = 30, 8, 8, 4
    E = synth.make_embedding(V, D, seed=6)
    pre, Wg, Wu, Wd = _weights(D, F, 7)
    out = of.selfcond_input(np.ones((R, D)), np.arange(R), E, pre, Wg, Wu, Wd,
                            commit_row=np.array([0, 1, 1, 0], bool))
    assert np.all(np.isnan(out[1:3])) and not np.isnan(out[[0, 3]]).any()


def test_out_of_range_tokens_give_nan_rows():
    V, D, F = 30, 8, 8
    E = synth.make_embedding(V, D, seed=6)
    pre, Wg, Wu, Wd = _weights(D, F, 7)
    out = of.selfcond_input(None, np.array([0, -1, V, 5]), E, pre, Wg, Wu, Wd)
    assert np.all(np.isnan(out[1:3])) and not np.isnan(out[[0, 3]]).any()
