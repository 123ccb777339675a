"""Parity of dg_vocab_pass (through the C ABI) with the fp64 oracle."""
import math
import os
import sys

import numpy as np
import pytest

from denoise_step_sampler_amd import synth
from oracle import vocab_pass as ovp
from parity import VocabInputs, compare_vocab

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


def _run(wl, seed, want_sc=True, E_t=None):
    from denoise_step_sampler_amd import runner
    b = runner.from_workload(wl, want_selfcond=want_sc, E=E_t)
    runner.vocab_pass(b, seed)
    torch.cuda.synchronize()
    return b


def _host(b, rows):
    out = {"lse": b.lse.cpu().numpy()[rows], "entropy": b.entropy.cpu().numpy()[rows],
           "argmax": b.argmax_tok.cpu().numpy()[rows], "gumbel": b.gumbel_tok.cpu().numpy()[rows]}
    out["sc"] = None if b.selfcond is None else b.selfcond.cpu().numpy()[rows]
    return out


def _inputs(wl, seed, E64, softcap=None, draw_T=None):
    return VocabInputs(E64=E64, h_bits=wl.h, temperature_row=np.repeat(wl.temperature, wl.C),
                       step_row=np.repeat(wl.step, wl.C), seed=seed, softcap=softcap,
                       draw_temperature_row=None if draw_T is None else np.repeat(draw_T, wl.C))


def _oracle(wl, rows, seed, E64=None, want_sc=True):
    E64 = ovp.widen_bf16(wl.E) if E64 is None else E64
    T = np.repeat(wl.temperature, wl.C)
    cm = np.repeat(wl.commit.astype(bool), wl.C)
    st = np.repeat(wl.step, wl.C)
    return ovp.vocab_pass_rows(E64, wl.h, rows, T, cm, seed, st, want_sc=want_sc), cm


def _check(wl, seed, rows=None, want_sc=True, E64=None, E_t=None, label="", max_exempt=None):
    _say(f"[vocab_pass] {label} n={wl.n_canvas} V={wl.V} d={wl.d} seed={seed}")
    b = _run(wl, seed, want_sc, E_t=E_t)
    rows = np.arange(wl.R) if rows is None else np.asarray(rows)
    E64 = ovp.widen_bf16(wl.E) if E64 is None else E64
    ref, cm = _oracle(wl, rows, seed, E64=E64, want_sc=want_sc)
    rep = compare_vocab(_host(b, rows), ref, cm, inputs=_inputs(wl, seed, E64),
                        max_exempt=max_exempt)
    _say("   ", rep)
    return b, rep


def test_tiny_workload_full():
    wl = synth.workload("tiny")
    _check(wl, seed=0, label="tiny")


@pytest.mark.parametrize("V,d,n", [(1000, 128, 2), (50, 128, 1), (129, 384, 1), (1, 128, 1),
                                   (1000, 256, 2), (1, 256, 1), (300, 640, 3), (5000, 1024, 2)])
def test_ragged_vocab_and_widths(V, d, n):
    """Vocabulary tails (V % 128 != 0, V < one tile, V = 1), widths of 1, 2, 3, 5 and 8 column
    blocks of 128."""
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=3)
    wl.temperature = np.linspace(0.7, 1.3, n).astype(np.float32)
    wl.step = np.arange(n, dtype=np.int32) + 5
    if n > 1:
        wl.commit = (np.arange(n) % 2).astype(np.uint8)
    _check(wl, seed=0xDEADBEEF12345, label="ragged")


@pytest.mark.parametrize("n", [5, 12, 33])
def test_canvas_rounds(n):
    """Canvas counts that split into rounds of several sizes (the logits pass runs rounds of
    up to 32 canvases, then the binary decomposition of the rest), commit canvases mixed in."""
    wl = synth.workload("lite", V=1500, d=128, n_canvas=n, seed=11)
    wl.temperature = np.linspace(0.6, 1.4, n).astype(np.float32)
    wl.step = (np.arange(n, dtype=np.int32) * 7) % 5
    wl.commit = (np.arange(n) % 3 == 1).astype(np.uint8)
    rows = np.sort(np.random.default_rng(n).choice(wl.R, size=min(wl.R, 160), replace=False))
    _check(wl, seed=77, rows=rows, label=f"rounds n={n}")


def test_uniform_and_peaked_rows():
    """h = 0 rows: entropy = lse = ln V, argmax 0, selfcond = mean E.  Peaked rows: argmax =
    Gumbel = target, entropy ~ 0.  The 64 zero rows tie every logit by construction, so their
    argmax decisions are exempt (and confirmed as exact ties by the recomputation)."""
    wl = synth.workload("tiny", V=3000, d=256, seed=4)
    h = wl.h.copy()
    h[:64] = 0
    t = wl.targets[64:128]
    h[64:128] = synth.round_to_bf16(60.0 * synth.bf16_to_f32(wl.E[t]))
    wl.h = h
    b, rep = _check(wl, seed=1, label="uniform+peaked", max_exempt=64)
    assert rep["argmax_exempt"] == 64
    H = b.entropy.cpu().numpy()
    assert np.allclose(H[:64], math.log(3000), rtol=1e-5)
    assert np.all(b.argmax_tok.cpu().numpy()[:64] == 0)
    mean_e = synth.bf16_to_f32(wl.E).astype(np.float64).mean(0)
    sc = b.selfcond.cpu().numpy()[:64]
    assert np.all(np.linalg.norm(sc - mean_e, axis=1) <= 2e-3 * np.linalg.norm(mean_e))
    assert np.array_equal(b.argmax_tok.cpu().numpy()[64:128], t)
    assert np.array_equal(b.gumbel_tok.cpu().numpy()[64:128], t)


def test_no_selfcond_and_determinism():
    wl = synth.workload("tiny", V=2000, d=128, n_canvas=2, seed=6)
    b1 = _run(wl, 9, want_sc=False)
    b2 = _run(wl, 9, want_sc=True)
    b3 = _run(wl, 9, want_sc=True)
    for k in ("lse", "entropy", "argmax_tok", "gumbel_tok"):
        x1, x2 = getattr(b1, k).cpu().numpy(), getattr(b2, k).cpu().numpy()
        assert np.array_equal(x1.view(np.uint32), x2.view(np.uint32)), k
    assert np.array_equal(b2.selfcond.cpu().numpy().view(np.uint32),
                          b3.selfcond.cpu().numpy().view(np.uint32))
    b4 = _run(wl, 10, want_sc=False)   # other seed, other samples
    assert not np.array_equal(b1.gumbel_tok.cpu().numpy(), b4.gumbel_tok.cpu().numpy())


def test_lite_workload_sampled_rows():
    wl = synth.workload("lite")
    rows = np.random.default_rng(0).choice(wl.R, size=96, replace=False)
    _check(wl, seed=0, rows=np.sort(rows), label="lite")


def test_determinism():
    """The pass is bit-reproducible (no atomics decide an order)."""
    wl = synth.workload("lite", V=20000, d=1024, n_canvas=3, seed=8)
    wl.commit = np.array([0, 1, 0], np.uint8)
    a = _run(wl, 5)
    b = _run(wl, 5)
    for k in ("lse", "entropy", "argmax_tok", "gumbel_tok", "selfcond"):
        x, y = getattr(a, k).cpu().numpy(), getattr(b, k).cpu().numpy()
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), k


@pytest.fixture(scope="module")
def large():
    _say("[vocab_pass] generating V=262144 d=2816 embedding")
    E = synth.make_embedding(262144, 2816, seed=0)
    from denoise_step_sampler_amd import runner
    E_t = runner.bf16_tensor(E)
    E64 = ovp.widen_bf16(E)
    yield E, E_t, E64


def test_large_vocab_single_canvas_sampled(large):
    E, E_t, E64 = large
    wl = synth.workload("large_v", E=E)
    rows = np.array([0, 1, 37, 100, 128, 200, 254, 255])
    _check(wl, seed=0, rows=rows, E64=E64, E_t=E_t, label="large_v")


def test_batched_serving_step_sampled(large):
    E, E_t, E64 = large
    wl = synth.workload("batched", E=E)
    rng = np.random.default_rng(1)
    canv = [0, 3, 5, 7, 22, 31]   # 3, 7, 31 commit
    rows = np.sort(np.concatenate([c * 256 + rng.choice(256, 3, replace=False) for c in canv]))
    b, rep = _check(wl, seed=0, rows=rows, E64=E64, E_t=E_t, label="batched")
    assert rep["commit_rows"] == 9
    # every commit row of every commit canvas untouched except argmax
    cm = np.repeat(wl.commit.astype(bool), 256)
    assert np.all(np.isnan(b.entropy.cpu().numpy()[cm]))
    assert np.all(b.argmax_tok.cpu().numpy() >= 0)


# --- final-logit soft cap ----------------------------------------------------------------

def _check_cap(wl, seed, c, rows=None, E64=None, E_t=None, label=""):
    from denoise_step_sampler_amd import runner
    _say(f"[vocab_pass softcap={c}] {label} n={wl.n_canvas} V={wl.V} d={wl.d} seed={seed}")
    b = runner.from_workload(wl, E=E_t)
    runner.vocab_pass(b, seed, softcap=c)
    torch.cuda.synchronize()
    rows = np.arange(wl.R) if rows is None else np.asarray(rows)
    E64 = ovp.widen_bf16(wl.E) if E64 is None else E64
    ref = ovp.vocab_pass_rows(E64, wl.h, rows, np.repeat(wl.temperature, wl.C),
                              np.repeat(wl.commit.astype(bool), wl.C), seed,
                              np.repeat(wl.step, wl.C), softcap=c)
    rep = compare_vocab(_host(b, rows), ref, np.repeat(wl.commit.astype(bool), wl.C),
                        inputs=_inputs(wl, seed, E64, softcap=c))
    _say("   ", rep)
    return b, rep


@pytest.mark.parametrize("c,scale,V,d", [(5.0, 1.0, 5000, 256), (30.0, 1.0, 1000, 128),
                                         (2.0, 8.0, 777, 384), (30.0, 3.0, 129, 256)])
def test_softcap_parity(c, scale, V, d):
    """Soft-capped logits against the oracle: a strong cap, a mild one, hidden states scaled
    so that most logits saturate, ragged vocabularies, a commit canvas mixed in."""
    wl = synth.workload("lite", V=V, d=d, n_canvas=3, seed=21)
    wl.h = synth.round_to_bf16(synth.bf16_to_f32(wl.h) * np.float32(scale))
    wl.temperature = np.array([0.4, 0.8, 1.0], np.float32)
    wl.step = np.array([0, 3, 9], np.int32)
    wl.commit = np.array([0, 1, 0], np.uint8)
    _check_cap(wl, 0x5EED, c, label=f"c={c} x{scale}")


def test_softcap_deterministic_and_differs_from_plain():
    """Two capped runs agree bit for bit; a cap below the logits' range changes lse."""
    from denoise_step_sampler_amd import runner
    wl = synth.workload("lite", V=3000, d=256, n_canvas=2, seed=5)
    outs = []
    for c in (3.0, 3.0, None):
        b = runner.from_workload(wl)
        runner.vocab_pass(b, 9, softcap=c)
        torch.cuda.synchronize()
        outs.append(b)
    for k in ("lse", "entropy", "argmax_tok", "gumbel_tok", "selfcond"):
        x, y = getattr(outs[0], k).cpu().numpy(), getattr(outs[1], k).cpu().numpy()
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), k
    assert np.array_equal(outs[0].argmax_tok.cpu().numpy(), outs[2].argmax_tok.cpu().numpy())
    assert not np.allclose(outs[0].lse.cpu().numpy(), outs[2].lse.cpu().numpy())


def test_softcap_batched_serving_step_sampled(large):
    """The 32-canvas serving step at V = 262144, d = 2816 with a cap of 30, sampled rows."""
    E, E_t, E64 = large
    wl = synth.workload("batched", E=E)
    rng = np.random.default_rng(2)
    canv = [0, 3, 9, 30]
    rows = np.sort(np.concatenate([c * 256 + rng.choice(256, 3, replace=False) for c in canv]))
    _check_cap(wl, 3, 30.0, rows=rows, E64=E64, E_t=E_t, label="batched")


# --- maximum sizes ------------------------------------------------------------------------

def test_maximum_width():
    """d = DG_MAX_D = 8192 with a ragged vocabulary and a commit canvas, every row."""
    wl = synth.workload("lite", V=700, d=8192, n_canvas=2, seed=13)
    wl.commit = np.array([0, 1], np.uint8)
    wl.temperature = np.array([0.7, 1.0], np.float32)
    _check(wl, seed=21, label="d=8192")


def test_maximum_canvases_with_sampler():
    """n = DG_MAX_CANVASES = 4096 canvases (1,048,576 rows), every third one committing: the
    vocabulary pass on every row of four canvases, first, middle, commit and last, and the
    accept/renoise step of those canvases against the oracle."""
    from denoise_step_sampler_amd import runner
    from oracle import sampler as osm
    from parity import compare_sampler
    n, V, d = 4096, 300, 128
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=17)
    wl.commit = (np.arange(n) % 3 == 2).astype(np.uint8)
    wl.step = (np.arange(n) % 7).astype(np.int32)
    seed = 99
    _say(f"[vocab_pass] n={n} V={V} d={d}")
    b = runner.from_workload(wl)
    runner.vocab_pass(b, seed)
    runner.accept_renoise(b, wl.budget, wl.confidence, wl.stability, seed)
    torch.cuda.synchronize()
    canv = np.array([0, 2047, 2048, 4095])
    assert wl.commit[2048] == 1 and wl.commit[2047] == 0
    rows = (canv[:, None] * 256 + np.arange(256)[None, :]).reshape(-1)
    E64 = ovp.widen_bf16(wl.E)
    ref, cm = _oracle(wl, rows, seed, E64=E64)
    _say("   ", compare_vocab(_host(b, rows), ref, cm, inputs=_inputs(wl, seed, E64)))
    # the sampler on the oracle's values for the same canvases (as one batch of four)
    sref = osm.accept_renoise(ref.entropy, ref.argmax, ref.gumbel, wl.commit[canv], 4, 256, V,
                              wl.budget, wl.confidence, wl.stability, seed, wl.step[canv],
                              np.full(4 * 256, -1), np.zeros(4, np.int64), canvas_ids=canv)
    got = {"next_tokens": b.next_tokens.cpu().numpy()[rows],
           "accept": b.accept_mask.cpu().numpy()[rows],
           "converged": b.converged.cpu().numpy()[canv],
           "mean_entropy": b.mean_entropy.cpu().numpy()[canv],
           "prev_argmax": b.prev_argmax.cpu().numpy()[rows],
           "stable_count": b.stable_count.cpu().numpy()[canv]}
    _say("   ", compare_sampler(got, sref, wl.commit[canv], 256, H=ref.entropy,
                               budget=wl.budget))


@pytest.mark.parametrize("scale,T", [(1.0, 0.02), (1.0, 50.0), (20.0, 0.4), (0.0, 0.3)])
def test_extreme_temperatures_and_logit_ranges(scale, T):
    """Very sharp (T = 0.02: z spans thousands of nats) and very flat (T = 50) distributions,
    logits twenty times the usual range, and all-zero hidden states (every logit ties, so every
    argmax decision is exempt by construction), against the oracle."""
    wl = synth.workload("lite", V=3000, d=256, n_canvas=2, seed=31)
    wl.h = synth.round_to_bf16(synth.bf16_to_f32(wl.h) * np.float32(scale))
    wl.temperature = np.full(2, T, np.float32)
    _check(wl, seed=4, label=f"x{scale} T={T}", max_exempt=wl.R if scale == 0.0 else None)


# --- a draw temperature of its own (dg_vocab_pass_ex) ---------------------------------------

def _run_ex(wl, seed, draw_T, softcap=None, want_sc=True):
    from denoise_step_sampler_amd import runner
    b = runner.from_workload(wl, want_selfcond=want_sc)
    b.draw_temperature = None if draw_T is None else torch.as_tensor(
        np.asarray(draw_T, np.float32)).cuda()
    runner.vocab_pass(b, seed, softcap=softcap)
    torch.cuda.synchronize()
    return b


@pytest.mark.parametrize("softcap,V,d", [(None, 3000, 256), (15.0, 1200, 384), (None, 129, 128)])
def test_draw_temperature_parity(softcap, V, d):
    """Statistics at T = 1 (the DiffusionGemma-Lite posterior) and the Gumbel draw at an
    annealed tau per canvas, a commit canvas mixed in, against the oracle."""
    wl = synth.workload("lite", V=V, d=d, n_canvas=3, seed=41)
    wl.temperature = np.ones(3, np.float32)
    wl.commit = np.array([0, 1, 0], np.uint8)
    wl.step = np.array([2, 4, 6], np.int32)
    tau = np.array([0.8, 0.6, 0.45], np.float32)
    seed = 0xABCD
    b = _run_ex(wl, seed, tau, softcap)
    rows = np.arange(wl.R)
    E64 = ovp.widen_bf16(wl.E)
    ref = ovp.vocab_pass_rows(E64, wl.h, rows, np.repeat(wl.temperature, wl.C),
                              np.repeat(wl.commit.astype(bool), wl.C), seed,
                              np.repeat(wl.step, wl.C), softcap=softcap,
                              draw_temperature_row=np.repeat(tau, wl.C))
    rep = compare_vocab(_host(b, rows), ref, np.repeat(wl.commit.astype(bool), wl.C),
                        inputs=_inputs(wl, seed, E64, softcap=softcap, draw_T=tau))
    _say("   ", rep)
    # the draw really follows tau: drawn at T = 1 instead, canvas 2 (tau = 0.45) changes about
    # half of its tokens (0.50 to 0.57 on these three cases in the oracle)
    flat = ovp.vocab_pass_rows(E64, wl.h, rows[512:], np.ones(wl.R), np.zeros(wl.R, bool), seed,
                               np.repeat(wl.step, wl.C), want_sc=False, softcap=softcap)
    assert (flat.gumbel != b.gumbel_tok.cpu().numpy()[512:]).mean() > 0.3


def test_draw_temperature_equal_to_statistics_is_the_plain_pass():
    """dg_vocab_pass_ex with the draw at the statistics' temperature gives dg_vocab_pass's
    bits (with and without the cap)."""
    wl = synth.workload("lite", V=2500, d=256, n_canvas=2, seed=43)
    wl.temperature = np.array([0.7, 1.3], np.float32)
    for cap in (None, 10.0):
        a = _run_ex(wl, 3, wl.temperature, cap)
        b = _run_ex(wl, 3, None, cap)
        for k in ("lse", "entropy", "argmax_tok", "gumbel_tok", "selfcond"):
            x, y = getattr(a, k).cpu().numpy(), getattr(b, k).cpu().numpy()
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), (cap, k)


# --- the fp16 embedding ---------------------------------------------------------------------

def test_embedding_f16_is_the_fp16_conversion():
    """dg_embedding_f16: fp16(E) (round to nearest even, numpy's conversion), zero entries past
    V up to the padded count, in the fragment order of the header; tiny and large entries
    included."""
    from denoise_step_sampler_amd import runner
    V, d = 1000, 256
    E = synth.bf16_to_f32(synth.make_embedding(V, d, seed=5)).copy()
    E[3, :8] = [1e-6, -3e-8, 6.1e-5, 65000.0, -65000.0, 1.0 + 2.0 ** -8, 2.0 ** -24, 0.0]
    E_bits = synth.round_to_bf16(E.astype(np.float32))
    t = runner.embedding_f16(runner.bf16_tensor(E_bits), V, d)
    torch.cuda.synchronize()
    rows = (V + 255) // 256 * 256
    want = np.zeros((rows, d), np.uint16)
    want[:V] = synth.bf16_to_f32(E_bits).astype(np.float16).view(np.uint16)
    got = t.cpu().numpy().view(np.uint16)
    from parity import fragment_order
    assert np.array_equal(got, fragment_order(want, d))


def test_prepared_embedding_gives_the_same_bits():
    """The pass with a caller-prepared fp16 embedding equals the pass that builds one in its
    workspace, bit for bit."""
    from denoise_step_sampler_amd import runner
    wl = synth.workload("lite", V=6000, d=384, n_canvas=3, seed=44)
    wl.commit = np.array([0, 1, 0], np.uint8)
    a = runner.from_workload(wl)
    runner.vocab_pass(a, 6)
    b = runner.from_workload(wl, E=a.E, E16=runner.embedding_f16(a.E, wl.V, wl.d))
    runner.vocab_pass(b, 6)
    torch.cuda.synchronize()
    for k in ("lse", "entropy", "argmax_tok", "gumbel_tok", "selfcond"):
        x, y = getattr(a, k).cpu().numpy(), getattr(b, k).cpu().numpy()
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), k


@pytest.mark.parametrize("V,d,T", [(101, 128, 3.0), (101, 512, 50.0), (1000, 128, 50.0),
                                   (5000, 256, 50.0), (1000, 2816, 3.0)])
def test_flat_distributions_expectation(V, d, T):
    """Near-uniform rows, where the expectation's rounding does not average down against its
    own size: every row within the 2e-3 bar (bf16 weights measured up to 2.6e-3 here in a CPU
    emulation; fp16 weights and the rescaled accumulator keep it near 3e-4)."""
    wl = synth.workload("lite", V=V, d=d, n_canvas=2, seed=V + d)
    wl.h = synth.round_to_bf16(synth.bf16_to_f32(wl.h) * np.float32(0.5))
    wl.temperature = np.full(2, T, np.float32)
    _, rep = _check(wl, seed=8, label=f"flat T={T}")
    assert rep["sc_max_rel"] < 1e-3

@pytest.mark.parametrize("levels", [(100.0, 41.0, -18.0, -77.0), (41.0, 100.0, -18.0, -77.0),
                                    (-120.0, 100.0, 41.0, -18.0)])
def test_expectation_reference_chains(levels):
    """Half tiles whose largest logits lie about 85 log2 units apart, in falling, mixed and
    rising order, the rest of the vocabulary far below: the expectation scales every half
    tile's weights to one unit per row (15 below the row's largest reference), exactly for the
    half tiles near the top and to nothing for those far below, whatever the order in which
    the half tiles arrive; the sums stay finite and meet the oracle at the bars of every
    other case."""
    V, d, n = 65536, 128, 1
    rng = np.random.default_rng(31)
    E = rng.normal(0.0, 0.05, (V, d)).astype(np.float32)
    k = np.arange(V) // 128
    lev = np.full(V, -150.0, np.float32)
    for i, L in enumerate(levels):
        lev[k == i] = L
    E[:, 0] = lev - 0.5 * (np.arange(V) % 8)
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=31, E=synth.round_to_bf16(E))
    h = np.zeros((wl.R, d), np.float32)
    h[:, 0] = 1.0
    h[:, 1:] = rng.normal(0.0, 0.5, (wl.R, d - 1))
    wl.h = synth.round_to_bf16(h)
    wl.temperature = np.ones(n, np.float32)
    wl.commit = np.zeros(n, np.uint8)
    b, rep = _check(wl, seed=3, rows=np.arange(0, wl.R, 8), label=f"chain {levels}")
    assert np.isfinite(b.selfcond.cpu().numpy()).all()
