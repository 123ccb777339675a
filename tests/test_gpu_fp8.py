"""The FP8 embedding through the C ABI: the quantiser's codes and exponents bit for bit against
the oracle's, and the vocabulary pass on the FP8 embedding against the oracle's pass on the
dequantised rows (E~ = 2^k value(code), exact bf16 numbers thanks to the power-of-two
scales), at every size the bars of the hot-path contract: tokens bit-exact but for
margin-exempt near-ties, statistics within 2e-3."""

import sys

import numpy as np
import pytest

from denoise_step_sampler_amd import synth
from oracle import fp8 as of8
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


def _host(b, rows=None):
    rows = slice(None) if rows is None else rows
    out = {"lse": b.lse.cpu().numpy()[rows], "entropy": b.entropy.cpu().numpy()[rows],
           "argmax": b.argmax_tok.cpu().numpy()[rows], "gumbel": b.gumbel_tok.cpu().numpy()[rows]}
    out["sc"] = None if b.selfcond is None else b.selfcond.cpu().numpy()[rows]
    return out


def _against_oracle(b, wl, Eq64, rows, seed, softcap=None, label=""):
    """The pass in b (run on the FP8 form of wl.E) against the oracle on the dequantised rows."""
    T = np.repeat(wl.temperature, C)
    cm = np.repeat(wl.commit.astype(bool), C)
    st = np.repeat(wl.step, C)
    ref = ovp.vocab_pass_rows(Eq64, wl.h, rows, T, cm, seed, st, softcap=softcap,
                              want_sc=b.selfcond is not None)
    inp = VocabInputs(E64=Eq64, h_bits=wl.h, temperature_row=T, step_row=st, seed=seed,
                      softcap=softcap)
    rep = compare_vocab(_host(b, rows), ref, cm, inputs=inp)
    _say(f"    {label}", rep)
    return rep


def _special_embedding(V, d, seed):
    E = synth.bf16_to_f32(synth.make_embedding(V, d, seed=seed)).copy()
    E[0] = 0.0                                        # zero row: exponent floor
    E[1] *= 2.0 ** -100                               # tiny row
    E[2] *= 2.0 ** 40                                 # large row
    E[3, :6] = [448.0, 1.0625, 1.1875, -3.0 * 2.0 ** -10, 2.0 ** -10, -448.0]  # ties, k = 0
    E[3, 6:] = 0.5
    E[4] = np.where(np.arange(d) % 2, 224.0, -1e-3)   # |max| exactly 224: k = -1
    return synth.round_to_bf16(E.astype(np.float32))


def _quantize_gpu(E_bits, V, d, with_e16=True):
    from denoise_step_sampler_amd import runner
    E_t = runner.bf16_tensor(E_bits)
    f = runner.quantize_embedding_fp8(E_t, V, d, with_e16=with_e16)
    torch.cuda.synchronize()
    return f, f.codes.cpu().numpy().reshape(V, d), f.row_exp.cpu().numpy()


def test_quantizer_bit_exact():
    V, d = 3000, 256
    E = _special_embedding(V, d, 4)
    f, codes, k = _quantize_gpu(E, V, d)
    q_ref, k_ref = of8.quantize_rows(ovp.widen_bf16(E))
    assert np.array_equal(k, k_ref), np.nonzero(k != k_ref)[0][:8]
    bad = np.argwhere(codes != q_ref)
    assert bad.size == 0, [(int(r), int(c), int(codes[r, c]), int(q_ref[r, c])) for r, c in bad[:8]]
    # the expectation's operand: the dequantised rows as fp16, zero entries past V, in the
    # fragment order of the header (the row scaled by 2^40 lies beyond fp16's range and becomes
    # infinities on both sides)
    from parity import fragment_order
    rows = (V + 255) // 256 * 256
    want = np.zeros((rows, d), np.uint16)
    with np.errstate(over="ignore"):
        want[:V] = of8.dequantize_rows(q_ref, k_ref).astype(np.float16).view(np.uint16)
    assert np.array_equal(f.E16.cpu().numpy().view(np.uint16), fragment_order(want, d))


@pytest.mark.parametrize("softcap,prepared", [(None, True), (15.0, True), (None, False)])
def test_fp8_vocab_pass_parity_and_bf16_identity(softcap, prepared):
    """The pass on the codes (with the quantiser's fp16 rows for the expectation, or rows the
    pass builds itself) against the oracle on the dequantised rows, and the bf16 pass on those
    rows against the same oracle."""
    from denoise_step_sampler_amd import runner
    V, d, n = 5000, 256, 3
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=9)
    wl.commit = np.array([0, 1, 0], np.uint8)
    wl.temperature = np.array([0.5, 0.8, 1.1], np.float32)
    f, codes, k = _quantize_gpu(wl.E, V, d, prepared)
    q_ref, k_ref = of8.quantize_rows(ovp.widen_bf16(wl.E))
    assert np.array_equal(codes, q_ref) and np.array_equal(k, k_ref)
    Eq = of8.dequantize_rows(q_ref, k_ref)              # the oracle's dequantised rows
    Eq_bits = synth.round_to_bf16(Eq.astype(np.float32))
    assert np.array_equal(ovp.widen_bf16(Eq_bits), Eq)  # exact in bf16
    seed = 0xF8
    _say(f"[vocab_pass_fp8] softcap={softcap} prepared={prepared} n={n} V={V} d={d}")
    b = runner.from_workload(wl)
    ws = runner.fp8_workspace(n, V, d)
    runner.vocab_pass_fp8(b, f, ws, seed, softcap=softcap)
    torch.cuda.synchronize()
    rows = np.arange(n * C)
    ref = ovp.vocab_pass_rows(Eq, wl.h, rows, np.repeat(wl.temperature, C),
                              np.repeat(wl.commit.astype(bool), C), seed, np.repeat(wl.step, C),
                              softcap=softcap)
    inp = VocabInputs(E64=Eq, h_bits=wl.h, temperature_row=np.repeat(wl.temperature, C),
                      step_row=np.repeat(wl.step, C), seed=seed, softcap=softcap)
    _say("   ", compare_vocab(_host(b), ref, np.repeat(wl.commit.astype(bool), C), inputs=inp))
    # the bf16 pass on the dequantised rows meets the same oracle
    b2 = runner.from_workload(wl, E=runner.bf16_tensor(Eq_bits))
    runner.vocab_pass(b2, seed, softcap=softcap)
    torch.cuda.synchronize()
    _say("    bf16 pass on the dequantised rows:",
         compare_vocab(_host(b2), ref, np.repeat(wl.commit.astype(bool), C), inputs=inp))
    # without the expectation the pass needs no dequantised copy
    b3 = runner.from_workload(wl, want_selfcond=False)
    runner.vocab_pass_fp8(b3, f, ws, seed, softcap=softcap)
    torch.cuda.synchronize()
    for key in ("lse", "entropy", "argmax_tok", "gumbel_tok"):
        x, y = getattr(b, key).cpu().numpy(), getattr(b3, key).cpu().numpy()
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), key


def test_fp8_full_size_batched():
    """V = 262144, d = 2816: quantiser rows against the oracle on a sample, and the FP8 pass on
    sampled rows against the oracle on the dequantised embedding, for 32 canvases and for one
    canvas."""
    from denoise_step_sampler_amd import runner
    _say("[vocab_pass_fp8] generating V=262144 d=2816 embedding")
    E = synth.make_embedding(262144, 2816, seed=0)
    wl = synth.workload("batched", E=E)
    V, d, n = wl.V, wl.d, wl.n_canvas
    f, codes, k = _quantize_gpu(E, V, d)
    sample = np.sort(np.random.default_rng(3).choice(V, 64, replace=False))
    q_ref, k_ref = of8.quantize_rows(ovp.widen_bf16(E[sample]))
    assert np.array_equal(codes[sample], q_ref) and np.array_equal(k[sample], k_ref)
    _say("    quantiser sample ok; running the 32-canvas pass")
    b = runner.from_workload(wl)
    ws = runner.fp8_workspace(n, V, d)
    runner.vocab_pass_fp8(b, f, ws, 5)
    torch.cuda.synchronize()
    # the embedding the pass computes with: the device codes dequantised by the oracle's decoder
    # (its 256 code values as a table, applied in row chunks to bound host memory)
    table = of8.e4m3_value(np.arange(256, dtype=np.uint8))
    Eq64 = np.empty((V, d), np.float64)
    for r0 in range(0, V, 16384):
        Eq64[r0:r0 + 16384] = table[codes[r0:r0 + 16384]] * np.exp2(
            k[r0:r0 + 16384].astype(np.float64))[:, None]
    rng = np.random.default_rng(4)
    canv = [0, 3, 6, 13, 31]     # 3 and 31 commit
    rows = np.sort(np.concatenate([c * C + rng.choice(C, 3, replace=False) for c in canv]))
    _against_oracle(b, wl, Eq64, rows, 5, label="32 canvases:")
    del b, ws
    wl1 = synth.workload("large_v", E=E)
    c1 = runner.from_workload(wl1)
    runner.vocab_pass_fp8(c1, f, runner.fp8_workspace(1, V, d), 7)
    torch.cuda.synchronize()
    _against_oracle(c1, wl1, Eq64, np.array([0, 5, 77, 128, 254]), 7, label="one canvas:")


# --- FP8 x FP8: hidden states quantised per row when the pass runs ----------------------------

def _dyn_reference(wl, E_codes, ke, rows, seed, softcap=None, want_sc=True):
    """The oracle on the dequantised rows (h~, E~) and the FP8 MFMA's logit bound."""
    from parity import fp8_logit_bound
    h_codes, kh, hq_bits = of8.activation_rows(wl.h)
    Eq = of8.dequantize_rows(E_codes, ke)
    T = np.repeat(wl.temperature, C)
    cm = np.repeat(wl.commit.astype(bool), C)
    st = np.repeat(wl.step, C)
    ref = ovp.vocab_pass_rows(Eq, hq_bits, rows, T, cm, seed, st, softcap=softcap,
                              want_sc=want_sc)
    inp = VocabInputs(E64=Eq, h_bits=hq_bits, temperature_row=T, step_row=st, seed=seed,
                      softcap=softcap)
    return ref, cm, inp, fp8_logit_bound(h_codes, kh, E_codes, ke)


@pytest.mark.parametrize("V,d,n,softcap", [(5000, 256, 3, None), (777, 384, 2, None),
                                           (129, 128, 1, None), (3000, 512, 2, 15.0),
                                           (300, 8192, 1, None)])
def test_fp8_dyn_parity(V, d, n, softcap):
    """The FP8 x FP8 pass against the oracle on the dequantised hidden states and embedding:
    statistics and expectation at the usual bars; tokens equal except where the oracle's
    margin lies within the FP8 MFMA's summation bound of the two candidates (those recomputed
    from exact sums and counted against a budget of 5 %).  d = 384 and 128 give an odd number
    of 128-wide K chunks, V = 129 a single ragged tile, d = 8192 the widest hidden state."""
    from denoise_step_sampler_amd import runner
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=V + d)
    wl.commit = (np.arange(n) % 3 == 1).astype(np.uint8)
    wl.temperature = np.linspace(0.7, 1.3, n).astype(np.float32)
    f, codes, k = _quantize_gpu(wl.E, V, d)
    seed = 0xD8
    _say(f"[vocab_pass_fp8_dyn] V={V} d={d} n={n} softcap={softcap}")
    b = runner.from_workload(wl, commit_any=True)
    ws = runner.fp8_workspace(n, V, d, activations=True)
    runner.vocab_pass_fp8(b, f, ws, seed, softcap=softcap, activations=True)
    torch.cuda.synchronize()
    rows = np.arange(n * C)
    ref, cm, inp, bound = _dyn_reference(wl, codes, k, rows, seed, softcap)
    rep = compare_vocab(_host(b), ref, cm, inputs=inp, logit_bound=bound,
                        max_exempt=max(2, int(0.05 * rows.size)))
    _say("   ", rep)


def test_fp8_dyn_full_size_sampled():
    """V = 262144, d = 2816: the FP8 x FP8 pass for 32 canvases and for one canvas on sampled
    rows against the oracle on the dequantised rows."""
    from denoise_step_sampler_amd import runner
    _say("[vocab_pass_fp8_dyn] generating V=262144 d=2816 embedding")
    E = synth.make_embedding(262144, 2816, seed=0)
    wl = synth.workload("batched", E=E)
    V, d, n = wl.V, wl.d, wl.n_canvas
    f, codes, k = _quantize_gpu(E, V, d)
    b = runner.from_workload(wl)
    runner.vocab_pass_fp8(b, f, runner.fp8_workspace(n, V, d, activations=True), 5,
                          activations=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    canv = [0, 3, 6, 13, 31]     # 3 and 31 commit
    rows = np.sort(np.concatenate([c * C + rng.choice(C, 3, replace=False) for c in canv]))
    ref, cm, inp, bound = _dyn_reference(wl, codes, k, rows, 5)
    _say("    32 canvases:", compare_vocab(_host(b, rows), ref, cm, inputs=inp, logit_bound=bound))
    del b
    wl1 = synth.workload("large_v", E=E)
    c1 = runner.from_workload(wl1)
    runner.vocab_pass_fp8(c1, f, runner.fp8_workspace(1, V, d, activations=True), 7,
                          activations=True)
    torch.cuda.synchronize()
    rows1 = np.array([0, 5, 77, 128, 254])
    ref1, cm1, inp1, bound1 = _dyn_reference(wl1, codes, k, rows1, 7)
    _say("    one canvas:", compare_vocab(_host(c1, rows1), ref1, cm1, inputs=inp1,
                                          logit_bound=bound1))
