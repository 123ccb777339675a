"""The FP8 embedding through the C ABI: the quantiser's codes and exponents bit for bit against
the oracle's, the vocabulary pass on the FP8 embedding against the oracle's pass on the
oracle's dequantised rows, and agreement with dg_vocab_pass on those rows (the power-of-two
scales make the dequantised rows exact bf16 numbers; the logits pass on the codes sums the
K positions of a chunk in another order, so the two agree to fp32 accumulation rounding)."""

import sys

import numpy as np
import pytest

from denoise_step_sampler_amd import synth
from oracle import fp8 as of8
from oracle import vocab_pass as ovp
from parity import compare_vocab

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


def _agree(a, b, nc):
    """Two passes over the same embedding values: tokens equal but for near-ties, statistics
    within fp32 accumulation rounding, expectation rows within the 2e-3 bar."""
    am = a.argmax_tok.cpu().numpy() == b.argmax_tok.cpu().numpy()
    gm = (a.gumbel_tok.cpu().numpy() == b.gumbel_tok.cpu().numpy())[nc]
    assert am.mean() > 0.999 and gm.mean() > 0.99, (am.mean(), gm.mean())
    for key in ("lse", "entropy"):
        x, y = getattr(a, key).cpu().numpy()[nc], getattr(b, key).cpu().numpy()[nc]
        assert np.allclose(x, y, rtol=1e-4, atol=1e-6), key
    if a.selfcond is not None:
        x, y = a.selfcond.cpu().numpy()[nc], b.selfcond.cpu().numpy()[nc]
        rel = np.linalg.norm(x - y, axis=1) / np.linalg.norm(y, axis=1)
        assert rel.max() < 2e-3, rel.max()
    return float(am.mean()), float(gm.mean())


def _special_embedding(V, d, seed):
    E = synth.bf16_to_f32(synth.make_embedding(V, d, seed=seed)).copy()
    E[0] = 0.0                                        # zero row: exponent floor
    E[1] *= 2.0 ** -100                               # tiny row
    E[2] *= 2.0 ** 40                                 # large row
    E[3, :6] = [448.0, 1.0625, 1.1875, -3.0 * 2.0 ** -10, 2.0 ** -10, -448.0]  # ties, k = 0
    E[3, 6:] = 0.5
    E[4] = np.where(np.arange(d) % 2, 224.0, -1e-3)   # |max| exactly 224: k = -1
    return synth.round_to_bf16(E.astype(np.float32))


def _quantize_gpu(E_bits, V, d, transposed=True):
    from denoise_step_sampler_amd import runner
    E_t = runner.bf16_tensor(E_bits)
    f = runner.quantize_embedding_fp8(E_t, V, d, transposed=transposed)
    torch.cuda.synchronize()
    return f, f.codes.cpu().numpy().reshape(V, d), f.row_exp.cpu().numpy()


def test_quantizer_bit_exact():
    V, d = 3000, 256
    E = _special_embedding(V, d, 4)
    _, codes, k = _quantize_gpu(E, V, d)
    q_ref, k_ref = of8.quantize_rows(ovp.widen_bf16(E))
    assert np.array_equal(k, k_ref), np.nonzero(k != k_ref)[0][:8]
    bad = np.argwhere(codes != q_ref)
    assert bad.size == 0, [(int(r), int(c), int(codes[r, c]), int(q_ref[r, c])) for r, c in bad[:8]]
    # the transposed codes: [d][pitch], zero past V
    f, _, _ = _quantize_gpu(E, V, d)
    pitch = (V + 255) // 256 * 256
    qT = f.codesT.cpu().numpy().reshape(d, pitch)
    assert np.array_equal(qT[:, :V], q_ref.T) and np.all(qT[:, V:] == 0)


@pytest.mark.parametrize("softcap,transposed", [(None, True), (15.0, True), (None, False)])
def test_fp8_vocab_pass_parity_and_bf16_identity(softcap, transposed):
    """The pass on the codes (transposed codes for the expectation, or its dequantised copy)
    against the oracle on the dequantised rows and against the bf16 pass on them."""
    from denoise_step_sampler_amd import runner
    V, d, n = 5000, 256, 3
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=9)
    wl.commit = np.array([0, 1, 0], np.uint8)
    wl.temperature = np.array([0.5, 0.8, 1.1], np.float32)
    f, codes, k = _quantize_gpu(wl.E, V, d, transposed)
    q_ref, k_ref = of8.quantize_rows(ovp.widen_bf16(wl.E))
    assert np.array_equal(codes, q_ref) and np.array_equal(k, k_ref)
    Eq = of8.dequantize_rows(q_ref, k_ref)              # the oracle's dequantised rows
    Eq_bits = synth.round_to_bf16(Eq.astype(np.float32))
    assert np.array_equal(ovp.widen_bf16(Eq_bits), Eq)  # exact in bf16
    seed = 0xF8
    _say(f"[vocab_pass_fp8] softcap={softcap} transposed={transposed} n={n} V={V} d={d}")
    b = runner.from_workload(wl)
    ws = runner.fp8_workspace(n, V, d)
    runner.vocab_pass_fp8(b, f, ws, seed, softcap=softcap)
    torch.cuda.synchronize()
    rows = np.arange(n * C)
    ref = ovp.vocab_pass_rows(Eq, wl.h, rows, np.repeat(wl.temperature, C),
                              np.repeat(wl.commit.astype(bool), C), seed, np.repeat(wl.step, C),
                              softcap=softcap)
    out = {"lse": b.lse.cpu().numpy(), "entropy": b.entropy.cpu().numpy(),
           "argmax": b.argmax_tok.cpu().numpy(), "gumbel": b.gumbel_tok.cpu().numpy(),
           "sc": b.selfcond.cpu().numpy()}
    _say("   ", compare_vocab(out, ref, np.repeat(wl.commit.astype(bool), C)))
    # the bf16 pass on the dequantised rows
    b2 = runner.from_workload(wl, E=runner.bf16_tensor(Eq_bits))
    runner.vocab_pass(b2, seed, softcap=softcap)
    torch.cuda.synchronize()
    _say("    agreement with the bf16 pass:", _agree(b, b2, np.repeat(wl.commit == 0, C)))
    # without the expectation the pass needs no dequantised copy
    b3 = runner.from_workload(wl, want_selfcond=False)
    runner.vocab_pass_fp8(b3, f, ws, seed, softcap=softcap)
    torch.cuda.synchronize()
    for key in ("lse", "entropy", "argmax_tok", "gumbel_tok"):
        x, y = getattr(b, key).cpu().numpy(), getattr(b3, key).cpu().numpy()
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), key


def test_fp8_full_size_batched():
    """V = 262144, d = 2816: quantiser rows against the oracle on a sample, and the FP8 pass
    against the bf16 pass on the dequantised rows, for 32 canvases (expectation on the
    dequantised copy) and for one canvas (expectation on the transposed codes)."""
    from denoise_step_sampler_amd import runner
    _say("[vocab_pass_fp8] generating V=262144 d=2816 embedding")
    E = synth.make_embedding(262144, 2816, seed=0)
    wl = synth.workload("batched", E=E)
    V, d, n = wl.V, wl.d, wl.n_canvas
    f, codes, k = _quantize_gpu(E, V, d)
    sample = np.sort(np.random.default_rng(3).choice(V, 64, replace=False))
    q_ref, k_ref = of8.quantize_rows(ovp.widen_bf16(E[sample]))
    assert np.array_equal(codes[sample], q_ref) and np.array_equal(k[sample], k_ref)
    _say("    quantiser sample ok; running both passes")
    b = runner.from_workload(wl)
    ws = runner.fp8_workspace(n, V, d)
    runner.vocab_pass_fp8(b, f, ws, 5)
    torch.cuda.synchronize()
    # dequantised rows of the device codes, decoded on the host
    vals = of8.e4m3_value(np.arange(256, dtype=np.uint8))
    vals[np.isnan(vals)] = 0.0
    Eq = (vals.astype(np.float32)[codes] * np.exp2(k.astype(np.float32))[:, None])
    b2 = runner.from_workload(wl, E=runner.bf16_tensor(synth.round_to_bf16(Eq)))
    del Eq
    runner.vocab_pass(b2, 5)
    torch.cuda.synchronize()
    _say("    agreement with the bf16 pass:", _agree(b, b2, np.repeat(wl.commit == 0, C)))
    # one canvas: the expectation pass streams the transposed codes
    E_q = b2.E
    del b, b2
    wl1 = synth.workload("large_v", E=E)
    c1 = runner.from_workload(wl1)
    runner.vocab_pass_fp8(c1, f, runner.fp8_workspace(1, V, d), 7)
    c2 = runner.from_workload(wl1, E=E_q)
    runner.vocab_pass(c2, 7)
    torch.cuda.synchronize()
    _say("    one canvas, streamed codes:", _agree(c1, c2, np.ones(C, bool)))
