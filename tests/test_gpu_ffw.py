"""Parity of dg_selfcond_input (through the C ABI) with the fp64 oracle.

Bar (outputs are bf16): per element |delta| <= 2^-7 (|ref| + rms(ref row)), and per row
||delta|| <= 2^-8 ||ref||.  The kernels and the oracle round to bf16 at the same points (x1,
y, out); fp32 against fp64 arithmetic before a rounding can flip it by one ulp.  A flip at
the output is within 2^-7 |ref| (two half-ulps).  A flip of an x1 entry moves it by its ulp,
2^-5 for the largest entries (|x1| in [4, 8), x1 having rms ~1 after the pre-norm); it
reaches every output entry of the row through d y_j / d x1_k (weights ~ 1 / sqrt(D), GELU
slopes <= 1.13), the down projection (a sum of F such terms with weights ~ 1 / sqrt(F)) and
the final scaling (~ 1 / rms of the row): a gain of order 1 / sqrt(D) per entry, so
2^-5 / sqrt(128) < 2^-7 rms at the smallest width tested.  The row bound keeps the aggregate
to a quarter of the output's own rounding."""
import math
import sys

import numpy as np
import pytest

from denoise_step_sampler_amd import synth
from oracle import selfcond_ffw as of

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


def _compare(got_bits, ref, label):
    got = synth.bf16_to_f32(got_bits).astype(np.float64)
    err = np.abs(got - ref)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    ok = err <= 2.0 ** -7 * (np.abs(ref) + rms)
    rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    _say(f"    {label}: max elem err {err.max():.3g}, max row rel {rel.max():.3g}, "
         f"elements off by > half an ulp: {int((err > 2.0 ** -9 * np.abs(ref)).sum())}")
    if not ok.all():
        bad = np.argwhere(~ok)[:8]
        _say("    off:", [(int(r), int(c), float(got[r, c]), float(ref[r, c])) for r, c in bad])
    assert ok.all(), f"{label}: {int((~ok).sum())} elements off, first rows {np.nonzero(~ok)[0][:8]}"
    assert (rel <= 2.0 ** -8).all(), f"{label}: row error {rel.max()}"


def _run(n, V, D, F, seed, first_step=False, commit=None, rows=None, E=None, E_t=None,
         bad_tokens=None):
    from denoise_step_sampler_amd import binding as B
    from denoise_step_sampler_amd import runner
    _say(f"[selfcond_input] n={n} V={V} D={D} F={F} seed={seed} first={first_step}")
    R = n * C
    E = synth.make_embedding(V, D, seed=seed) if E is None else E
    sc, tok = synth.make_selfcond_rows(E, R, seed)
    if bad_tokens is not None:
        tok[bad_tokens] = np.array([-1, V] * len(bad_tokens))[:len(bad_tokens)]
    pre, Wg, Wu, Wd = synth.make_ffw_weights(D, F, seed)
    W = runner.ffw_weights(pre, Wg, Wu, Wd, eps=1e-6)
    E_t = runner.bf16_tensor(E) if E_t is None else E_t
    out = torch.full((R, D), 0x7FBF, dtype=torch.int16, device="cuda")
    ws = runner.ffw_workspace(n, D, F)
    cm_t = None if commit is None else torch.as_tensor(commit.astype(np.uint8)).cuda()
    B.dg_selfcond_input(None if first_step else torch.from_numpy(sc).cuda(),
                        torch.from_numpy(tok).cuda(), E_t, W.pre_norm, W.W_gate, W.W_up,
                        W.W_down, cm_t, n, C, V, D, F, 1e-6, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    rows = np.arange(R) if rows is None else np.asarray(rows)
    cm_row = None if commit is None else np.repeat(commit.astype(bool), C)
    ref = of.selfcond_input(None if first_step else sc, tok, E, pre, Wg, Wu, Wd,
                            commit_row=cm_row, eps=1e-6, rows=rows)
    return got[rows], ref, cm_row, rows


@pytest.mark.parametrize("n,V,D,F", [(1, 1000, 128, 64), (2, 500, 192, 192), (3, 3000, 256, 512),
                                     (1, 64, 320, 128)])
def test_selfcond_input_parity(n, V, D, F):
    """Tile tails in both products (D = 192 and 320 are not multiples of the 128-wide output
    tile of the down projection), several canvases."""
    got, ref, _, _ = _run(n, V, D, F, seed=n + D)
    _compare(got, ref, f"n={n} D={D} F={F}")


def test_selfcond_input_first_step_and_commit():
    """sc = NULL (first decode step: the plain normalised embedding) and a commit canvas whose
    rows stay untouched."""
    got, ref, _, _ = _run(2, 700, 256, 256, seed=4, first_step=True)
    _compare(got, ref, "first step")
    commit = np.array([0, 1, 0])
    got, ref, cm, rows = _run(3, 700, 256, 256, seed=5, commit=commit)
    assert np.all(got[cm] == 0x7FBF)
    _compare(got[~cm], ref[~cm], "with commit canvas")


def test_selfcond_input_bad_tokens_give_nan_rows():
    got, ref, _, _ = _run(1, 300, 128, 128, seed=6, bad_tokens=[3, 77])
    vals = synth.bf16_to_f32(got)
    assert np.all(np.isnan(vals[[3, 77]]))
    keep = np.setdiff1d(np.arange(C), [3, 77])
    _compare(got[keep], ref[keep], "valid rows")


def test_selfcond_input_full_size_sampled():
    """32 canvases, V = 262144, D = 2816, F = 2816 (the serving step's shape), sampled rows of
    every kind of tile position."""
    E = synth.make_embedding(262144, 2816, seed=0)
    from denoise_step_sampler_amd import runner
    E_t = runner.bf16_tensor(E)
    rows = np.array([0, 1, 127, 128, 255, 256, 4000, 4095, 4096, 6143, 8064, 8191])
    got, ref, _, _ = _run(32, 262144, 2816, 2816, seed=0, rows=rows, E=E, E_t=E_t)
    _compare(got, ref, "full size")


@pytest.mark.parametrize("D,F", [(16384, 128), (128, 65536)])
def test_selfcond_input_maximum_widths(D, F):
    """The largest widths the entry point accepts: D = 16384 and F = 65536."""
    got, ref, _, _ = _run(1, 97, D, F, seed=D % 97 + F % 89)
    _compare(got, ref, f"D={D} F={F}")
