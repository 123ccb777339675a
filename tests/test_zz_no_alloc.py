"""The allocation-free vocabulary pass (dg_vocab_pass_ex_noalloc, the library's static per-GPU
scratch in place of a workspace) against dg_vocab_pass_ex with a workspace, through the C ABI:
two calls in a row on one GPU, the second on a smaller shape (fewer canvases, a smaller
vocabulary and width, a prepared fp16 embedding, a separate draw temperature and a soft cap),
each bit for bit equal to the workspace pass on the same inputs."""
import sys

import numpy as np
import pytest

from denoise_step_sampler_amd import synth

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


def _case(n, V, d, seed, prepared, draw, softcap):
    from denoise_step_sampler_amd import binding as B
    from denoise_step_sampler_amd import runner
    _say(f"[noalloc] n={n} V={V} d={d} prepared={prepared} draw={draw is not None} "
         f"softcap={softcap}")
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=seed)
    wl.commit = (np.arange(n) % 3 == 1).astype(np.uint8)
    E_t = runner.bf16_tensor(wl.E)
    E16 = runner.embedding_f16(E_t, V, d) if prepared else None
    need = B.dg_vocab_pass_ex_workspace_size(n, B.DG_CANVAS, V, d, prepared)
    assert 0 < need <= B.DG_NOALLOC_SCRATCH_BYTES
    a = runner.from_workload(wl, commit_any=True, E=E_t, E16=E16)
    dt = None if draw is None else torch.as_tensor(np.asarray(draw, np.float32)).cuda()
    B.dg_vocab_pass_ex(a.E, E16, a.h, n, a.C, V, d, a.temperature, dt, softcap, a.commit, seed,
                       a.step, a.lse, a.entropy, a.argmax_tok, a.gumbel_tok, a.selfcond,
                       a.workspace)
    # the same fills as the workspace pass's outputs (NaN, -7): the rows of committing canvases
    # keep them in both (only their argmax is written), every other element must be written
    # with the same bits
    R = a.R
    nan = float("nan")
    out = dict(lse=torch.full((R,), nan, device="cuda"),
               entropy=torch.full((R,), nan, device="cuda"),
               argmax_tok=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
               gumbel_tok=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
               selfcond=torch.full((R, d), nan, device="cuda"))
    B.dg_vocab_pass_ex_noalloc(a.E, E16, a.h, n, a.C, V, d, a.temperature, dt, softcap,
                               a.commit, seed, a.step, out["lse"], out["entropy"],
                               out["argmax_tok"], out["gumbel_tok"], out["selfcond"])
    torch.cuda.synchronize()
    live = np.repeat(wl.commit == 0, a.C)
    assert np.isfinite(out["lse"].cpu().numpy()[live]).all()
    assert np.isfinite(out["selfcond"].cpu().numpy()[live]).all()
    assert (out["argmax_tok"].cpu().numpy() >= 0).all()
    for k, y in out.items():
        x = getattr(a, k).cpu().numpy()
        y = y.cpu().numpy()
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), k
    _say("    identical outputs")


def test_noalloc_equals_the_workspace_pass_twice_then_smaller():
    _case(3, 5000, 256, 21, prepared=False, draw=None, softcap=0.0)
    _case(1, 1200, 128, 22, prepared=True, draw=[0.7], softcap=12.0)
