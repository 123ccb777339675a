"""The remaining entry points under HIP graph capture: q_sample, the FP8 vocabulary pass, the
Lite sampler and the self-conditioning consumer queue only kernels on the caller's stream, so
one captured sequence of all four replays bit for bit like the same calls made eagerly (three
replays, the in-place state reset eagerly before each)."""
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


def _bits(x):
    x = x.cpu().numpy()
    return x.view(np.uint32) if x.dtype == np.float32 else x


def test_fp8_lite_ffw_q_sample_captured_in_a_hip_graph():
    from denoise_step_sampler_amd import binding as B
    from denoise_step_sampler_amd import runner
    n, V, d, F = 3, 5000, 256, 512
    _say(f"[graph] q_sample + vocab_pass_fp8 + lite_step + selfcond_input n={n} V={V} d={d} F={F}")
    wl = synth.workload("lite", V=V, d=d, n_canvas=n, seed=4)
    wl.commit = np.array([0, 0, 1], np.uint8)
    b = runner.from_workload(wl)
    f = runner.quantize_embedding_fp8(b.E, V, d)
    ws8 = runner.fp8_workspace(n, V, d)
    W = runner.ffw_weights(*synth.make_ffw_weights(d, F, seed=4))
    wsf = runner.ffw_workspace(n, d, F)
    s = runner.lite_state(n)
    x0 = torch.as_tensor(np.random.default_rng(4).integers(0, V, n * b.C, dtype=np.int32)).cuda()
    kappa = torch.tensor([0.2, 0.5, 0.9], dtype=torch.float32, device="cuda")
    xt = torch.full((n * b.C,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((n * b.C, d), 0x7FBF, dtype=torch.int16, device="cuda")  # bf16 NaN bits

    def reset():
        s.x.zero_()
        s.prev_argmax.fill_(-1)
        s.prev_conf.fill_(float("inf"))
        s.committed.zero_()
        s.stable_count.zero_()
        b.next_tokens.copy_(x0)

    def seq():
        st = torch.cuda.current_stream()
        B.dg_q_sample(x0, n, b.C, V, kappa, 11, xt, stream=st)
        runner.vocab_pass_fp8(b, f, ws8, 11, stream=st)
        runner.lite_step(b, s, 0.5, 2, 11, stream=st)
        runner.selfcond_input(b, W, out, wsf, stream=st)

    keys = {"xt": lambda: xt, "lse": lambda: b.lse, "entropy": lambda: b.entropy,
            "argmax": lambda: b.argmax_tok, "gumbel": lambda: b.gumbel_tok,
            "selfcond": lambda: b.selfcond, "x": lambda: s.x, "conf": lambda: s.conf,
            "committed": lambda: s.committed, "final": lambda: s.final_tokens,
            "converged": lambda: s.converged, "mean_entropy": lambda: s.mean_entropy,
            "stable": lambda: s.stable_count, "ffw_out": lambda: out}
    reset()
    seq()
    torch.cuda.synchronize()
    ref = {k: _bits(g()) for k, g in keys.items()}
    live = np.repeat(wl.commit == 0, b.C)                # commit canvases' rows are not written
    y = (out.cpu().numpy().astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
    assert np.isfinite(y[live]).all() and (out.cpu().numpy()[~live] == 0x7FBF).all()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        seq()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        seq()
    for rep in range(3):
        reset()
        for t in (b.lse, b.entropy, b.selfcond, s.conf, s.mean_entropy):
            t.fill_(float("nan"))
        out.fill_(0x7FBF)
        xt.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, g in keys.items():
            assert np.array_equal(_bits(g()), ref[k]), (rep, k)
    _say("    three replays bit-identical to the eager sequence")
