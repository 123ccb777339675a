"""Benchmark of one denoising step of the hot path on one MI355X.

A step = dg_vocab_pass + dg_accept_renoise over one batch of canvases, inputs resident in
HBM.  Default workload: the batched serving step (32 canvases x 256 positions, V = 262144,
d = 2816, 8 canvases commit).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload batched|large_v|lite|tiny|full_loop] [--no-cpu-baseline]
                    [--graph] [--fp8 | --fp8-act] [--softcap C]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# the logits kernel's source and the headers it includes (the counters are void once any changes)
KERNEL_SRCS = [os.path.join(ROOT, "denoise_step_sampler_amd", "csrc", f)
               for f in ("vocab_gemm.hip", "dg_device.h", "dg_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_gemm_logits.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of k_gemm_logits from the committed counter summary, or None when
    there is none for this workload or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash(KERNEL_SRCS):
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else float(w["hbm_bytes_per_launch"])


def copy_probe(mb: int, reps: int) -> int:
    """A plain device copy of mb MiB, repeated: the calibration kernel for the HBM counters."""
    import torch
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "reps": reps}), flush=True)
    return 0


def algorithmic_flops(wl) -> float:
    """2 R V d for the logits of every row + 2 R_nc V d for the expectation of non-commit rows."""
    R = wl.R
    R_nc = int((wl.commit == 0).sum()) * wl.C
    return 2.0 * R * wl.V * wl.d + 2.0 * R_nc * wl.V * wl.d


def cpu_baseline(wl, gpu: dict, seed: int, step: int, budget_s: float = 20.0):
    """The fp64 oracle, untuned, on a bounded sample of rows of the same workload (the same
    seed and step as the GPU outputs in `gpu`), timed; and the comparison of those rows with
    the GPU's at the bars of the hot-path contract (tokens equal unless the oracle's margin is
    below 1e-4, lse / entropy / expectation rows within 2e-3)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import vocab_pass as ovp
    t0 = time.perf_counter()
    E64 = ovp.widen_bf16(wl.E)
    widen_s = time.perf_counter() - t0
    T = np.repeat(wl.temperature, wl.C)
    cm = np.repeat(wl.commit.astype(bool), wl.C)
    st = np.full(wl.R, step)
    nc_rows = np.nonzero(~cm)[0]
    # rows spread over the non-commit canvases, in a fixed shuffled order
    order = np.random.default_rng(12345).permutation(nc_rows.size)
    rows_done, spent, k = 0, 0.0, 0
    chunk = 4
    refs = []
    while spent < budget_s and k * chunk < nc_rows.size:
        rows = np.sort(nc_rows[order[k * chunk:(k + 1) * chunk]])
        t0 = time.perf_counter()
        refs.append(ovp.vocab_pass_rows(E64, wl.h, rows, T, cm, seed, st, want_sc=True))
        spent += time.perf_counter() - t0
        rows_done += rows.size
        k += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    cpu_model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    base = {"value": rows_done / spent, "unit": "canvas-positions/s", "cores": int(threads),
            "cpu_model": cpu_model, "kind": "oracle",
            "sample": f"{rows_done} non-commit positions (rows) of the {wl.name} workload, spread "
                      f"over its canvases, full vocabulary (logits, softmax, entropy, argmax, "
                      f"Gumbel, selfcond), fp64 numpy, {spent:.1f}s; bf16->fp64 widening of E "
                      f"({widen_s:.1f}s) excluded"}
    if gpu is None:
        return base, None
    # parity of the same rows
    rows = np.concatenate([r.rows for r in refs])
    cat = lambda f: np.concatenate([getattr(r, f) for r in refs])
    am, gm = cat("argmax"), cat("gumbel")
    mu_a, mu_g = cat("mu_argmax"), cat("mu_gumbel")
    ex_a, ex_g = mu_a < 1e-4, mu_g < 1e-4
    rel = lambda x, y: np.abs(x - y) / np.maximum(np.abs(y), 1e-30)
    sc_ref = np.concatenate([r.sc for r in refs])
    sc_got = gpu["selfcond"][rows].astype(np.float64)
    sc_rel = np.linalg.norm(sc_got - sc_ref, axis=1) / np.linalg.norm(sc_ref, axis=1)
    lse_rel = rel(gpu["lse"][rows].astype(np.float64), cat("lse"))
    h_ref = cat("entropy")
    h_err = np.abs(gpu["entropy"][rows].astype(np.float64) - h_ref)
    par = {"rows": int(rows.size),
           "argmax_equal": int((gpu["argmax"][rows] == am).sum()),
           "argmax_exempt": int(ex_a.sum()),
           "gumbel_equal": int((gpu["gumbel"][rows] == gm).sum()),
           "gumbel_exempt": int(ex_g.sum()),
           "lse_max_rel": float(lse_rel.max()),
           "entropy_max_rel": float((h_err / np.maximum(h_ref, 1e-30)).max()),
           "selfcond_max_rel": float(sc_rel.max())}
    par["within_bars"] = bool(
        np.all((gpu["argmax"][rows] == am) | ex_a) and np.all((gpu["gumbel"][rows] == gm) | ex_g)
        and np.all(lse_rel <= 2e-3) and np.all((h_err <= 2e-3 * h_ref) | (h_err <= 1e-6))
        and np.all(sc_rel <= 2e-3))
    return base, par


def full_loop(args) -> int:
    """The full denoise loop (8 canvases, 32 steps, a canvas committed once converged) with the
    hidden states synthesised on the GPU between steps, so that no host round trip sits inside
    the loop: value = canvas-positions of the non-converged canvases / GPU time of the steps
    (synthesis excluded)."""
    import numpy as np
    import torch

    from denoise_step_sampler_amd import runner, synth
    wl = synth.workload("full_loop", seed=args.seed)
    E_t = runner.bf16_tensor(wl.E)
    E16 = runner.embedding_f16(E_t, wl.V, wl.d)
    sched = None if args.anneal is None else tuple(float(x) for x in args.anneal.split(","))
    log("[bench] full loop: warmup")
    runner.run_loop_device(wl, args.seed, max_steps=max(1, args.warmup), E=E_t, E16=E16,
                           softcap=args.softcap)
    torch.cuda.synchronize()
    log("[bench] full loop: timed run")
    res = runner.run_loop_device(wl, args.seed, max_steps=32, E=E_t, E16=E16, schedule=sched,
                                 softcap=args.softcap)
    ms = float(np.mean(res.step_ms))
    flops = 4.0 * res.positions * wl.V * wl.d   # logits + expectation of the active canvases
    out = {
        "metric": "canvas-positions/sec per denoise step",
        "value": res.positions_per_s, "unit": "canvas-positions/s",
        "n_gpus": 1, "steps": res.steps_run, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full_loop", "n_canvas": wl.n_canvas, "C": wl.C, "V": wl.V,
                   "d": wl.d, "max_steps": 32,
                   "temperature": (float(wl.temperature[0]) if sched is None else
                                   {"anneal_from": sched[0], "anneal_to": sched[1]}),
                   "softcap": args.softcap,
                   "entropy_budget": wl.budget, "confidence": wl.confidence,
                   "stability": wl.stability,
                   "hidden_states": "synthesised on the GPU between steps (not timed)"},
        "pct_bf16_mfma_peak": 100.0 * flops / (sum(res.step_ms) * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "step_ms_p10_p50_p90": [float(x) for x in np.percentile(res.step_ms, [10, 50, 90])],
        "steps_to_converge": res.steps_to_converge.tolist(),
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="batched")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB MiB (counter calibration)")
    ap.add_argument("--fp8", action="store_true",
                    help="run the step on the FP8 form of the embedding (dg_vocab_pass_fp8)")
    ap.add_argument("--fp8-act", action="store_true",
                    help="FP8 embedding and hidden states quantised per row in the pass, FP8 x "
                         "FP8 MFMA (dg_vocab_pass_fp8_dyn); implies --fp8")
    ap.add_argument("--softcap", type=float, default=None,
                    help="final-logit soft cap c (logits c tanh(S / c)); default: none")
    ap.add_argument("--ffw-F", type=int, default=2816, metavar="F",
                    help="hidden width of the self-conditioning MLP timed beside the step "
                         "(0: skip)")
    ap.add_argument("--anneal", default=None, metavar="TMAX,TMIN",
                    help="full_loop only: linear temperature schedule over the 32 steps")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as a captured HIP graph (the step counter advanced by a "
                         "kernel inside it), one replay per step, instead of eager launches")
    args = ap.parse_args()
    args.fp8 = args.fp8 or args.fp8_act
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the vocabulary pass would shard by canvas or by vocabulary range)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from denoise_step_sampler_amd import runner, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        return copy_probe(args.copy_probe, 5)
    if args.workload == "full_loop":
        return full_loop(args)
    log(f"[bench] building inputs for workload {args.workload}")
    wl = synth.workload(args.workload, seed=args.seed)
    E_t = runner.bf16_tensor(wl.E)
    # the fp16 embedding the expectation multiplies, prepared once per embedding
    # (as the FP8 codes are), outside the timed region
    E16 = runner.embedding_f16(E_t, wl.V, wl.d)
    b = runner.from_workload(wl, E=E_t, E16=E16)
    stream = torch.cuda.current_stream()
    seed = args.seed
    if args.fp8:
        f8 = runner.quantize_embedding_fp8(b.E, wl.V, wl.d, stream=stream)
        ws8 = runner.fp8_workspace(wl.n_canvas, wl.V, wl.d, activations=args.fp8_act)

    def vocab(k_stream):
        if args.fp8:
            runner.vocab_pass_fp8(b, f8, ws8, seed, k_stream, args.softcap,
                                  activations=args.fp8_act)
        else:
            runner.vocab_pass(b, seed, k_stream, args.softcap)

    def step(k):
        b.step.fill_(k)
        vocab(stream)
        runner.accept_renoise(b, wl.budget, wl.confidence, wl.stability, seed, stream)

    log(f"[bench] warmup {args.warmup}")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # timed region: whole steps, plus per-launch events around the vocabulary pass
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for k in range(args.steps):
        b.step.fill_(args.warmup + k)
        ev[k][0].record(stream)
        vocab(stream)
        ev[k][1].record(stream)
        runner.accept_renoise(b, wl.budget, wl.confidence, wl.stability, seed, stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    vp_ms = [a.elapsed_time(z) for a, z in ev]
    vp_avg = float(np.mean(vp_ms))
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (wall {wall:.3f}s), "
        f"vocab pass {vp_avg:.3f} ms (min {min(vp_ms):.3f})")
    eager_ms_step = ms_step
    if args.graph:
        # the same step captured once (the entry points queue only kernels: no allocation,
        # memset or synchronisation) and replayed; a kernel inside advances the step counter
        def graph_step():
            cur = torch.cuda.current_stream()
            b.step.add_(1)
            vocab(cur)
            runner.accept_renoise(b, wl.budget, wl.confidence, wl.stability, seed, cur)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            graph_step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            graph_step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        ms_step = g0.elapsed_time(g1) / args.steps
        log(f"[bench] {args.steps} graph replays: {ms_step:.3f} ms/step "
            f"(eager launches: {eager_ms_step:.3f})")

    # the dominant kernel, k_gemm_logits (logits + epilogue, 2 R V d flops): the same pass
    # without the expectation runs it plus two small kernels (canvas order, row statistics),
    # timed the same way on the same stream
    from denoise_step_sampler_amd import binding as B
    ev2 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for k in range(args.steps):
        ev2[k][0].record(stream)
        if args.fp8:
            fn = B.dg_vocab_pass_fp8_dyn if args.fp8_act else B.dg_vocab_pass_fp8
            fn(f8.codes, f8.E16, f8.row_exp, b.h, b.n_canvas, b.C, b.V, b.d, b.temperature,
               b.commit, seed, b.step, b.lse, b.entropy, b.argmax_tok, b.gumbel_tok, None, ws8,
               stream=stream, softcap=args.softcap or 0.0)
        else:
            B.dg_vocab_pass_ex(b.E, b.E16, b.h, b.n_canvas, b.C, b.V, b.d, b.temperature, None,
                               args.softcap or 0.0, b.commit, seed, b.step, b.lse, b.entropy,
                               b.argmax_tok, b.gumbel_tok, None, b.workspace, stream=stream)
        ev2[k][1].record(stream)
    torch.cuda.synchronize()
    k1_ms = float(np.mean([a.elapsed_time(z) for a, z in ev2]))
    log(f"[bench] logits kernel (pass without the expectation): {k1_ms:.3f} ms")

    # the self-conditioning consumer (f2): the next step's input rows from this step's sc and
    # renoised tokens, timed alone (it is not part of the step above)
    ffw = None
    if args.ffw_F > 0:
        W = runner.ffw_weights(*synth.make_ffw_weights(wl.d, args.ffw_F, seed))
        x_next = torch.empty((wl.R, wl.d), dtype=torch.int16, device=dev)
        ws_f = runner.ffw_workspace(wl.n_canvas, wl.d, args.ffw_F)
        for _ in range(2):
            runner.selfcond_input(b, W, x_next, ws_f, stream=stream)
        ev3 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            ev3[k][0].record(stream)
            runner.selfcond_input(b, W, x_next, ws_f, stream=stream)
            ev3[k][1].record(stream)
        torch.cuda.synchronize()
        f_ms = float(np.mean([a.elapsed_time(z) for a, z in ev3]))
        R_nc = int((wl.commit == 0).sum()) * wl.C
        f_flops = 6.0 * R_nc * wl.d * args.ffw_F
        ffw = {"F": args.ffw_F, "avg_launch_ms": f_ms, "algorithmic_flops": f_flops,
               "achieved_tflops": f_flops / (f_ms * 1e-3) / 1e12,
               "frac_bf16_peak": f_flops / (f_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)}
        log(f"[bench] self-conditioning input (F={args.ffw_F}): {f_ms:.3f} ms")

    # the latency-bound pieces, timed alone: accept/renoise of this batch, and q_sample on the
    # 64 x 256 training-corruption shape (V = 50,257)
    def timed(fn, reps=20):
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        torch.cuda.synchronize()
        for a, z in evs:
            a.record(stream)
            fn()
            z.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(z) for a, z in evs]

    ar_ms = timed(lambda: runner.accept_renoise(b, wl.budget, wl.confidence, wl.stability, seed,
                                                stream))
    qw = synth.qsample_workload()
    x0_t = torch.from_numpy(qw.x0).to(dev)
    kap_t = torch.from_numpy(qw.kappa).to(dev)
    xt_t = torch.empty_like(x0_t)
    qs_ms = timed(lambda: B.dg_q_sample(x0_t, qw.n_canvas, 256, qw.V, kap_t, seed, xt_t,
                                        stream=stream))

    flops = algorithmic_flops(wl)
    flops_k1 = 2.0 * wl.R * wl.V * wl.d
    ach_k1 = flops_k1 / (k1_ms * 1e-3) / 1e12
    # the logits contraction's own dtype sets its peak (FP8 x FP8 with --fp8-act)
    peak_k1 = PEAK_FP8_TFLOPS if args.fp8_act else PEAK_BF16_TFLOPS
    positions = wl.R
    res = {
        "metric": "canvas-positions/sec per denoise step",
        "value": positions / (ms_step * 1e-3),
        "unit": "canvas-positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 logits, fp16 expectation" if args.fp8_act else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "n_canvas": wl.n_canvas, "C": wl.C, "V": wl.V,
                   "d": wl.d, "commit_canvases": int(wl.commit.sum()),
                   "temperature": float(wl.temperature[0]), "entropy_budget": wl.budget,
                   "softcap": args.softcap,
                   "embedding": (("fp8-e4m3, power-of-two row scales"
                                  + (", hidden states quantised per row in the pass"
                                     if args.fp8_act else "")) if args.fp8 else "bf16")
                   + "; its fp16 copy for the expectation prepared once, untimed",
                   "caches": "warm: no L2 / MALL flush between steps",
                   "launch": ("one HIP graph replay per step (eager launches: "
                              f"{eager_ms_step:.3f} ms/step)") if args.graph
                   else "eager launches on one stream"},
        "pct_bf16_mfma_peak": 100.0 * flops / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "e_stream_hbm_frac": (2.0 * wl.V * wl.d) / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "vocab_pass": {"avg_launch_ms": vp_avg, "algorithmic_flops": flops,
                       "achieved_tflops": flops / (vp_avg * 1e-3) / 1e12,
                       "p10_p50_p90_ms": [float(x) for x in np.percentile(vp_ms, [10, 50, 90])]},
        "accept_renoise": {"median_us": 1e3 * float(np.median(ar_ms)),
                           "p10_p90_us": [1e3 * float(x) for x in np.percentile(ar_ms, [10, 90])]},
        "q_sample": {"shape": f"{qw.n_canvas}x256, V={qw.V}",
                     "median_us": 1e3 * float(np.median(qs_ms)),
                     "tokens_per_s": qw.n_canvas * 256 / (float(np.median(qs_ms)) * 1e-3)},
        "roofline": {
            "kernel": "k_gemm_logits",
            "bound": "mfma", "achieved": ach_k1, "peak": peak_k1,
            "unit": "TFLOP/s", "frac": ach_k1 / peak_k1,
            # the counters were taken on the uncapped kernel
            "traffic": (measured_traffic(args.workload)
                        if args.softcap is None and not args.fp8 else None),
            "algorithmic_flops_per_launch": flops_k1, "avg_launch_ms": k1_ms},
    }
    if ffw is not None:
        res["selfcond_input"] = ffw
    if not args.no_cpu_baseline:
        # one more full step at a known step id, its outputs compared with the oracle's rows
        # (on the FP8 embedding the pass computes with other values than E: not compared)
        step(0)
        torch.cuda.synchronize()
        gpu = None if args.fp8 else {
            "lse": b.lse.cpu().numpy(), "entropy": b.entropy.cpu().numpy(),
            "argmax": b.argmax_tok.cpu().numpy(), "gumbel": b.gumbel_tok.cpu().numpy(),
            "selfcond": b.selfcond.cpu().numpy()}
        log(f"[bench] cpu baseline (~{args.cpu_seconds:.0f}s of oracle work)")
        res["cpu_baseline"], par = cpu_baseline(wl, gpu, seed, 0, args.cpu_seconds)
        if par is not None:
            res["parity_sample"] = par
            log(f"[bench] parity of the sampled rows: {par}")
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
