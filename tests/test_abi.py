"""The C-ABI library loads without a GPU, exports every symbol include/dg.h declares, and
rejects invalid arguments on the host before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "denoise_step_sampler_amd", "libdg.so")
HDR = os.path.join(ROOT, "include", "dg.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdg.so not built")


def _declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_0-9]+)\s*\(", text)))


def _lib():
    import torch  # noqa: F401  (share torch's HIP runtime)
    from denoise_step_sampler_amd import binding
    return binding.load(LIB)


def test_header_symbols_exported():
    decl = _declared()
    assert set(decl) == {"dg_vocab_pass_workspace_size", "dg_vocab_pass_ex_workspace_size",
                         "dg_embedding_f16_bytes", "dg_embedding_f16", "dg_vocab_pass",
                         "dg_vocab_pass_softcap", "dg_vocab_pass_ex", "dg_vocab_pass_ex_noalloc",
                         "dg_accept_renoise",
                         "dg_q_sample",
                         "dg_selfcond_input_workspace_size", "dg_selfcond_input",
                         "dg_lite_step", "dg_quantize_embedding_fp8",
                         "dg_vocab_pass_fp8_workspace_size", "dg_vocab_pass_fp8",
                         "dg_vocab_pass_fp8_dyn_workspace_size", "dg_vocab_pass_fp8_dyn",
                         "dg_status_string", "dg_last_error"}
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [s for s in decl if s not in exported]
    assert not missing, missing
    lib = _lib()
    for s in decl:
        assert hasattr(lib, s)


def test_workspace_size_pure_host():
    lib = _lib()
    f = lib.dg_vocab_pass_workspace_size
    # the FP8 x FP8 pass adds the quantised hidden states (codes and exponents, 256-aligned)
    dyn, f8 = lib.dg_vocab_pass_fp8_dyn_workspace_size, lib.dg_vocab_pass_fp8_workspace_size
    for n, V, d in ((1, 4096, 256), (3, 5000, 384), (32, 262144, 2816)):
        R = 256 * n
        assert dyn(n, 256, V, d) == f8(n, 256, V, d) + (R * d + 255) // 256 * 256 + \
            (4 * R + 255) // 256 * 256
    assert dyn(1, 256, 4096, 192) == 0
    assert f(1, 256, 4096, 256) > 0
    assert f(32, 256, 262144, 2816) > f(1, 256, 262144, 2816) > 0
    assert f(1, 128, 4096, 256) == 0      # C != 256
    assert f(1, 256, 4096, 96) == 0       # d % 128
    assert f(1, 256, 4096, 192) == 0      # d % 128
    assert f(1, 256, (1 << 26) + 1, 256) == 0
    g = lib.dg_vocab_pass_ex_workspace_size
    # a caller-prepared fp16 embedding needs no room in the workspace
    assert f(2, 256, 4096, 256) - g(2, 256, 4096, 256, 1) == lib.dg_embedding_f16_bytes(4096, 256)
    assert g(2, 256, 4096, 256, 0) == f(2, 256, 4096, 256)
    assert lib.dg_embedding_f16_bytes(4096, 256) == 256 * 4096 * 2
    assert lib.dg_embedding_f16_bytes(4000, 256) == 256 * 4096 * 2   # padded to whole tiles
    assert lib.dg_embedding_f16_bytes(4096, 192) == 0
    assert f(0, 256, 4096, 256) == 0
    assert f(1, 256, 0, 256) == 0
    assert f(1, 256, 4096, 8192 + 64) == 0


def _vp(lib, **kw):
    args = dict(E=1 << 20, h=1 << 20, n=1, C=256, V=4096, d=256, T=1 << 20, commit=None, seed=0,
                step=1 << 20, lse=None, H=1 << 20, am=1 << 20, gm=1 << 20, sc=None, ws=1 << 20,
                wsb=1 << 40, stream=None)
    args.update(kw)
    return lib.dg_vocab_pass(args["E"], args["h"], args["n"], args["C"], args["V"], args["d"],
                             args["T"], args["commit"], args["seed"], args["step"], args["lse"],
                             args["H"], args["am"], args["gm"], args["sc"], args["ws"],
                             args["wsb"], args["stream"])


def test_vocab_pass_validation_errors():
    """Every case fails validation, so no pointer is dereferenced and no kernel is queued."""
    from denoise_step_sampler_amd.binding import (DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED,
                                                  DG_ERR_WORKSPACE)
    lib = _lib()
    assert _vp(lib, E=None) == DG_ERR_INVALID_ARG
    assert _vp(lib, H=None) == DG_ERR_INVALID_ARG
    assert _vp(lib, C=128) == DG_ERR_UNSUPPORTED
    assert b"C=128" in lib.dg_last_error()
    assert _vp(lib, d=96) == DG_ERR_UNSUPPORTED
    assert _vp(lib, d=192) == DG_ERR_UNSUPPORTED
    assert _vp(lib, n=0) == DG_ERR_INVALID_ARG
    assert _vp(lib, V=0) == DG_ERR_INVALID_ARG
    assert _vp(lib, E=(1 << 20) + 2) == DG_ERR_INVALID_ARG          # misaligned
    assert _vp(lib, ws=None) == DG_ERR_WORKSPACE
    assert _vp(lib, wsb=16) == DG_ERR_WORKSPACE
    assert b"needed" in lib.dg_last_error()
    assert lib.dg_status_string(DG_ERR_WORKSPACE) == b"workspace too small"


def test_accept_and_qsample_validation_errors():
    from denoise_step_sampler_amd.binding import DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED
    lib = _lib()
    P = 1 << 20

    def ar(**kw):
        a = dict(H=P, am=P, gm=P, commit=None, n=1, C=256, V=100, budget=4.0, conf=0.1, thr=1,
                 seed=0, step=P, prev=P, cnt=P, nxt=P, acc=None, conv=P, mean=None)
        a.update(kw)
        return lib.dg_accept_renoise(a["H"], a["am"], a["gm"], a["commit"], a["n"], a["C"], a["V"],
                                     a["budget"], a["conf"], a["thr"], a["seed"], a["step"],
                                     a["prev"], a["cnt"], a["nxt"], a["acc"], a["conv"], a["mean"],
                                     None)
    assert ar(budget=-1.0) == DG_ERR_INVALID_ARG
    assert ar(budget=float("nan")) == DG_ERR_INVALID_ARG
    assert ar(budget=float("inf")) == DG_ERR_INVALID_ARG
    assert ar(conf=float("nan")) == DG_ERR_INVALID_ARG
    assert ar(thr=0) == DG_ERR_INVALID_ARG
    assert ar(prev=None) == DG_ERR_INVALID_ARG
    assert ar(C=255) == DG_ERR_UNSUPPORTED
    assert ar(V=0) == DG_ERR_INVALID_ARG
    q = lib.dg_q_sample
    assert q(P, 1, 256, 10, P, 0, P, None) == DG_ERR_INVALID_ARG     # xt aliases x0
    assert q(P, 1, 256, 10, None, 0, P + 4096, None) == DG_ERR_INVALID_ARG
    assert q(P, 1, 256, 0, P, 0, P + 4096, None) == DG_ERR_INVALID_ARG
    assert q(P, 5000, 256, 10, P, 0, P + 4096, None) == DG_ERR_INVALID_ARG


def test_binding_refuses_missing_library(tmp_path):
    import torch  # noqa: F401
    from denoise_step_sampler_amd import binding
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="no CPU fallback"):
            binding.load(str(tmp_path / "absent.so"))
    finally:
        binding._lib = saved


def test_softcap_value_rejected_on_host():
    """A soft cap that is not finite and > 0 is refused before any device work."""
    import ctypes
    lib = _lib()
    f = lib.dg_vocab_pass_softcap
    P = ctypes.c_void_p
    f.argtypes = [P, P] + [ctypes.c_int] * 4 + [P, P, ctypes.c_uint64] + [P] * 7 + \
        [ctypes.c_size_t, P, ctypes.c_float]
    f.restype = ctypes.c_int
    lib.dg_last_error.restype = ctypes.c_char_p
    for c in (0.0, -2.0, float("inf"), float("nan")):
        st = f(None, None, 1, 256, 4096, 256, None, None, 0, None, None, None, None, None, None,
               None, 0, None, c)
        assert st == 1, c
        assert b"softcap" in lib.dg_last_error()


def test_selfcond_input_workspace_and_validation_on_host():
    """Workspace sizes of the self-conditioning consumer and its host-side refusals."""
    import ctypes
    lib = _lib()
    ws = lib.dg_selfcond_input_workspace_size
    ws.restype = ctypes.c_size_t
    R, D, F = 2 * 256, 256, 512
    n = ws(2, 256, D, F)
    assert n >= R * D * 2 + R * F * 2 + R * D * 4 and n % 256 == 0
    assert ws(2, 128, D, F) == 0          # C != 256
    assert ws(2, 256, 96, F) == 0         # D % 64
    assert ws(2, 256, D, 100) == 0        # F % 64
    assert ws(0, 256, D, F) == 0
    f = lib.dg_selfcond_input
    P = ctypes.c_void_p
    f.argtypes = [P] * 8 + [ctypes.c_int] * 5 + [ctypes.c_float, P, P, ctypes.c_size_t, P]
    f.restype = ctypes.c_int
    lib.dg_last_error.restype = ctypes.c_char_p
    dummy = 4096  # never dereferenced: validation fails first
    # eps < 0
    assert f(None, dummy, dummy, None, None, None, None, None, 1, 256, 100, 64, 64, -1.0,
             dummy, dummy, 1 << 30, None) == 1
    # MLP weights missing while sc is given
    assert f(dummy, dummy, dummy, None, None, None, None, None, 1, 256, 100, 64, 64, 1e-6,
             dummy, dummy, 1 << 30, None) == 1
    assert b"weights" in lib.dg_last_error()
    # workspace too small
    assert f(None, dummy, dummy, None, None, None, None, None, 1, 256, 100, 64, 64, 1e-6,
             dummy, dummy, 16, None) == 3


def test_vocab_pass_ex_refusals_on_host():
    """dg_vocab_pass_ex refuses a bad soft cap, and a draw temperature on a width the two-GEMM
    path does not tile, before any device work; the binding declares the symbol."""
    from denoise_step_sampler_amd import binding
    lib = _lib()
    assert "dg_vocab_pass_ex" in binding.EXPORTED
    f = lib.dg_vocab_pass_ex
    P = 1 << 20
    for c in (-1.0, float("inf"), float("nan")):
        st = f(P, P, P, 1, 256, 4096, 256, P, P, c, None, 0, P, None, P, P, P, None, P, 1 << 40,
               None)
        assert st == binding.DG_ERR_INVALID_ARG, c
        assert b"softcap" in lib.dg_last_error()
    st = f(P, P, P, 1, 256, 4096, 192, P, P, 0.0, None, 0, P, None, P, P, P, None, P, 1 << 40,
           None)
    assert st == binding.DG_ERR_UNSUPPORTED
    assert b"128" in lib.dg_last_error()
    st = f(P, P, P, 1, 256, 4096, 256, None, P, 0.0, None, 0, P, None, P, P, P, None, P, 1 << 40,
           None)
    assert st == binding.DG_ERR_INVALID_ARG       # temperature is required
    st = f(P, P + 8, P, 1, 256, 4096, 256, P, None, 0.0, None, 0, P, None, P, P, P, P, P,
           1 << 40, None)
    assert st == binding.DG_ERR_INVALID_ARG       # E16 misaligned
    e = lib.dg_embedding_f16
    assert e(P, 4096, 192, P, None) == binding.DG_ERR_UNSUPPORTED
    assert e(None, 4096, 256, P, None) == binding.DG_ERR_INVALID_ARG
    assert e(P, 0, 256, P, None) == binding.DG_ERR_INVALID_ARG


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """dg_vocab_pass_ex_noalloc refuses, on the host and before any device call, a shape whose
    workspace exceeds the static scratch, and a bad soft cap; a shape within it passes the
    size check (the library's static scratch is 64 MiB, the binding states the same)."""
    from denoise_step_sampler_amd import binding
    lib = _lib()
    assert binding.DG_NOALLOC_SCRATCH_BYTES == 64 << 20
    f = lib.dg_vocab_pass_ex_noalloc
    g = lib.dg_vocab_pass_ex_workspace_size
    P = 1 << 20
    big = (32, 256, 262144, 2816)
    assert g(*big, 0) > binding.DG_NOALLOC_SCRATCH_BYTES
    st = f(P, None, P, *big, P, None, 0.0, None, 0, P, None, P, P, P, P, None)
    assert st == binding.DG_ERR_WORKSPACE
    assert b"static scratch" in lib.dg_last_error()
    # with a prepared fp16 embedding the same shape still needs far more than the scratch
    st = f(P, P, P, *big, P, None, 0.0, None, 0, P, None, P, P, P, P, None)
    assert st == binding.DG_ERR_WORKSPACE
    st = f(P, None, P, 1, 256, 4096, 256, P, None, -1.0, None, 0, P, None, P, P, P, P, None)
    assert st == binding.DG_ERR_INVALID_ARG and b"softcap" in lib.dg_last_error()
    st = f(None, None, P, 1, 256, 4096, 256, P, None, 0.0, None, 0, P, None, P, P, P, P, None)
    assert st == binding.DG_ERR_INVALID_ARG
    st = f(P, None, P, 1, 256, 4096, 192, P, None, 0.0, None, 0, P, None, P, P, P, P, None)
    assert st == binding.DG_ERR_UNSUPPORTED
    assert g(3, 256, 5000, 256, 0) <= binding.DG_NOALLOC_SCRATCH_BYTES
