"""Python binding of libdg.so: argument marshalling only.

Every function takes torch CUDA tensors (device memory owned by the caller), checks dtype,
device and contiguity, and hands raw pointers and sizes to the C entry point of the same
name.  All arithmetic happens in the HIP kernels.  There is no fallback: without the built
library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdg.so")

DG_OK, DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_WORKSPACE, DG_ERR_HIP = range(5)
DG_CANVAS = 256

EXPORTED = ("dg_vocab_pass_workspace_size", "dg_vocab_pass_ex_workspace_size",
            "dg_embedding_f16_bytes", "dg_embedding_f16", "dg_vocab_pass", "dg_vocab_pass_softcap",
            "dg_vocab_pass_ex", "dg_vocab_pass_ex_noalloc", "dg_accept_renoise", "dg_q_sample", "dg_selfcond_input_workspace_size",
            "dg_selfcond_input", "dg_lite_step", "dg_quantize_embedding_fp8",
            "dg_vocab_pass_fp8_workspace_size", "dg_vocab_pass_fp8",
            "dg_vocab_pass_fp8_dyn_workspace_size", "dg_vocab_pass_fp8_dyn", "dg_status_string",
            "dg_last_error")


class DGError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdg.so (after torch, so that the library shares torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, I, U64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
    lib.dg_vocab_pass_workspace_size.argtypes = [I, I, I, I]
    lib.dg_vocab_pass_workspace_size.restype = SZ
    lib.dg_vocab_pass_ex_workspace_size.argtypes = [I, I, I, I, I]
    lib.dg_vocab_pass_ex_workspace_size.restype = SZ
    lib.dg_embedding_f16_bytes.argtypes = [I, I]
    lib.dg_embedding_f16_bytes.restype = SZ
    lib.dg_embedding_f16.argtypes = [P, I, I, P, P]
    lib.dg_embedding_f16.restype = I
    lib.dg_vocab_pass.argtypes = [P, P, I, I, I, I, P, P, U64, P, P, P, P, P, P, P, SZ, P]
    lib.dg_vocab_pass.restype = I
    lib.dg_vocab_pass_softcap.argtypes = [P, P, I, I, I, I, P, P, U64, P, P, P, P, P, P, P, SZ, P,
                                          F]
    lib.dg_vocab_pass_softcap.restype = I
    lib.dg_vocab_pass_ex.argtypes = [P, P, P, I, I, I, I, P, P, F, P, U64, P, P, P, P, P, P, P, SZ,
                                     P]
    lib.dg_vocab_pass_ex.restype = I
    lib.dg_vocab_pass_ex_noalloc.argtypes = [P, P, P, I, I, I, I, P, P, F, P, U64, P, P, P, P, P,
                                             P, P]
    lib.dg_vocab_pass_ex_noalloc.restype = I
    lib.dg_accept_renoise.argtypes = [P, P, P, P, I, I, I, F, F, I, U64, P, P, P, P, P, P, P, P]
    lib.dg_accept_renoise.restype = I
    lib.dg_q_sample.argtypes = [P, I, I, I, P, U64, P, P]
    lib.dg_q_sample.restype = I
    lib.dg_selfcond_input_workspace_size.argtypes = [I, I, I, I]
    lib.dg_selfcond_input_workspace_size.restype = SZ
    lib.dg_selfcond_input.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, F, P, P, SZ, P]
    lib.dg_selfcond_input.restype = I
    lib.dg_lite_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, F, F, I, U64, P, P, P, P, P,
                                 P, P, P, P, P, P]
    lib.dg_lite_step.restype = I
    lib.dg_quantize_embedding_fp8.argtypes = [P, I, I, P, P, P, P]
    lib.dg_quantize_embedding_fp8.restype = I
    lib.dg_vocab_pass_fp8_workspace_size.argtypes = [I, I, I, I]
    lib.dg_vocab_pass_fp8_workspace_size.restype = SZ
    lib.dg_vocab_pass_fp8.argtypes = [P, P, P, P, I, I, I, I, P, P, U64, P, P, P, P, P, P, P, SZ,
                                      P, F]
    lib.dg_vocab_pass_fp8.restype = I
    lib.dg_vocab_pass_fp8_dyn_workspace_size.argtypes = [I, I, I, I]
    lib.dg_vocab_pass_fp8_dyn_workspace_size.restype = SZ
    lib.dg_vocab_pass_fp8_dyn.argtypes = [P, P, P, P, I, I, I, I, P, P, U64, P, P, P, P, P, P, P,
                                          SZ, P, F]
    lib.dg_vocab_pass_fp8_dyn.restype = I
    lib.dg_status_string.argtypes = [I]
    lib.dg_status_string.restype = ctypes.c_char_p
    lib.dg_last_error.argtypes = []
    lib.dg_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != DG_OK:
        lib = load()
        raise DGError(status, f"{lib.dg_status_string(status).decode()}: "
                              f"{lib.dg_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor], dtype: torch.dtype, numel: Optional[int], name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def dg_vocab_pass_workspace_size(n_canvas: int, C: int, V: int, d: int) -> int:
    return int(load().dg_vocab_pass_workspace_size(n_canvas, C, V, d))


def dg_vocab_pass(E: torch.Tensor, h: torch.Tensor, n_canvas: int, C: int, V: int, d: int,
                  temperature: torch.Tensor, commit: Optional[torch.Tensor], seed: int,
                  step: torch.Tensor, lse: Optional[torch.Tensor], entropy: torch.Tensor,
                  argmax_tok: torch.Tensor, gumbel_tok: torch.Tensor,
                  selfcond: Optional[torch.Tensor], workspace: torch.Tensor, stream=None) -> None:
    """E, h: bf16 bit patterns as torch.int16/uint16 or torch.bfloat16."""
    _vocab_pass(None, E, h, n_canvas, C, V, d, temperature, commit, seed, step, lse, entropy,
                argmax_tok, gumbel_tok, selfcond, workspace, stream)


def dg_vocab_pass_softcap(E: torch.Tensor, h: torch.Tensor, n_canvas: int, C: int, V: int,
                          d: int, temperature: torch.Tensor, commit: Optional[torch.Tensor],
                          seed: int, step: torch.Tensor, lse: Optional[torch.Tensor],
                          entropy: torch.Tensor, argmax_tok: torch.Tensor,
                          gumbel_tok: torch.Tensor, selfcond: Optional[torch.Tensor],
                          workspace: torch.Tensor, stream=None, softcap: float = 30.0) -> None:
    """dg_vocab_pass on the soft-capped logits softcap * tanh(S / softcap)."""
    _vocab_pass(float(softcap), E, h, n_canvas, C, V, d, temperature, commit, seed, step, lse,
                entropy, argmax_tok, gumbel_tok, selfcond, workspace, stream)


def e16_rows(V: int) -> int:
    """Rows of the fp16 embedding: V padded to whole 256-entry tiles (DG_E16_ROWS)."""
    return (V + 255) // 256 * 256


def dg_vocab_pass_ex_workspace_size(n_canvas: int, C: int, V: int, d: int, with_e16: bool) -> int:
    return int(load().dg_vocab_pass_ex_workspace_size(n_canvas, C, V, d, int(bool(with_e16))))


def dg_embedding_f16(E: torch.Tensor, V: int, d: int, E16: torch.Tensor, stream=None) -> None:
    """E16: [e16_rows(V) * d] fp16 bits (torch.int16/uint16 or torch.float16)."""
    _check(load().dg_embedding_f16(_bf16_ptr(E, V * d, "E"), V, d,
                                    _f16_ptr(E16, d * e16_rows(V), "E16"), _stream(stream)))


def _f16_ptr(t: Optional[torch.Tensor], numel: int, name: str):
    if t is None:
        return None
    if t.dtype not in (torch.float16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: dtype {t.dtype}, expected fp16 bits")
    return _ptr(t, t.dtype, numel, name)


def dg_vocab_pass_ex(E: torch.Tensor, E16: Optional[torch.Tensor], h: torch.Tensor,
                     n_canvas: int, C: int, V: int, d: int,
                     temperature: torch.Tensor, draw_temperature: Optional[torch.Tensor],
                     softcap: float, commit: Optional[torch.Tensor], seed: int,
                     step: torch.Tensor, lse: Optional[torch.Tensor], entropy: torch.Tensor,
                     argmax_tok: torch.Tensor, gumbel_tok: torch.Tensor,
                     selfcond: Optional[torch.Tensor], workspace: torch.Tensor,
                     stream=None) -> None:
    """Statistics at `temperature`, the Gumbel-max draw at `draw_temperature` (None: the
    same); softcap 0 for none; E16 the prepared fp16 embedding or None."""
    R = n_canvas * C
    lib = load()
    st = lib.dg_vocab_pass_ex(
        _bf16_ptr(E, V * d, "E"), _f16_ptr(E16, d * e16_rows(V), "E16"),
        _bf16_ptr(h, R * d, "h"), n_canvas, C, V, d,
        _ptr(temperature, torch.float32, n_canvas, "temperature"),
        _ptr(draw_temperature, torch.float32, n_canvas, "draw_temperature"),
        ctypes.c_float(softcap),
        _ptr(commit, torch.uint8, n_canvas, "commit"),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
        _ptr(step, torch.int32, n_canvas, "step"),
        _ptr(lse, torch.float32, R, "lse"),
        _ptr(entropy, torch.float32, R, "entropy"),
        _ptr(argmax_tok, torch.int32, R, "argmax_tok"),
        _ptr(gumbel_tok, torch.int32, R, "gumbel_tok"),
        _ptr(selfcond, torch.float32, R * d, "selfcond"),
        _ptr(workspace, torch.uint8, None, "workspace"),
        workspace.numel(), _stream(stream))
    _check(st)


def _vocab_pass(softcap, E, h, n_canvas, C, V, d, temperature, commit, seed, step, lse, entropy,
                argmax_tok, gumbel_tok, selfcond, workspace, stream) -> None:
    R = n_canvas * C
    lib = load()
    eb = _bf16_ptr(E, V * d, "E")
    hb = _bf16_ptr(h, R * d, "h")
    fn = lib.dg_vocab_pass if softcap is None else lib.dg_vocab_pass_softcap
    extra = () if softcap is None else (ctypes.c_float(softcap),)
    st = fn(
        eb, hb, n_canvas, C, V, d,
        _ptr(temperature, torch.float32, n_canvas, "temperature"),
        _ptr(commit, torch.uint8, n_canvas, "commit"),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
        _ptr(step, torch.int32, n_canvas, "step"),
        _ptr(lse, torch.float32, R, "lse"),
        _ptr(entropy, torch.float32, R, "entropy"),
        _ptr(argmax_tok, torch.int32, R, "argmax_tok"),
        _ptr(gumbel_tok, torch.int32, R, "gumbel_tok"),
        _ptr(selfcond, torch.float32, R * d, "selfcond"),
        _ptr(workspace, torch.uint8, None, "workspace"),
        workspace.numel(), _stream(stream), *extra)
    _check(st)


def _bf16_ptr(t: torch.Tensor, numel: int, name: str):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: dtype {t.dtype}, expected bf16 bits")
    return _ptr(t, t.dtype, numel, name)


def dg_accept_renoise(entropy: torch.Tensor, argmax_tok: torch.Tensor, gumbel_tok: torch.Tensor,
                      commit: Optional[torch.Tensor], n_canvas: int, C: int, V: int,
                      entropy_budget: float, confidence_threshold: float,
                      stability_threshold: int, seed: int, step: torch.Tensor,
                      prev_argmax: torch.Tensor, stable_count: torch.Tensor,
                      next_tokens: torch.Tensor, accept_mask: Optional[torch.Tensor],
                      converged: torch.Tensor, mean_entropy: Optional[torch.Tensor],
                      stream=None) -> None:
    R = n_canvas * C
    st = load().dg_accept_renoise(
        _ptr(entropy, torch.float32, R, "entropy"),
        _ptr(argmax_tok, torch.int32, R, "argmax_tok"),
        _ptr(gumbel_tok, torch.int32, R, "gumbel_tok"),
        _ptr(commit, torch.uint8, n_canvas, "commit"),
        n_canvas, C, V, float(entropy_budget), float(confidence_threshold),
        int(stability_threshold), ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
        _ptr(step, torch.int32, n_canvas, "step"),
        _ptr(prev_argmax, torch.int32, R, "prev_argmax"),
        _ptr(stable_count, torch.int32, n_canvas, "stable_count"),
        _ptr(next_tokens, torch.int32, R, "next_tokens"),
        _ptr(accept_mask, torch.uint8, R, "accept_mask"),
        _ptr(converged, torch.uint8, n_canvas, "converged"),
        _ptr(mean_entropy, torch.float32, n_canvas, "mean_entropy"),
        _stream(stream))
    _check(st)


def dg_q_sample(x0: torch.Tensor, n_canvas: int, C: int, V: int, kappa: torch.Tensor, seed: int,
                xt: torch.Tensor, stream=None) -> None:
    R = n_canvas * C
    st = load().dg_q_sample(
        _ptr(x0, torch.int32, R, "x0"), n_canvas, C, V,
        _ptr(kappa, torch.float32, n_canvas, "kappa"),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
        _ptr(xt, torch.int32, R, "xt"), _stream(stream))
    _check(st)


def dg_selfcond_input_workspace_size(n_canvas: int, C: int, D: int, F: int) -> int:
    return int(load().dg_selfcond_input_workspace_size(n_canvas, C, D, F))


def dg_selfcond_input(sc: Optional[torch.Tensor], tokens: torch.Tensor, E: torch.Tensor,
                      pre_norm: Optional[torch.Tensor], W_gate: Optional[torch.Tensor],
                      W_up: Optional[torch.Tensor], W_down: Optional[torch.Tensor],
                      commit: Optional[torch.Tensor], n_canvas: int, C: int, V: int, D: int,
                      F: int, eps: float, out: torch.Tensor, workspace: torch.Tensor,
                      stream=None) -> None:
    """Weights and E as bf16 bits (int16/uint16) or torch.bfloat16; out likewise."""
    R = n_canvas * C
    lib = load()
    opt = lambda t, n, name: None if t is None else _bf16_ptr(t, n, name)
    st = lib.dg_selfcond_input(
        _ptr(sc, torch.float32, R * D, "sc"),
        _ptr(tokens, torch.int32, R, "tokens"),
        _bf16_ptr(E, V * D, "E"),
        opt(pre_norm, D, "pre_norm"), opt(W_gate, F * D, "W_gate"), opt(W_up, F * D, "W_up"),
        opt(W_down, D * F, "W_down"),
        _ptr(commit, torch.uint8, n_canvas, "commit"),
        n_canvas, C, V, D, F, ctypes.c_float(eps),
        _bf16_ptr(out, R * D, "out"),
        _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream))
    _check(st)


def dg_lite_step(h: torch.Tensor, E: torch.Tensor, temperature: torch.Tensor, lse: torch.Tensor,
                 entropy: torch.Tensor, argmax_tok: torch.Tensor, gumbel_tok: torch.Tensor,
                 n_canvas: int, C: int, V: int, d: int, softcap: float, entropy_threshold: float,
                 stability_steps: int, seed: int, step: torch.Tensor, conf: torch.Tensor,
                 x: torch.Tensor, prev_argmax: torch.Tensor, prev_conf: torch.Tensor,
                 committed: torch.Tensor, stable_count: torch.Tensor,
                 final_tokens: Optional[torch.Tensor], converged: torch.Tensor,
                 mean_entropy: Optional[torch.Tensor], stream=None) -> None:
    R = n_canvas * C
    lib = load()
    st = lib.dg_lite_step(
        _bf16_ptr(h, R * d, "h"), _bf16_ptr(E, V * d, "E"),
        _ptr(temperature, torch.float32, n_canvas, "temperature"),
        _ptr(lse, torch.float32, R, "lse"), _ptr(entropy, torch.float32, R, "entropy"),
        _ptr(argmax_tok, torch.int32, R, "argmax_tok"),
        _ptr(gumbel_tok, torch.int32, R, "gumbel_tok"),
        n_canvas, C, V, d, ctypes.c_float(softcap), ctypes.c_float(entropy_threshold),
        stability_steps, ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
        _ptr(step, torch.int32, n_canvas, "step"), _ptr(conf, torch.float32, R, "conf"),
        _ptr(x, torch.int32, R, "x"), _ptr(prev_argmax, torch.int32, R, "prev_argmax"),
        _ptr(prev_conf, torch.float32, R, "prev_conf"),
        _ptr(committed, torch.uint8, R, "committed"),
        _ptr(stable_count, torch.int32, n_canvas, "stable_count"),
        _ptr(final_tokens, torch.int32, R, "final_tokens"),
        _ptr(converged, torch.uint8, n_canvas, "converged"),
        _ptr(mean_entropy, torch.float32, n_canvas, "mean_entropy"), _stream(stream))
    _check(st)


DG_NOALLOC_SCRATCH_BYTES = 64 << 20


def dg_vocab_pass_ex_noalloc(E: torch.Tensor, E16: Optional[torch.Tensor], h: torch.Tensor,
                             n_canvas: int, C: int, V: int, d: int,
                             temperature: torch.Tensor, draw_temperature: Optional[torch.Tensor],
                             softcap: float, commit: Optional[torch.Tensor], seed: int,
                             step: torch.Tensor, lse: Optional[torch.Tensor],
                             entropy: torch.Tensor, argmax_tok: torch.Tensor,
                             gumbel_tok: torch.Tensor, selfcond: Optional[torch.Tensor],
                             stream=None) -> None:
    """dg_vocab_pass_ex in the library's static per-GPU scratch (no workspace, no allocation;
    shapes beyond DG_NOALLOC_SCRATCH_BYTES of workspace raise DG_ERR_WORKSPACE)."""
    R = n_canvas * C
    lib = load()
    st = lib.dg_vocab_pass_ex_noalloc(
        _bf16_ptr(E, V * d, "E"), _f16_ptr(E16, d * e16_rows(V), "E16"),
        _bf16_ptr(h, R * d, "h"), n_canvas, C, V, d,
        _ptr(temperature, torch.float32, n_canvas, "temperature"),
        _ptr(draw_temperature, torch.float32, n_canvas, "draw_temperature"),
        ctypes.c_float(softcap),
        _ptr(commit, torch.uint8, n_canvas, "commit"),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
        _ptr(step, torch.int32, n_canvas, "step"),
        _ptr(lse, torch.float32, R, "lse"),
        _ptr(entropy, torch.float32, R, "entropy"),
        _ptr(argmax_tok, torch.int32, R, "argmax_tok"),
        _ptr(gumbel_tok, torch.int32, R, "gumbel_tok"),
        _ptr(selfcond, torch.float32, R * d, "selfcond"),
        _stream(stream))
    _check(st)


def dg_quantize_embedding_fp8(E: torch.Tensor, V: int, d: int, codes: torch.Tensor,
                              E16: Optional[torch.Tensor], row_exp: torch.Tensor,
                              stream=None) -> None:
    lib = load()
    _check(lib.dg_quantize_embedding_fp8(_bf16_ptr(E, V * d, "E"), V, d,
                                         _ptr(codes, torch.uint8, V * d, "codes"),
                                         _f16_ptr(E16, d * e16_rows(V), "E16"),
                                         _ptr(row_exp, torch.int32, V, "row_exp"),
                                         _stream(stream)))


def dg_vocab_pass_fp8_workspace_size(n_canvas: int, C: int, V: int, d: int) -> int:
    return int(load().dg_vocab_pass_fp8_workspace_size(n_canvas, C, V, d))


def _fp8_pass(fn, codes, E16, row_exp, h, n_canvas, C, V, d, temperature, commit, seed, step,
              lse, entropy, argmax_tok, gumbel_tok, selfcond, workspace, stream, softcap):
    R = n_canvas * C
    st = fn(
        _ptr(codes, torch.uint8, V * d, "codes"),
        _f16_ptr(E16, d * e16_rows(V), "E16"),
        _ptr(row_exp, torch.int32, V, "row_exp"),
        _bf16_ptr(h, R * d, "h"), n_canvas, C, V, d,
        _ptr(temperature, torch.float32, n_canvas, "temperature"),
        _ptr(commit, torch.uint8, n_canvas, "commit"),
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
        _ptr(step, torch.int32, n_canvas, "step"), _ptr(lse, torch.float32, R, "lse"),
        _ptr(entropy, torch.float32, R, "entropy"),
        _ptr(argmax_tok, torch.int32, R, "argmax_tok"),
        _ptr(gumbel_tok, torch.int32, R, "gumbel_tok"),
        _ptr(selfcond, torch.float32, R * d, "selfcond"),
        _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream),
        ctypes.c_float(softcap))
    _check(st)


def dg_vocab_pass_fp8(codes: torch.Tensor, E16: Optional[torch.Tensor], row_exp: torch.Tensor,
                      h: torch.Tensor, n_canvas: int,
                      C: int, V: int, d: int, temperature: torch.Tensor,
                      commit: Optional[torch.Tensor], seed: int, step: torch.Tensor,
                      lse: Optional[torch.Tensor], entropy: torch.Tensor,
                      argmax_tok: torch.Tensor, gumbel_tok: torch.Tensor,
                      selfcond: Optional[torch.Tensor], workspace: torch.Tensor, stream=None,
                      softcap: float = 0.0) -> None:
    _fp8_pass(load().dg_vocab_pass_fp8, codes, E16, row_exp, h, n_canvas, C, V, d, temperature,
              commit, seed, step, lse, entropy, argmax_tok, gumbel_tok, selfcond, workspace,
              stream, softcap)


def dg_vocab_pass_fp8_dyn_workspace_size(n_canvas: int, C: int, V: int, d: int) -> int:
    return int(load().dg_vocab_pass_fp8_dyn_workspace_size(n_canvas, C, V, d))


def dg_vocab_pass_fp8_dyn(codes: torch.Tensor, E16: Optional[torch.Tensor],
                          row_exp: torch.Tensor, h: torch.Tensor, n_canvas: int,
                          C: int, V: int, d: int, temperature: torch.Tensor,
                          commit: Optional[torch.Tensor], seed: int, step: torch.Tensor,
                          lse: Optional[torch.Tensor], entropy: torch.Tensor,
                          argmax_tok: torch.Tensor, gumbel_tok: torch.Tensor,
                          selfcond: Optional[torch.Tensor], workspace: torch.Tensor,
                          stream=None, softcap: float = 0.0) -> None:
    """dg_vocab_pass_fp8 with h quantised per row to FP8 inside the call (FP8 x FP8 MFMA)."""
    _fp8_pass(load().dg_vocab_pass_fp8_dyn, codes, E16, row_exp, h, n_canvas, C, V, d,
              temperature, commit, seed, step, lse, entropy, argmax_tok, gumbel_tok, selfcond,
              workspace, stream, softcap)
