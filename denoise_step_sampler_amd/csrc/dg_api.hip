// C ABI of libdg.so: host-side validation, workspace sizing and launches.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "dg_internal.h"

namespace {

thread_local char g_err[512] = "";

dg_status fail(dg_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dg_status fail(dg_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dg_status hip_fail(hipError_t e, const char* what) {
  return fail(DG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the vocabulary pass: the two-GEMM pieces, then (when the caller gives no fp16
// embedding and the expectation is asked for) room to build one.
size_t gemm_bytes(int n_canvas, int V, int d) { return al256(dg::gemm_plan(n_canvas, V, d).bytes); }
// FP8 x FP8 pass: the hidden states' codes [R, d] and row exponents [R], quantised per call
size_t a8_bytes(int n_canvas, int d) {
  const size_t R = (size_t)n_canvas * DG_CANVAS;
  return al256(R * (size_t)d) + al256(R * 4);
}
size_t pass_bytes(int n_canvas, int V, int d, bool build_e16, bool a8 = false) {
  return gemm_bytes(n_canvas, V, d) + (build_e16 ? al256(dg::e16_bytes(V, d)) : 0) +
         (a8 ? a8_bytes(n_canvas, d) : 0);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void split_seed(uint64_t seed, uint32_t* k0, uint32_t* k1) {
  *k0 = (uint32_t)(seed & 0xFFFFFFFFull);
  *k1 = (uint32_t)(seed >> 32);
}

dg_status check_canvas(int n_canvas, int C) {
  if (n_canvas < 1 || n_canvas > DG_MAX_CANVASES)
    return fail(DG_ERR_INVALID_ARG, "n_canvas=%d outside [1, %d]", n_canvas, DG_MAX_CANVASES);
  if (C != DG_CANVAS) return fail(DG_ERR_UNSUPPORTED, "C=%d: only C=%d is supported", C, DG_CANVAS);
  return DG_OK;
}

dg_status check_vocab_shape(int n_canvas, int C, int V, int d) {
  dg_status s = check_canvas(n_canvas, C);
  if (s != DG_OK) return s;
  if (V < 1 || V > DG_MAX_V) return fail(DG_ERR_INVALID_ARG, "V=%d outside [1, %d]", V, DG_MAX_V);
  if (d < 1 || d > DG_MAX_D) return fail(DG_ERR_INVALID_ARG, "d=%d outside [1, %d]", d, DG_MAX_D);
  if (d % 128 != 0) return fail(DG_ERR_UNSUPPORTED, "d=%d: d must be a multiple of 128", d);
  return DG_OK;
}

dg_status check_ffw_shape(int n_canvas, int C, int D, int F) {
  dg_status s = check_canvas(n_canvas, C);
  if (s != DG_OK) return s;
  if (D < 64 || D > 16384 || D % 64 != 0)
    return fail(DG_ERR_UNSUPPORTED, "D=%d: need a multiple of 64 in [64, 16384]", D);
  if (F < 64 || F > 65536 || F % 64 != 0)
    return fail(DG_ERR_UNSUPPORTED, "F=%d: need a multiple of 64 in [64, 65536]", F);
  return DG_OK;
}

}  // namespace

extern "C" {

const char* dg_status_string(dg_status s) {
  switch (s) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARG: return "invalid argument";
    case DG_ERR_UNSUPPORTED: return "unsupported";
    case DG_ERR_WORKSPACE: return "workspace too small";
    case DG_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* dg_last_error(void) { return g_err; }

size_t dg_vocab_pass_workspace_size(int n_canvas, int C, int V, int d) {
  return dg_vocab_pass_ex_workspace_size(n_canvas, C, V, d, 0);
}

size_t dg_vocab_pass_ex_workspace_size(int n_canvas, int C, int V, int d, int with_e16) {
  char keep[sizeof(g_err)];
  memcpy(keep, g_err, sizeof(g_err));
  const dg_status s = check_vocab_shape(n_canvas, C, V, d);
  memcpy(g_err, keep, sizeof(g_err));
  if (s != DG_OK) return 0;
  return pass_bytes(n_canvas, V, d, with_e16 == 0);
}

size_t dg_embedding_f16_bytes(int V, int d) {
  if (V < 1 || V > DG_MAX_V || d < 128 || d > DG_MAX_D || d % 128 != 0) return 0;
  return dg::e16_bytes(V, d);
}

dg_status dg_embedding_f16(const uint16_t* E, int V, int d, uint16_t* E16, void* stream) {
  g_err[0] = 0;
  if (V < 1 || V > DG_MAX_V) return fail(DG_ERR_INVALID_ARG, "V=%d outside [1, %d]", V, DG_MAX_V);
  if (d < 128 || d > DG_MAX_D || d % 128 != 0)
    return fail(DG_ERR_UNSUPPORTED, "d=%d: need a multiple of 128 in [128, %d]", d, DG_MAX_D);
  if (!E || !E16) return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(E) || !aligned16(E16))
    return fail(DG_ERR_INVALID_ARG, "E and E16 must be 16-byte aligned");
  const hipError_t e = dg::e16_launch(E, V, d, E16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fp16 embedding launch");
  return DG_OK;
}

}  // extern "C"

namespace {

// E: the bf16 embedding (read by the logits pass unless E8 is given, and by the combine's
// exact corrections); E8 / E_exp: the FP8 form the logits pass streams instead; E16: the fp16
// embedding for the expectation, or null: built in the workspace (from E8 when
// given, else from E).
dg_status vocab_pass(const uint16_t* E, const uint16_t* h, int n_canvas, int C, int V, int d,
                     const float* temperature, const uint8_t* commit, uint64_t seed,
                     const int32_t* step, float* lse, float* entropy, int32_t* argmax_tok,
                     int32_t* gumbel_tok, float* selfcond, void* workspace,
                     size_t workspace_bytes, void* stream, float softcap, const uint8_t* E8,
                     const int32_t* E_exp, const uint16_t* E16,
                     const float* draw_temperature, bool a8 = false) {
  dg_status s = check_vocab_shape(n_canvas, C, V, d);
  if (s != DG_OK) return s;
  if ((!E && !E8) || !h || !temperature || !step || !entropy || !argmax_tok || !gumbel_tok)
    return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((E && !aligned16(E)) || !aligned16(h) || (E16 && !aligned16(E16)))
    return fail(DG_ERR_INVALID_ARG, "E, E16 and h must be 16-byte aligned");
  if (selfcond && !aligned16(selfcond))
    return fail(DG_ERR_INVALID_ARG, "selfcond must be 16-byte aligned");
  const bool build = selfcond != nullptr && E16 == nullptr;
  const size_t need = pass_bytes(n_canvas, V, d, build, a8);
  if (!workspace || workspace_bytes < need)
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(DG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (build) {
    uint16_t* e16 = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) +
                                                gemm_bytes(n_canvas, V, d));
    const hipError_t e = E8 ? dg::e16_fp8_launch(E8, E_exp, V, d, e16, st)
                            : dg::e16_launch(E, V, d, e16, st);
    if (e != hipSuccess) return hip_fail(e, "fp16 embedding launch");
    E16 = e16;
  }
  uint8_t* h8 = nullptr;
  int32_t* h_exp = nullptr;
  if (a8) {  // the hidden states quantised per row (dynamic activations)
    char* q = static_cast<char*>(workspace) + gemm_bytes(n_canvas, V, d) +
              (build ? al256(dg::e16_bytes(V, d)) : 0);
    const size_t R = (size_t)n_canvas * DG_CANVAS;
    h8 = reinterpret_cast<uint8_t*>(q);
    h_exp = reinterpret_cast<int32_t*>(q + al256(R * (size_t)d));
    const hipError_t e = dg::fp8_quantize_launch(h, (int)R, d, h8, h_exp, st);
    if (e != hipSuccess) return hip_fail(e, "fp8 quantize launch");
  }
  dg::VocabArgs a{};
  a.E = E;
  a.h = h;
  a.n_canvas = n_canvas;
  a.V = V;
  a.d = d;
  a.temperature = temperature;
  a.draw_temperature = draw_temperature;
  a.commit = commit;
  split_seed(seed, &a.k0, &a.k1);
  a.step = step;
  a.lse = lse;
  a.entropy = entropy;
  a.argmax_tok = argmax_tok;
  a.gumbel_tok = gumbel_tok;
  a.selfcond = selfcond;
  a.softcap = softcap;
  a.E8 = E8;
  a.E_exp = E_exp;
  a.E16 = E16;
  a.h8 = h8;
  a.h_exp = h_exp;
  const hipError_t e = dg::gemm_launch(a, dg::gemm_plan(n_canvas, V, d), workspace, st);
  if (e != hipSuccess) return hip_fail(e, "vocab pass launch");
  return DG_OK;
}

}  // namespace

extern "C" {

dg_status dg_vocab_pass(const uint16_t* E, const uint16_t* h, int n_canvas, int C, int V, int d,
                        const float* temperature, const uint8_t* commit, uint64_t seed,
                        const int32_t* step, float* lse, float* entropy, int32_t* argmax_tok,
                        int32_t* gumbel_tok, float* selfcond, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  return vocab_pass(E, h, n_canvas, C, V, d, temperature, commit, seed, step, lse, entropy,
                    argmax_tok, gumbel_tok, selfcond, workspace, workspace_bytes, stream, 0.0f,
                    nullptr, nullptr, nullptr, nullptr);
}

dg_status dg_vocab_pass_softcap(const uint16_t* E, const uint16_t* h, int n_canvas, int C, int V,
                                int d, const float* temperature, const uint8_t* commit,
                                uint64_t seed, const int32_t* step, float* lse, float* entropy,
                                int32_t* argmax_tok, int32_t* gumbel_tok, float* selfcond,
                                void* workspace, size_t workspace_bytes, void* stream,
                                float softcap) {
  g_err[0] = 0;
  if (!(softcap > 0.0f) || !isfinite(softcap))
    return fail(DG_ERR_INVALID_ARG, "softcap must be finite and > 0");
  return vocab_pass(E, h, n_canvas, C, V, d, temperature, commit, seed, step, lse, entropy,
                    argmax_tok, gumbel_tok, selfcond, workspace, workspace_bytes, stream, softcap,
                    nullptr, nullptr, nullptr, nullptr);
}

dg_status dg_vocab_pass_ex(const uint16_t* E, const uint16_t* E16, const uint16_t* h,
                           int n_canvas, int C, int V, int d, const float* temperature,
                           const float* draw_temperature, float softcap, const uint8_t* commit,
                           uint64_t seed, const int32_t* step, float* lse, float* entropy,
                           int32_t* argmax_tok, int32_t* gumbel_tok, float* selfcond,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (softcap != 0.0f && (!(softcap > 0.0f) || !isfinite(softcap)))
    return fail(DG_ERR_INVALID_ARG, "softcap must be 0 or finite and > 0");
  if (!E) return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  return vocab_pass(E, h, n_canvas, C, V, d, temperature, commit, seed, step, lse, entropy,
                    argmax_tok, gumbel_tok, selfcond, workspace, workspace_bytes, stream, softcap,
                    nullptr, nullptr, E16, draw_temperature);
}

}  // extern "C"

namespace {

// Scratch of dg_vocab_pass_ex_noalloc: one copy on every GPU the library runs on, held until
// the process ends.  Host code never passes `scratch` itself (on the host it names a stand-in,
// not device memory): each device's address comes from hipGetSymbolAddress, taken once per
// device with that device current.
static __device__ __align__(256) unsigned char scratch[DG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dg_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DG_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u))
      return fail(DG_ERR_HIP, "scratch of device %d has no usable address", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DG_OK;
}

}  // namespace

extern "C" {

dg_status dg_vocab_pass_ex_noalloc(const uint16_t* E, const uint16_t* E16, const uint16_t* h,
                                   int n_canvas, int C, int V, int d, const float* temperature,
                                   const float* draw_temperature, float softcap,
                                   const uint8_t* commit, uint64_t seed, const int32_t* step,
                                   float* lse, float* entropy, int32_t* argmax_tok,
                                   int32_t* gumbel_tok, float* selfcond, void* stream) {
  g_err[0] = 0;
  if (softcap != 0.0f && (!(softcap > 0.0f) || !isfinite(softcap)))
    return fail(DG_ERR_INVALID_ARG, "softcap must be 0 or finite and > 0");
  if (!E) return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  dg_status s = check_vocab_shape(n_canvas, C, V, d);
  if (s != DG_OK) return s;
  const size_t need = pass_bytes(n_canvas, V, d, selfcond != nullptr && E16 == nullptr);
  if (need > DG_NOALLOC_SCRATCH_BYTES)
    return fail(DG_ERR_WORKSPACE,
                "n_canvas=%d V=%d d=%d needs %zu bytes of scratch; the static scratch holds %zu "
                "(use dg_vocab_pass_ex with a workspace)",
                n_canvas, V, d, need, (size_t)DG_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != DG_OK) return s;
  // nothing in the scratch needs to start at zero: every byte the kernels read is written
  // earlier in the same call
  return vocab_pass(E, h, n_canvas, C, V, d, temperature, commit, seed, step, lse, entropy,
                    argmax_tok, gumbel_tok, selfcond, ws, DG_NOALLOC_SCRATCH_BYTES, stream,
                    softcap, nullptr, nullptr, E16, draw_temperature);
}

size_t dg_vocab_pass_fp8_workspace_size(int n_canvas, int C, int V, int d) {
  return dg_vocab_pass_ex_workspace_size(n_canvas, C, V, d, 0);
}

dg_status dg_quantize_embedding_fp8(const uint16_t* E, int V, int d, uint8_t* codes,
                                    uint16_t* E16, int32_t* row_exp, void* stream) {
  g_err[0] = 0;
  if (V < 1 || V > DG_MAX_V) return fail(DG_ERR_INVALID_ARG, "V=%d outside [1, %d]", V, DG_MAX_V);
  if (d < 128 || d > DG_MAX_D || d % 128 != 0)
    return fail(DG_ERR_UNSUPPORTED, "d=%d: need a multiple of 128 in [128, %d]", d, DG_MAX_D);
  if (!E || !codes || !row_exp) return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(E) || !aligned16(codes) || (E16 && !aligned16(E16)))
    return fail(DG_ERR_INVALID_ARG, "E, codes and E16 must be 16-byte aligned");
  hipError_t e = dg::fp8_quantize_launch(E, V, d, codes, row_exp, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fp8 quantize launch");
  if (E16) {
    e = dg::e16_fp8_launch(codes, row_exp, V, d, E16, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "fp16 embedding launch");
  }
  return DG_OK;
}

dg_status dg_vocab_pass_fp8(const uint8_t* codes, const uint16_t* E16, const int32_t* row_exp,
                            const uint16_t* h,
                            int n_canvas, int C, int V, int d, const float* temperature,
                            const uint8_t* commit, uint64_t seed, const int32_t* step,
                            float* lse, float* entropy, int32_t* argmax_tok,
                            int32_t* gumbel_tok, float* selfcond, void* workspace,
                            size_t workspace_bytes, void* stream, float softcap) {
  g_err[0] = 0;
  if (!codes || !row_exp) return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(codes) || !aligned16(row_exp))
    return fail(DG_ERR_INVALID_ARG, "codes and row_exp must be 16-byte aligned");
  if (softcap != 0.0f && (!(softcap > 0.0f) || !isfinite(softcap)))
    return fail(DG_ERR_INVALID_ARG, "softcap must be 0 or finite and > 0");
  return vocab_pass(nullptr, h, n_canvas, C, V, d, temperature, commit, seed, step, lse, entropy,
                    argmax_tok, gumbel_tok, selfcond, workspace, workspace_bytes, stream, softcap,
                    codes, row_exp, E16, nullptr);
}

size_t dg_vocab_pass_fp8_dyn_workspace_size(int n_canvas, int C, int V, int d) {
  const size_t g = dg_vocab_pass_ex_workspace_size(n_canvas, C, V, d, 0);
  return g == 0 ? 0 : g + a8_bytes(n_canvas, d);
}

dg_status dg_vocab_pass_fp8_dyn(const uint8_t* codes, const uint16_t* E16,
                                const int32_t* row_exp, const uint16_t* h, int n_canvas, int C,
                                int V, int d, const float* temperature, const uint8_t* commit,
                                uint64_t seed, const int32_t* step, float* lse, float* entropy,
                                int32_t* argmax_tok, int32_t* gumbel_tok, float* selfcond,
                                void* workspace, size_t workspace_bytes, void* stream,
                                float softcap) {
  g_err[0] = 0;
  if (!codes || !row_exp) return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(codes) || !aligned16(row_exp))
    return fail(DG_ERR_INVALID_ARG, "codes and row_exp must be 16-byte aligned");
  if (softcap != 0.0f && (!(softcap > 0.0f) || !isfinite(softcap)))
    return fail(DG_ERR_INVALID_ARG, "softcap must be 0 or finite and > 0");
  return vocab_pass(nullptr, h, n_canvas, C, V, d, temperature, commit, seed, step, lse, entropy,
                    argmax_tok, gumbel_tok, selfcond, workspace, workspace_bytes, stream, softcap,
                    codes, row_exp, E16, nullptr, true);
}

dg_status dg_accept_renoise(const float* entropy, const int32_t* argmax_tok,
                            const int32_t* gumbel_tok, const uint8_t* commit, int n_canvas, int C,
                            int V, float entropy_budget, float confidence_threshold,
                            int stability_threshold, uint64_t seed, const int32_t* step,
                            int32_t* prev_argmax, int32_t* stable_count, int32_t* next_tokens,
                            uint8_t* accept_mask, uint8_t* converged, float* mean_entropy,
                            void* stream) {
  g_err[0] = 0;
  dg_status s = check_canvas(n_canvas, C);
  if (s != DG_OK) return s;
  if (V < 1 || V > (1 << 30)) return fail(DG_ERR_INVALID_ARG, "V=%d outside [1, 2^30]", V);
  if (!entropy || !argmax_tok || !gumbel_tok || !step || !prev_argmax || !stable_count ||
      !next_tokens || !converged)
    return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!(entropy_budget >= 0.0f) || !isfinite(entropy_budget))
    return fail(DG_ERR_INVALID_ARG, "entropy_budget must be finite and >= 0");
  if (!isfinite(confidence_threshold))
    return fail(DG_ERR_INVALID_ARG, "confidence_threshold must be finite");
  if (stability_threshold < 1)
    return fail(DG_ERR_INVALID_ARG, "stability_threshold must be >= 1");
  dg::AcceptArgs a{};
  a.entropy = entropy;
  a.argmax_tok = argmax_tok;
  a.gumbel_tok = gumbel_tok;
  a.commit = commit;
  a.n_canvas = n_canvas;
  a.V = V;
  a.budget = entropy_budget;
  a.confidence = confidence_threshold;
  a.stability = stability_threshold;
  split_seed(seed, &a.k0, &a.k1);
  a.step = step;
  a.prev_argmax = prev_argmax;
  a.stable_count = stable_count;
  a.next_tokens = next_tokens;
  a.accept_mask = accept_mask;
  a.converged = converged;
  a.mean_entropy = mean_entropy;
  const hipError_t e = dg::accept_renoise_launch(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "accept/renoise launch");
  return DG_OK;
}

dg_status dg_lite_step(const uint16_t* h, const uint16_t* E, const float* temperature,
                       const float* lse, const float* entropy, const int32_t* argmax_tok,
                       const int32_t* gumbel_tok, int n_canvas, int C, int V, int d,
                       float softcap, float entropy_threshold, int stability_steps,
                       uint64_t seed, const int32_t* step, float* conf, int32_t* x,
                       int32_t* prev_argmax, float* prev_conf, uint8_t* committed,
                       int32_t* stable_count, int32_t* final_tokens, uint8_t* converged,
                       float* mean_entropy, void* stream) {
  g_err[0] = 0;
  dg_status s = check_vocab_shape(n_canvas, C, V, d);
  if (s != DG_OK) return s;
  if (!h || !E || !temperature || !lse || !entropy || !argmax_tok || !gumbel_tok || !step ||
      !conf || !x || !prev_argmax || !prev_conf || !committed || !stable_count || !converged)
    return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(h) || !aligned16(E))
    return fail(DG_ERR_INVALID_ARG, "h and E must be 16-byte aligned");
  if (!(softcap >= 0.0f) || !isfinite(softcap))
    return fail(DG_ERR_INVALID_ARG, "softcap must be finite and >= 0");
  if (!isfinite(entropy_threshold))
    return fail(DG_ERR_INVALID_ARG, "entropy_threshold must be finite");
  if (stability_steps < 0) return fail(DG_ERR_INVALID_ARG, "stability_steps must be >= 0");
  dg::LiteArgs a{};
  a.h = h;
  a.E = E;
  a.temperature = temperature;
  a.lse = lse;
  a.entropy = entropy;
  a.argmax_tok = argmax_tok;
  a.gumbel_tok = gumbel_tok;
  a.R = n_canvas * C;
  a.V = V;
  a.d = d;
  a.softcap = softcap;
  a.threshold = entropy_threshold;
  a.stability_steps = stability_steps;
  split_seed(seed, &a.k0, &a.k1);
  a.step = step;
  a.conf = conf;
  a.x = x;
  a.prev_argmax = prev_argmax;
  a.prev_conf = prev_conf;
  a.committed = committed;
  a.stable_count = stable_count;
  a.final_tokens = final_tokens;
  a.converged = converged;
  a.mean_entropy = mean_entropy;
  const hipError_t e = dg::lite_step_launch(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "lite sampler launch");
  return DG_OK;
}

size_t dg_selfcond_input_workspace_size(int n_canvas, int C, int D, int F) {
  char keep[sizeof(g_err)];
  memcpy(keep, g_err, sizeof(g_err));
  const dg_status s = check_ffw_shape(n_canvas, C, D, F);
  memcpy(g_err, keep, sizeof(g_err));
  if (s != DG_OK) return 0;
  return dg::ffw_plan(n_canvas, D, F).bytes;
}

dg_status dg_selfcond_input(const float* sc, const int32_t* tokens, const uint16_t* E,
                            const uint16_t* pre_norm, const uint16_t* W_gate,
                            const uint16_t* W_up, const uint16_t* W_down,
                            const uint8_t* commit, int n_canvas, int C, int V, int D, int F,
                            float eps, uint16_t* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  g_err[0] = 0;
  dg_status s = check_ffw_shape(n_canvas, C, D, F);
  if (s != DG_OK) return s;
  if (V < 1 || V > (1 << 30)) return fail(DG_ERR_INVALID_ARG, "V=%d outside [1, 2^30]", V);
  if (!(eps >= 0.0f) || !isfinite(eps))
    return fail(DG_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!tokens || !E || !out) return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (sc && (!pre_norm || !W_gate || !W_up || !W_down))
    return fail(DG_ERR_INVALID_ARG, "the MLP weights are NULL");
  const void* ptrs[] = {sc, tokens, E, pre_norm, W_gate, W_up, W_down, out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(DG_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const dg::FfwPlan plan = dg::ffw_plan(n_canvas, D, F);
  if (!workspace || workspace_bytes < plan.bytes)
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                plan.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(DG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  dg::FfwArgs a{};
  a.sc = sc;
  a.tokens = tokens;
  a.E = E;
  a.pre_norm = pre_norm;
  a.W_gate = W_gate;
  a.W_up = W_up;
  a.W_down = W_down;
  a.commit = commit;
  a.V = V;
  a.D = D;
  a.F = F;
  a.eps = eps;
  a.out = out;
  const hipError_t e = dg::ffw_launch(a, plan, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "self-conditioning input launch");
  return DG_OK;
}

dg_status dg_q_sample(const int32_t* x0, int n_canvas, int C, int V, const float* kappa,
                      uint64_t seed, int32_t* xt, void* stream) {
  g_err[0] = 0;
  dg_status s = check_canvas(n_canvas, C);
  if (s != DG_OK) return s;
  if (V < 1 || V > (1 << 30)) return fail(DG_ERR_INVALID_ARG, "V=%d outside [1, 2^30]", V);
  if (!x0 || !kappa || !xt) return fail(DG_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((const void*)x0 == (const void*)xt) return fail(DG_ERR_INVALID_ARG, "xt may not alias x0");
  uint32_t k0, k1;
  split_seed(seed, &k0, &k1);
  const hipError_t e = dg::q_sample_launch(x0, n_canvas, V, kappa, k0, k1, xt, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "q_sample launch");
  return DG_OK;
}

}  // extern "C"
