// Internal host/device interfaces shared by the translation units of libdg.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dg.h"

namespace dg {

// Arguments of one vocabulary pass (device pointers).
struct VocabArgs {
  const uint16_t* E;
  const uint16_t* h;
  int n_canvas;
  int V;
  int d;
  const float* temperature;
  const float* draw_temperature;  // temperature of the Gumbel-max draw alone, or null (the
                                  // draw uses `temperature`)
  const uint8_t* commit;
  uint32_t k0, k1;  // Philox key
  const int32_t* step;
  float* lse;
  float* entropy;
  int32_t* argmax_tok;
  int32_t* gumbel_tok;
  float* selfcond;
  float softcap;  // > 0: z = softcap tanh(S / softcap) / T; 0: z = S / T
  // FP8 embedding for the logits pass: E4M3 codes [V, d] and row exponents [V],
  // E = 2^E_exp[v] * value(codes); null: the logits pass reads E (then E is not read at all)
  const uint8_t* E8;
  const int32_t* E_exp;
  // FP8 hidden states (with E8): E4M3 codes [R, d] and row exponents [R] of h, quantised per
  // row when the pass runs; the logits pass then multiplies codes by codes on FP8 MFMA
  const uint8_t* h8;
  const int32_t* h_exp;
  // the expectation pass's operand: the embedding as fp16 in the expectation MFMA's B-fragment
  // order (embedding_f16.hip), e16_rows(V) x d entries, zero past V (required with selfcond)
  const uint16_t* E16;
};

// Rows of the fp16 embedding: the vocabulary padded to whole 256-entry tiles.
inline int e16_rows(int V) { return (V + 255) / 256 * 256; }
inline size_t e16_bytes(int V, int d) { return (size_t)e16_rows(V) * (size_t)d * 2; }
hipError_t e16_launch(const uint16_t* E, int V, int d, uint16_t* E16, hipStream_t stream);
hipError_t e16_fp8_launch(const uint8_t* codes, const int32_t* kexp, int V, int d,
                          uint16_t* E16, hipStream_t stream);

// The vocabulary pass (vocab_gemm.hip): two GEMMs over the same E, d % 128 == 0.
struct GemmPlan {
  size_t R;
  int n_tiles;    // vocabulary tiles of 256
  size_t vpad;    // n_tiles * 256
  int ncb;        // 16-column blocks per wave of the expectation pass
  int n_range;    // vocabulary ranges of the expectation pass
  int n_colblk;   // column blocks of the expectation pass
  int n_rounds;   // canvas rounds of the logits pass (256 workgroups each)
  int n_units_xcd;  // expectation units per XCD at most (pair-per-XCD mapping)
  int n_units;      // expectation units (flat mapping)
  int flat;         // 1: flat unit mapping
  int gmax;         // largest canvas round of the logits pass
  int st_stride;    // statistic slots per row
  size_t off_small, off_P, off_ref, off_st, off_accp, off_accM, off_fac;
  size_t bytes;
};
bool gemm_supported(int d);
GemmPlan gemm_plan(int n_canvas, int V, int d);
hipError_t gemm_launch(const VocabArgs& a, const GemmPlan& p, void* workspace,
                       hipStream_t stream);

struct AcceptArgs {
  const float* entropy;
  const int32_t* argmax_tok;
  const int32_t* gumbel_tok;
  const uint8_t* commit;
  int n_canvas;
  int V;
  float budget;
  float confidence;
  int stability;
  uint32_t k0, k1;
  const int32_t* step;
  int32_t* prev_argmax;
  int32_t* stable_count;
  int32_t* next_tokens;
  uint8_t* accept_mask;
  uint8_t* converged;
  float* mean_entropy;
};
hipError_t accept_renoise_launch(const AcceptArgs& a, hipStream_t stream);

// Self-conditioning consumer (selfcond_ffw.hip).
struct FfwArgs {
  const float* sc;          // [R, D] or null (first decode step)
  const int32_t* tokens;    // [R]
  const uint16_t* E;        // [V, D]
  const uint16_t* pre_norm; // [D]
  const uint16_t* W_gate;   // [F, D]
  const uint16_t* W_up;     // [F, D]
  const uint16_t* W_down;   // [D, F]
  const uint8_t* commit;    // [n_canvas] or null
  int V, D, F;
  float eps;
  uint16_t* out;            // [R, D]
};
struct FfwPlan {
  size_t R;
  size_t off_x1, off_y, off_res;
  size_t bytes;
};
FfwPlan ffw_plan(int n_canvas, int D, int F);
hipError_t ffw_launch(const FfwArgs& a, const FfwPlan& p, void* workspace, hipStream_t stream);

// DiffusionGemma-Lite sampler step (lite_sampler.hip).
struct LiteArgs {
  const uint16_t* h;
  const uint16_t* E;
  const float* temperature;
  const float* lse;
  const float* entropy;
  const int32_t* argmax_tok;
  const int32_t* gumbel_tok;
  int R, V, d;
  float softcap;      // 0: none
  float threshold;
  int stability_steps;  // 0: adaptive stop off
  uint32_t k0, k1;
  const int32_t* step;
  float* conf;
  int32_t* x;
  int32_t* prev_argmax;
  float* prev_conf;
  uint8_t* committed;
  int32_t* stable_count;
  int32_t* final_tokens;
  uint8_t* converged;
  float* mean_entropy;
};
hipError_t lite_step_launch(const LiteArgs& a, hipStream_t stream);

// FP8 embedding (fp8.hip): E4M3 codes with one power-of-two scale per row.
hipError_t fp8_quantize_launch(const uint16_t* E, int V, int d, uint8_t* codes, int32_t* kexp,
                               hipStream_t stream);

hipError_t q_sample_launch(const int32_t* x0, int n_canvas, int V, const float* kappa,
                           uint32_t k0, uint32_t k1, int32_t* xt, hipStream_t stream);

}  // namespace dg
