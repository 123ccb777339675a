/* dg.h -- C ABI of libdg.so: the per-step hot path of uniform-state block-diffusion
 * decoding over 256-position canvases with a tied embedding, for AMD MI355X (gfx950).
 *
 * Sources of the operations (web pages; cited by title and section):
 *  [TR]   "DiffusionGemma Technical Report -- part 2/6": sec. 2.1.1 eq. (1) forward process,
 *         sec. 3.2 eq. (5)-(6) denoising iteration, sec. 3.3 entropy-bounded sampler,
 *         temperature annealing and adaptive stopping.
 *  [EXP]  "DiffusionGemma Explained": "Sampling" (temperature, entropy, low-entropy prefix,
 *         renoise, early stop), "Lazy Sampling", tied embeddings and self-conditioning.
 *  [VLLM] "DiffusionGemma: the first dLLM natively supported in vLLM": the sampler step
 *         (Gumbel-max candidate, entropy bound, renoise, argmax record, convergence) and
 *         per-request state kept in preallocated GPU tensors.
 *  [LITE] "DiffusionGemma-Lite DIFFUSION.html": closed-form forward corruption (q_sample),
 *         chunked p@E and chunked logsumexp (prior art for the split-vocabulary combine).
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless marked [host].  The caller owns every buffer; the
 *    library keeps no pointer past the call and allocates nothing.  Buffers must stay valid
 *    until the work queued on `stream` has completed.
 *  - Work is queued on `stream` (a hipStream_t; 0 = the null stream) and the call returns
 *    without waiting for it.  No call synchronises the device.
 *  - Arguments are validated on the host before anything is queued.  On a validation error
 *    nothing is queued and no output is written; dg_last_error() describes the error.
 *  - Values the host cannot check without a device read (non-finite E or h, temperature <= 0,
 *    token ids outside [0, V)) give unspecified outputs but never out-of-bounds accesses
 *    of the caller's buffers.
 *  - Layouts: bf16 is IEEE binary32 truncated to its top 16 bits, stored as uint16_t.
 *    Row r = c * C + i is position i of canvas c.  All matrices are row-major.
 *  - Random numbers: Philox4x32-10 (Salmon et al., SC'11) with key (seed & 0xffffffff,
 *    seed >> 32).  Counters: Gumbel noise of (row r, vocab v) at step s: (v >> 2, r, s,
 *    0x47554D42), word v & 3; renoise token of row r at step s: (0, r, s, 0x52454E4F),
 *    word 0; q_sample of row r: (0, r, 0, 0x51534D50), words 0 (keep test) and 1 (token).
 *    Uniform in (0,1): u = ((x >> 9) + 0.5) * 2^-23.  Uniform token: (x * V) >> 32.
 *  - The library is thread-safe; calls on different streams may overlap.
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = 1, /* NULL required pointer, bad size, non-finite scalar */
  DG_ERR_UNSUPPORTED = 2, /* valid but not implemented (C != 256, d % 128 != 0, ...) */
  DG_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than dg_vocab_pass_workspace_size */
  DG_ERR_HIP = 4          /* a HIP runtime call failed; see dg_last_error() */
} dg_status;

/* Size limits checked by every entry point. */
#define DG_CANVAS 256        /* positions per canvas (the only supported C) */
#define DG_MAX_D 8192        /* largest hidden width */
#define DG_MAX_CANVASES 4096 /* largest number of canvases per call */
#define DG_MAX_V (1 << 26)   /* largest vocabulary */

/* Bytes of device workspace dg_vocab_pass, dg_vocab_pass_softcap and dg_vocab_pass_fp8 need
 * for this shape ([host], pure function; 0 for a shape they would reject).  It includes room
 * for the fp16 embedding the expectation multiplies (see dg_embedding_f16), which
 * these entry points build in the workspace when the expectation is asked for. */
size_t dg_vocab_pass_workspace_size(int n_canvas, int C, int V, int d);

/* As dg_vocab_pass_workspace_size, for dg_vocab_pass_ex: with_e16 != 0 when the caller
 * passes its own E16 (then no room for one is needed), 0 otherwise. */
size_t dg_vocab_pass_ex_workspace_size(int n_canvas, int C, int V, int d, int with_e16);

/* dg_embedding_f16 -- the embedding in the form the self-conditioning expectation multiplies:
 * fp16 (round to nearest even), the vocabulary padded with zero entries to DG_E16_ROWS(V), in
 * the B-fragment order of the expectation's MFMA: for the entry block b (entries 32 b ..
 * 32 b + 31) and the column block c (columns 16 c .. 16 c + 15), the 1,024-byte block at byte
 * offset (b * (d / 16) + c) * 1024 holds fp16(E[32 b + 8 g + e, 16 c + n]) at byte
 * 16 (n + 16 g) + 2 e (n < 16, g < 4, e < 8); entries V .. DG_E16_ROWS(V) - 1 are 0.  The
 * expectation sum_v p_v E_v ([TR] eq. (6)) runs on fp16 MFMA because probability weights in
 * bf16 (8 significant bits) leave a relative error of about 1e-3 in the expectation of a flat
 * distribution, at the 2e-3 bar; fp16 has 11 bits.  The embedding is constant across denoising
 * steps: a caller builds this once (like the FP8 codes) and hands it to dg_vocab_pass_ex; the
 * other entry points build it per call.
 *  E      [V, d] bf16, |E| < 65504 (larger values give unspecified expectation rows).
 *  V      1 .. DG_MAX_V;  d: multiple of 128, 128 .. DG_MAX_D.
 *  E16    DG_E16_ROWS(V) * d uint16 (fp16 bits) out, dg_embedding_f16_bytes(V, d) bytes.
 *  E and E16 16-byte aligned.
 * Errors: DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_HIP. */
#define DG_E16_ROWS(V) ((((V) + 255) / 256) * 256)
size_t dg_embedding_f16_bytes(int V, int d);
dg_status dg_embedding_f16(const uint16_t* E, int V, int d, uint16_t* E16, void* stream);

/* dg_vocab_pass -- the vocabulary pass of one denoising step.
 *
 * For each row r (canvas c = r / C) with logits S[r, v] = sum_k h[r, k] E[v, k] (the tied
 * embedding used as the unembedding, [TR] eq. (5); [EXP] tied embeddings) and tempered
 * logits z = S / temperature[c] ([TR] eq. (6); [EXP] "Apply temperature"):
 *   lse[r]        = log sum_v exp(z_v)
 *   entropy[r]    = -sum_v p_v log p_v,  p = softmax(z)            ([EXP] "Compute entropy")
 *   argmax_tok[r] = smallest v attaining max_v S[r, v]              ([VLLM] clean argmax)
 *   gumbel_tok[r] = smallest v attaining max_v (z_v + g_v), g = -ln(-ln u) with u from the
 *                   Gumbel counter of (r, v, step[c])                ([VLLM] Gumbel-max)
 *   selfcond[r,:] = sum_v p_v E[v, :]                    ([TR] eq. (6), the argument of FFW)
 * The [R, V] logits are never written to memory; with selfcond, fp16 probability weights
 * 2^(z2 - ref) (each relative to its row's 128-entry reference) pass through the workspace
 * between the logits and the expectation contractions.  For a commit canvas (commit[c] != 0)
 * only argmax_tok is written; its rows of lse, entropy, gumbel_tok and selfcond are untouched.
 *
 *  E            [V, d] bf16, read only.
 *  h            [n_canvas * C, d] bf16 final hidden states, read only.
 *  n_canvas     1 .. DG_MAX_CANVASES.   C: must be DG_CANVAS.
 *  V            1 .. DG_MAX_V.   d: 128 .. DG_MAX_D, multiple of 128.
 *  temperature  [n_canvas] fp32, > 0.
 *  commit       [n_canvas] uint8 or NULL (no canvas commits).
 *  seed         Philox key.   step: [n_canvas] int32 step ids (third Gumbel counter word).
 *  lse          [R] fp32 or NULL.    entropy: [R] fp32 (nats).
 *  argmax_tok   [R] int32.           gumbel_tok: [R] int32.
 *  selfcond     [R, d] fp32 or NULL (then the expectation is not computed).  The expectation
 *               multiplies fp16 probability weights by the fp16 embedding (dg_embedding_f16,
 *               built here in the workspace when selfcond is given).
 *  workspace    device scratch of at least dg_vocab_pass_workspace_size(n_canvas, C, V, d)
 *               bytes; its contents on entry do not matter and are clobbered.
 * Errors: DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_WORKSPACE, DG_ERR_HIP. */
dg_status dg_vocab_pass(const uint16_t* E, const uint16_t* h, int n_canvas, int C, int V, int d,
                        const float* temperature, const uint8_t* commit, uint64_t seed,
                        const int32_t* step, float* lse, float* entropy, int32_t* argmax_tok,
                        int32_t* gumbel_tok, float* selfcond, void* workspace,
                        size_t workspace_bytes, void* stream);

/* dg_vocab_pass_softcap -- dg_vocab_pass with the final-logit soft cap of the model's logits
 * path applied before the temperature ([EXP] final logits: the raw logits are capped to
 * (-softcap, softcap) by softcap * tanh(S / softcap), then divided by the temperature;
 * [TR] sec. 3.3 temperature schedule, the temperature being the caller's per canvas):
 *   z = softcap * tanh(S / softcap) / temperature[c]
 * replaces z = S / temperature[c] in lse, entropy, the Gumbel-max sample and the
 * self-conditioning weights; argmax_tok stays the smallest v attaining max S (the cap is
 * increasing, so it is also the argmax of the capped logits).  All other arguments, layouts
 * and outputs as dg_vocab_pass.
 *  softcap      > 0 and finite ([host] scalar; the pages do not print its value).
 * Errors: as dg_vocab_pass; DG_ERR_INVALID_ARG for a softcap that is not finite and > 0. */
dg_status dg_vocab_pass_softcap(const uint16_t* E, const uint16_t* h, int n_canvas, int C, int V,
                                int d, const float* temperature, const uint8_t* commit,
                                uint64_t seed, const int32_t* step, float* lse, float* entropy,
                                int32_t* argmax_tok, int32_t* gumbel_tok, float* selfcond,
                                void* workspace, size_t workspace_bytes, void* stream,
                                float softcap);

/* dg_vocab_pass_ex -- dg_vocab_pass_softcap (softcap > 0) or dg_vocab_pass (softcap = 0) whose
 * Gumbel-max draw may use its own temperature and whose expectation may take a prepared
 * fp16 embedding.  The statistics (lse, entropy, selfcond) describe
 * p = softmax(cap(S) / temperature[c]); the sample is
 *   gumbel_tok[r] = smallest v attaining max_v (cap(S_v) / draw_temperature[c] + g_v)
 * with the same noise g as dg_vocab_pass.  This is the DiffusionGemma-Lite sampler's split
 * ([LITE] sec. 4.2 "The commit rule": the posterior p = softmax(logits) that the commit rule
 * and the stop entropy of sec. 4.4 read is untempered, and only the x0-hat draw of step k
 * uses the annealed temperature tau(k), item 4): call it with temperature = 1 and
 * draw_temperature = tau(k).  draw_temperature = NULL draws at `temperature`, which is
 * dg_vocab_pass_softcap / dg_vocab_pass exactly (same bits).
 *  E16               dg_embedding_f16(E) or NULL (then built in the workspace when selfcond
 *                    is given); the same values either way.
 *  draw_temperature  [n_canvas] fp32, > 0, or NULL.
 *  softcap           0 (no cap) or > 0 and finite ([host] scalar).
 *  workspace         dg_vocab_pass_ex_workspace_size(n_canvas, C, V, d, E16 != NULL) bytes.
 * Other arguments, layouts and outputs as dg_vocab_pass.
 * Errors: as dg_vocab_pass_softcap. */
dg_status dg_vocab_pass_ex(const uint16_t* E, const uint16_t* E16, const uint16_t* h,
                           int n_canvas, int C, int V, int d, const float* temperature,
                           const float* draw_temperature, float softcap, const uint8_t* commit,
                           uint64_t seed, const int32_t* step, float* lse, float* entropy,
                           int32_t* argmax_tok, int32_t* gumbel_tok, float* selfcond,
                           void* workspace, size_t workspace_bytes, void* stream);

/* dg_vocab_pass_ex_noalloc -- dg_vocab_pass_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument and no allocation.  The pass runs in a static device array of
 * DG_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs on until the
 * process ends (its address is looked up once per device, on the first call with that device
 * current).  Shapes whose dg_vocab_pass_ex_workspace_size(n_canvas, C, V, d, E16 != NULL)
 * exceeds it fail with DG_ERR_WORKSPACE before anything is launched.  Every call on one GPU
 * uses that GPU's one array: calls that may overlap on a GPU (different streams, or threads
 * without ordering) race and give undefined results; calls ordered on one stream are safe.
 * Arguments, layouts, outputs and results (bit for bit) as dg_vocab_pass_ex.
 * Errors: as dg_vocab_pass_ex. */
#define DG_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dg_status dg_vocab_pass_ex_noalloc(const uint16_t* E, const uint16_t* E16, const uint16_t* h,
                                   int n_canvas, int C, int V, int d, const float* temperature,
                                   const float* draw_temperature, float softcap,
                                   const uint8_t* commit, uint64_t seed, const int32_t* step,
                                   float* lse, float* entropy, int32_t* argmax_tok,
                                   int32_t* gumbel_tok, float* selfcond, void* stream);

/* dg_quantize_embedding_fp8 -- the tied embedding as FP8 ([VLLM] ships an FP8 checkpoint with
 * quantised weights; the pages give no scale scheme): OCP E4M3 codes (bias 7, largest finite
 * 448, no infinities) with one power-of-two scale 2^k per row,
 *   k_v = the smallest integer >= -117 with max_j |E_vj| <= 448 * 2^k_v (-117 for a zero row)
 *   codes_vj = the E4M3 value nearest to E_vj / 2^k_v, ties to the even code (zero -> 0x00).
 * A power-of-two scale makes every dequantised value 2^k * value(code) an exact bf16 number.
 *  E        [V, d] bf16, finite, |E| < 2^127.   d % 128 == 0, 128 <= d <= DG_MAX_D.
 *  codes    [V, d] uint8 out;  row_exp [V] int32 out.
 *  E16      DG_E16_ROWS(V) * d fp16 out (the layout of dg_embedding_f16), or NULL: the
 *           expectation pass's operand built from the dequantised rows (dg_embedding_f16 of E~
 *           below).
 *  E, codes and E16 16-byte aligned.
 * Errors: DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_HIP. */
dg_status dg_quantize_embedding_fp8(const uint16_t* E, int V, int d, uint8_t* codes,
                                    uint16_t* E16, int32_t* row_exp, void* stream);

/* dg_vocab_pass_fp8_workspace_size -- bytes of workspace dg_vocab_pass_fp8 needs ([host],
 * pure; 0 if unsupported): as dg_vocab_pass_workspace_size. */
size_t dg_vocab_pass_fp8_workspace_size(int n_canvas, int C, int V, int d);

/* dg_vocab_pass_fp8 -- dg_vocab_pass (dg_vocab_pass_softcap when softcap > 0) on the FP8
 * embedding (codes, row_exp, and E16) of dg_quantize_embedding_fp8: the embedding is
 * E~_vj = 2^row_exp[v] * value(codes_vj), and the logits, statistics, samples and
 * self-conditioning expectation are those of E~.  The logits pass streams the codes and
 * scales each entry's sum by 2^row_exp[v] (exact); the expectation multiplies E16 (built from
 * the codes in the workspace when NULL and selfcond is given).  Results equal those of
 * dg_vocab_pass on E~ up to the order of fp32 accumulation.  softcap: 0 (none) or finite > 0.
 * Other arguments, outputs and errors as dg_vocab_pass; codes and row_exp 16-byte aligned. */
dg_status dg_vocab_pass_fp8(const uint8_t* codes, const uint16_t* E16, const int32_t* row_exp,
                            const uint16_t* h,
                            int n_canvas, int C, int V, int d, const float* temperature,
                            const uint8_t* commit, uint64_t seed, const int32_t* step,
                            float* lse, float* entropy, int32_t* argmax_tok,
                            int32_t* gumbel_tok, float* selfcond, void* workspace,
                            size_t workspace_bytes, void* stream, float softcap);

/* dg_vocab_pass_fp8_dyn_workspace_size -- bytes of workspace dg_vocab_pass_fp8_dyn needs
 * ([host], pure; 0 if unsupported): dg_vocab_pass_fp8_workspace_size plus room for the
 * quantised hidden states (n_canvas C d bytes of codes and n_canvas C exponents). */
size_t dg_vocab_pass_fp8_dyn_workspace_size(int n_canvas, int C, int V, int d);

/* dg_vocab_pass_fp8_dyn -- dg_vocab_pass_fp8 with the hidden states in FP8 as well ([VLLM]:
 * an FP8 checkpoint with quantised weights and dynamic activations).  Each row of h is
 * quantised when the pass runs, by the rule of dg_quantize_embedding_fp8 applied to that row
 * alone (E4M3 codes, power-of-two scale 2^kh_r), and the logits are those of the dequantised
 * rows: S~[r, v] = 2^(kh_r + row_exp[v]) sum_j value(hq_rj) value(codes_vj), multiplied code by
 * code on FP8 MFMA with both scales applied by the MFMA.  The MFMA sums each 64-wide block of
 * products with an error of up to about 2^-12 of the block's largest product (its own
 * rounding, not fp32's), so S~ is met to that accuracy rather than to fp32 rounding; the
 * statistics, samples and expectation follow from it as in dg_vocab_pass.
 *  workspace  dg_vocab_pass_fp8_dyn_workspace_size(n_canvas, C, V, d) bytes.
 * Other arguments, layouts, outputs and errors as dg_vocab_pass_fp8. */
dg_status dg_vocab_pass_fp8_dyn(const uint8_t* codes, const uint16_t* E16,
                                const int32_t* row_exp, const uint16_t* h, int n_canvas, int C,
                                int V, int d, const float* temperature, const uint8_t* commit,
                                uint64_t seed, const int32_t* step, float* lse, float* entropy,
                                int32_t* argmax_tok, int32_t* gumbel_tok, float* selfcond,
                                void* workspace, size_t workspace_bytes, void* stream,
                                float softcap);

/* dg_accept_renoise -- per-canvas acceptance, renoising and convergence of one step.
 *
 * For a canvas that does not commit ([TR] sec. 3.3 "Entropy-bounded token refinement",
 * "Adaptive stopping heuristic"; [EXP] "Keep a low-entropy prefix and renoise the rest",
 * "Check for early stopping"; [VLLM] sampler step):
 *   order its C positions by (entropy, position) ascending; position of rank k is accepted
 *   iff the entropies of ranks 0..k-1 sum to <= entropy_budget (rank 0 always accepted);
 *   next_tokens = accepted ? gumbel_tok : uniform token from the renoise counter (r, step[c]);
 *   stable = (argmax_tok == prev_argmax at every position); stable_count = stable ?
 *   stable_count + 1 : 0; prev_argmax = argmax_tok; mean_entropy = mean of the C entropies;
 *   converged = stable_count >= stability_threshold && mean_entropy < confidence_threshold.
 *   The prefix sums and the mean are taken in fp64.
 * A commit canvas ([VLLM] commit emits the clean argmax): next_tokens = argmax_tok,
 * accept_mask = 1, prev_argmax = -1, stable_count = 0, converged = 0, mean_entropy untouched.
 *
 *  entropy, argmax_tok, gumbel_tok  [R] inputs as produced by dg_vocab_pass (entropy and
 *               gumbel_tok are not read for commit canvases).
 *  commit       [n_canvas] uint8 or NULL.     V: vocabulary size (renoise range).
 *  entropy_budget >= 0 and finite;  confidence_threshold finite;  stability_threshold >= 1.
 *  prev_argmax  [R] int32 in/out (-1 = no previous canvas).  stable_count: [n_canvas] in/out.
 *  next_tokens  [R] int32 out.   accept_mask: [R] uint8 out or NULL.
 *  converged    [n_canvas] uint8 out.   mean_entropy: [n_canvas] fp32 out or NULL.
 * Errors: DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_HIP. */
dg_status dg_accept_renoise(const float* entropy, const int32_t* argmax_tok,
                            const int32_t* gumbel_tok, const uint8_t* commit, int n_canvas, int C,
                            int V, float entropy_budget, float confidence_threshold,
                            int stability_threshold, uint64_t seed, const int32_t* step,
                            int32_t* prev_argmax, int32_t* stable_count, int32_t* next_tokens,
                            uint8_t* accept_mask, uint8_t* converged, float* mean_entropy,
                            void* stream);

/* dg_lite_step -- the DiffusionGemma-Lite sampler step, a second sampler on the vocabulary
 * pass outputs ([LITE] sec. 4.2 "The commit rule", sec. 4.4 "Entropy-bounded adaptive
 * stopping").  Per row r of canvas c, with conf_r the probability of the argmax token under
 * the distribution the pass's statistics describe, exp(z_am - lse_r), z_am =
 * cap(h_r . E[am]) / T_c (cap(S) = softcap tanh(S / softcap), or S when softcap == 0).  The
 * page's posterior is untempered (p = softmax(logits); only the x0-hat draw uses the annealed
 * tau(k)), so the pass for this sampler is dg_vocab_pass_ex with temperature = 1 and
 * draw_temperature = tau(k), and T_c here is that statistics temperature (1):
 *   commit = (argmax_tok == prev_argmax) || (conf >= prev_conf)   (unchanged-or-stronger)
 *   fresh  = commit && !committed                                 (frozen tokens stay)
 *   x      = fresh ? gumbel_tok : committed ? x : uniform token of the renoise counter
 *            (r, step[c]);  committed |= fresh;  prev_argmax = argmax_tok;  prev_conf = conf
 *   final_tokens = committed ? x : gumbel_tok                       (the returned canvas)
 * and per canvas the fp64 mean entropy m: with stability_steps > 0, stable_count = m <
 * entropy_threshold ? stable_count + 1 : 0 and converged = stable_count >= stability_steps;
 * with stability_steps == 0 (adaptive stop off) converged = 0 and stable_count is untouched.
 * Initial state (no previous posterior, nothing commits at the first step): prev_argmax = -1,
 * prev_conf = +inf, committed = 0, stable_count = 0.
 *  h, E, temperature, lse, entropy, argmax_tok, gumbel_tok: the vocabulary pass's inputs and
 *            outputs of the step (temperature: the statistics temperature the pass was given;
 *            lse, entropy, gumbel_tok of every row must be written: no commit canvases);
 *            softcap: the value given to the pass, else 0.
 *  entropy_threshold finite; stability_steps >= 0.
 *  conf      [R] fp32 out.   x, prev_argmax [R] int32 in/out; prev_conf [R] fp32 in/out;
 *  committed [R] uint8 in/out; stable_count [n_canvas] in/out; final_tokens [R] out or NULL;
 *  converged [n_canvas] uint8 out; mean_entropy [n_canvas] fp32 out or NULL.
 *  h and E 16-byte aligned.  An argmax outside [0, V) gives conf = NaN (never commits by the
 *  confidence test).
 * Errors: DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_HIP. */
dg_status dg_lite_step(const uint16_t* h, const uint16_t* E, const float* temperature,
                       const float* lse, const float* entropy, const int32_t* argmax_tok,
                       const int32_t* gumbel_tok, int n_canvas, int C, int V, int d,
                       float softcap, float entropy_threshold, int stability_steps,
                       uint64_t seed, const int32_t* step, float* conf, int32_t* x,
                       int32_t* prev_argmax, float* prev_conf, uint8_t* committed,
                       int32_t* stable_count, int32_t* final_tokens, uint8_t* converged,
                       float* mean_entropy, void* stream);

/* dg_q_sample -- closed-form forward corruption ([TR] sec. 2.1.1 eq. (1); [LITE] forward
 * process, one draw, never iterating the chain): row r of canvas c keeps x0[r] iff
 * (w0 >> 8) < floor(kappa[c] * 2^24), else takes the uniform token of w1, with (w0, w1)
 * the q_sample counter words of r.  P(xt = x0) = kappa + (1 - kappa) / V up to the 24-bit
 * quantisation of kappa.
 *  x0     [n_canvas * C] int32 clean tokens.   kappa: [n_canvas] fp32 in [0, 1].
 *  xt     [n_canvas * C] int32 out (may not alias x0).
 * Errors: DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_HIP. */
dg_status dg_q_sample(const int32_t* x0, int n_canvas, int C, int V, const float* kappa,
                      uint64_t seed, int32_t* xt, void* stream);

/* dg_selfcond_input_workspace_size -- bytes of workspace dg_selfcond_input needs ([host],
 * pure): 256-byte aligned buffers for x1 [R, D] bf16, y [R, F] bf16 and res [R, D] fp32,
 * R = n_canvas * C.  0 for an unsupported shape. */
size_t dg_selfcond_input_workspace_size(int n_canvas, int C, int D, int F);

/* dg_selfcond_input -- the next decode step's input rows: the renoised tokens' embeddings
 * plus the self-conditioning signal, normalised ([EXP] "Self-conditioning" and the decode
 * forward: the expectation P @ E scaled by sqrt(D), passed through the conditioning MLP,
 * added to the scaled token embedding, RMS-normalised; the conditioning MLP is the gated
 * GELU MLP of [EXP] "Mixture of Experts" with a weighted pre-norm; RMSNorm as in [EXP]
 * "RMSNorm", eps added to the row norm; [TR] sec. 3.2 eq. (6) FFW(p_hat_0 E)):
 *   cx  = sc * sqrt(D)
 *   x1  = bf16(pre_norm * cx * sqrt(D) / (||cx||_2 + eps))
 *   y   = bf16((x1 W_up^T) * GELU(x1 W_gate^T)),  GELU(x) = x (1 + erf(x / sqrt 2)) / 2
 *   res = y W_down^T                                   (fp32)
 *   out = bf16(x * sqrt(D) / (||x||_2 + eps)),  x = E[tokens] * sqrt(D) + res
 * bf16 MFMA products with fp32 accumulation; norms and elementwise work in fp32.
 *  sc        [R, D] fp32 (dg_vocab_pass's selfcond), or NULL on the first decode step: the
 *            MLP maps zero to zero, so res = 0 and W_* and pre_norm are not read.
 *  tokens    [R] int32 renoised tokens (dg_accept_renoise's next_tokens); a token outside
 *            [0, V) gives a row of NaN.
 *  E         [V, D] bf16 tied embedding.   pre_norm: [D] bf16 weight of the MLP's pre-norm.
 *  W_gate, W_up [F, D] bf16; W_down [D, F] bf16 (rows are output features).
 *  commit    [n_canvas] uint8 or NULL: the rows of a commit canvas are neither read nor
 *            written.
 *  C == 256; D % 64 == 0, 64 <= D <= 16384; F % 64 == 0, 64 <= F <= 65536; eps >= 0 finite.
 *  out       [R, D] bf16 (may not alias any input).   Every pointer 16-byte aligned.
 *  workspace of dg_selfcond_input_workspace_size bytes, 256-byte aligned.
 * Errors: DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_WORKSPACE, DG_ERR_HIP. */
dg_status dg_selfcond_input(const float* sc, const int32_t* tokens, const uint16_t* E,
                            const uint16_t* pre_norm, const uint16_t* W_gate,
                            const uint16_t* W_up, const uint16_t* W_down,
                            const uint8_t* commit, int n_canvas, int C, int V, int D, int F,
                            float eps, uint16_t* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Static text of a status code ([host]). */
const char* dg_status_string(dg_status s);
/* Message of the last error raised on the calling host thread ([host], thread-local; "" if
 * none).  Valid until the next dg_* call on that thread. */
const char* dg_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DG_H_ */
