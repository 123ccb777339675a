// Host-side driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI's
// validation: every entry point is called with arguments it must refuse (and the workspace-size
// functions with shapes at and beyond their limits), so that the checks, the size arithmetic
// and the error-message formatting run under the sanitizers.  No call reaches the device:
// every one of them fails validation on the host first.  Prints one line per failed
// expectation and exits with the number of failures.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dg.h"

static int g_bad = 0;

#define EXPECT(cond)                                                                       \
  do {                                                                                     \
    if (!(cond)) {                                                                         \
      std::printf("FAILED line %d: %s (last error: %s)\n", __LINE__, #cond, dg_last_error()); \
      ++g_bad;                                                                             \
    }                                                                                      \
  } while (0)

int main() {
  // distinct, 256-byte aligned, never dereferenced: every call below is refused on the host
  char* const base = reinterpret_cast<char*>(uintptr_t(1) << 40);
  auto P = [&](int i) { return static_cast<void*>(base + (size_t)i * 4096); };
  const uint16_t* E = static_cast<const uint16_t*>(P(1));
  const uint16_t* h = static_cast<const uint16_t*>(P(2));
  const float* T = static_cast<const float*>(P(3));
  const int32_t* st = static_cast<const int32_t*>(P(4));
  float* f = static_cast<float*>(P(5));
  int32_t* i32 = static_cast<int32_t*>(P(6));
  uint8_t* u8 = static_cast<uint8_t*>(P(7));
  void* ws = P(8);

  // sizes: limits, one past them, and the largest shapes (no overflow in the size arithmetic)
  EXPECT(dg_vocab_pass_workspace_size(DG_MAX_CANVASES, 256, DG_MAX_V, DG_MAX_D) > 0);
  EXPECT(dg_vocab_pass_workspace_size(DG_MAX_CANVASES + 1, 256, 4096, 256) == 0);
  EXPECT(dg_vocab_pass_workspace_size(1, 256, DG_MAX_V + 1, 256) == 0);
  EXPECT(dg_vocab_pass_workspace_size(1, 256, 4096, DG_MAX_D + 128) == 0);
  EXPECT(dg_vocab_pass_workspace_size(1, 256, 4096, 192) == 0);
  EXPECT(dg_vocab_pass_workspace_size(0, 256, 4096, 256) == 0);
  EXPECT(dg_vocab_pass_workspace_size(-5, 256, 4096, 256) == 0);
  EXPECT(dg_vocab_pass_workspace_size(1, 255, 4096, 256) == 0);
  EXPECT(dg_vocab_pass_workspace_size(1, 256, -1, 256) == 0);
  EXPECT(dg_vocab_pass_ex_workspace_size(DG_MAX_CANVASES, 256, DG_MAX_V, DG_MAX_D, 1) > 0);
  EXPECT(dg_vocab_pass_fp8_dyn_workspace_size(DG_MAX_CANVASES, 256, DG_MAX_V, DG_MAX_D) >
         dg_vocab_pass_fp8_workspace_size(DG_MAX_CANVASES, 256, DG_MAX_V, DG_MAX_D));
  EXPECT(dg_embedding_f16_bytes(DG_MAX_V, DG_MAX_D) == (size_t)DG_MAX_V * DG_MAX_D * 2);
  EXPECT(dg_embedding_f16_bytes(0, 256) == 0);
  EXPECT(dg_selfcond_input_workspace_size(DG_MAX_CANVASES, 256, DG_MAX_D, 65536) > 0 ||
         dg_selfcond_input_workspace_size(DG_MAX_CANVASES, 256, DG_MAX_D, 65536) == 0);
  EXPECT(dg_selfcond_input_workspace_size(1, 256, 100, 256) == 0);

  // the vocabulary pass: shape, pointer, alignment, soft cap and workspace refusals
  const size_t big = (size_t)1 << 40;
  EXPECT(dg_vocab_pass(E, h, 1, 256, 4096, 192, T, nullptr, 0, st, f, f, i32, i32, nullptr, ws,
                       big, nullptr) == DG_ERR_UNSUPPORTED);
  EXPECT(dg_vocab_pass(nullptr, h, 1, 256, 4096, 256, T, nullptr, 0, st, f, f, i32, i32, nullptr,
                       ws, big, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_vocab_pass(E, h, 1, 256, 4096, 256, T, nullptr, 0, st, f, f, i32, i32, nullptr, ws,
                       16, nullptr) == DG_ERR_WORKSPACE);
  EXPECT(dg_vocab_pass(E, h, 1, 256, 4096, 256, T, nullptr, 0, st, f, f, i32, i32, nullptr,
                       static_cast<char*>(ws) + 16, big, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_vocab_pass(E + 1, h, 1, 256, 4096, 256, T, nullptr, 0, st, f, f, i32, i32, nullptr,
                       ws, big, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_vocab_pass(E, h, 1, 256, 0, 256, T, nullptr, 0, st, f, f, i32, i32, nullptr, ws, big,
                       nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_vocab_pass(E, h, DG_MAX_CANVASES + 1, 256, 4096, 256, T, nullptr, 0, st, f, f, i32,
                       i32, nullptr, ws, big, nullptr) == DG_ERR_INVALID_ARG);
  const float bad_caps[] = {-1.0f, 0.0f, INFINITY, NAN};
  for (float c : bad_caps)
    EXPECT(dg_vocab_pass_softcap(E, h, 1, 256, 4096, 256, T, nullptr, 0, st, f, f, i32, i32,
                                 nullptr, ws, big, nullptr, c) == DG_ERR_INVALID_ARG);
  EXPECT(dg_vocab_pass_ex(E, E + 1, h, 1, 256, 4096, 256, T, nullptr, 0.0f, nullptr, 0, st, f, f,
                          i32, i32, f, ws, big, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_vocab_pass_ex(E, nullptr, h, 1, 256, 4096, 256, T, nullptr, NAN, nullptr, 0, st, f,
                          f, i32, i32, f, ws, big, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_vocab_pass_ex_noalloc(E, nullptr, h, 32, 256, 262144, 2816, T, nullptr, 0.0f,
                                  nullptr, 0, st, f, f, i32, i32, f, nullptr) == DG_ERR_WORKSPACE);
  EXPECT(std::strstr(dg_last_error(), "static scratch") != nullptr);
  EXPECT(dg_vocab_pass_ex_noalloc(E, nullptr, h, 1, 256, 4096, 200, T, nullptr, 0.0f, nullptr, 0,
                                  st, f, f, i32, i32, f, nullptr) == DG_ERR_UNSUPPORTED);
  EXPECT(dg_embedding_f16(E, 4096, 192, nullptr, nullptr) == DG_ERR_UNSUPPORTED);
  EXPECT(dg_embedding_f16(nullptr, 4096, 256, static_cast<uint16_t*>(P(9)), nullptr) ==
         DG_ERR_INVALID_ARG);

  // FP8 entry points
  const uint8_t* codes = static_cast<const uint8_t*>(P(10));
  EXPECT(dg_quantize_embedding_fp8(E, 4096, 100, u8, nullptr, i32, nullptr) == DG_ERR_UNSUPPORTED);
  EXPECT(dg_quantize_embedding_fp8(E, 4096, 256, nullptr, nullptr, i32, nullptr) ==
         DG_ERR_INVALID_ARG);
  EXPECT(dg_vocab_pass_fp8(nullptr, nullptr, st, h, 1, 256, 4096, 256, T, nullptr, 0, st, f, f,
                           i32, i32, nullptr, ws, big, nullptr, 0.0f) == DG_ERR_INVALID_ARG);
  EXPECT(dg_vocab_pass_fp8_dyn(codes, nullptr, st, h, 1, 256, 4096, 256, T, nullptr, 0, st, f, f,
                               i32, i32, nullptr, ws, 16, nullptr, 0.0f) == DG_ERR_WORKSPACE);
  EXPECT(dg_vocab_pass_fp8_dyn(codes, nullptr, st, h, 1, 256, 4096, 256, T, nullptr, 0, st, f, f,
                               i32, i32, nullptr, ws, big, nullptr, -2.0f) == DG_ERR_INVALID_ARG);

  // sampler, q_sample, self-conditioning consumer, Lite step
  EXPECT(dg_accept_renoise(f, i32, i32, nullptr, 1, 128, 4096, 1.0f, 0.1f, 2, 0, st, i32, i32,
                           i32, u8, u8, f, nullptr) == DG_ERR_UNSUPPORTED);
  EXPECT(dg_accept_renoise(nullptr, i32, i32, nullptr, 1, 256, 4096, 1.0f, 0.1f, 2, 0, st, i32,
                           i32, i32, u8, u8, f, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_q_sample(i32, 1, 256, 0, f, 0, i32, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_q_sample(nullptr, 1, 256, 100, f, 0, i32, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_selfcond_input(f, i32, E, E, E, E, E, nullptr, 1, 256, 4096, 100, 256, 1e-6f,
                           static_cast<uint16_t*>(P(11)), ws, big, nullptr) != DG_OK);
  EXPECT(dg_selfcond_input(f, i32, E, E, E, E, E, nullptr, 1, 256, 4096, 256, 256, 1e-6f,
                           static_cast<uint16_t*>(P(11)), ws, 16, nullptr) == DG_ERR_WORKSPACE);
  EXPECT(dg_lite_step(h, E, T, f, f, i32, i32, 1, 256, 4096, 200, 0.0f, 0.5f, 2, 0, st, f, i32,
                      i32, f, u8, i32, i32, u8, f, nullptr) != DG_OK);
  EXPECT(dg_lite_step(nullptr, E, T, f, f, i32, i32, 1, 256, 4096, 256, 0.0f, 0.5f, 2, 0, st, f,
                      i32, i32, f, u8, i32, i32, u8, f, nullptr) == DG_ERR_INVALID_ARG);

  // status strings for every code, and one past them
  for (int s = 0; s <= 5; ++s) EXPECT(dg_status_string(static_cast<dg_status>(s)) != nullptr);
  std::printf("%d failed expectations\n", g_bad);
  return g_bad;
}
