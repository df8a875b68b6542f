// Host-side argument checks of every libmoe entry point, for a run under AddressSanitizer and
// UndefinedBehaviorSanitizer with no GPU: each call below is refused by its host-side validation
// before any device call (pointers are fake, never dereferenced), and the sizing functions are
// driven over normal, ragged, huge and degenerate shapes.  Exits 0 when every status matches;
// the sanitizers abort on the first report.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;

#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (int)(call);                                                       \
    if (got_ != (int)(want)) {                                                          \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
              got_, (int)(want));                                                       \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

int main() {
  void* F = (void*)(uintptr_t)(1u << 20);           // a fake, 16-byte aligned device pointer
  void* F2 = (void*)((uintptr_t)F + 2);
  void* F4 = (void*)((uintptr_t)F + 4);
  void* F8 = (void*)((uintptr_t)F + 8);
  float* Ff = (float*)F;
  int32_t* Fi = (int32_t*)F;
  const size_t BIG = (size_t)1 << 40;
  const moe_dtype BF = MOE_BF16, F32 = MOE_F32;
  const moe_gating G0 = MOE_GATE_SOFTMAX_TOPK;

  // status strings, including a value outside the enum
  for (int s = 0; s <= 5; ++s) {
    const char* str = moe_status_str((moe_status)s);
    if (!str || !strlen(str)) ++failures;
  }

  // workspace sizing over normal, ragged, degenerate and huge shapes
  const int shapes[][5] = {{4096, 4096, 14336, 8, 2}, {8192, 7168, 2048, 256, 8},
                           {32, 4096, 14336, 8, 2},   {1, 8, 8, 1, 1},
                           {257, 136, 264, 8, 2},     {2048, 512, 2048, 8, 1},
                           {0, 8, 8, 4, 2},           {4, 0, 8, 4, 2},
                           {1 << 20, 8, 8, 1024, 32}, {-5, 8, 8, 4, 2}};
  size_t acc = 0;
  for (const auto& s : shapes) {
    for (int dt = 0; dt < 2; ++dt) {
      acc += moe_workspace_bytes(s[0], s[1], s[2], s[3], s[4], (moe_dtype)dt);
      acc += moe_backward_workspace_bytes(s[0], s[1], s[2], s[3], s[4], (moe_dtype)dt);
      acc += moe_gathered_workspace_bytes(s[0], s[1], s[2], s[3], (moe_dtype)dt);
    }
    acc += moe_q_workspace_bytes(s[0], s[1], s[2], s[3], s[4], 8);
    acc += moe_q_workspace_bytes(s[0], s[1], s[2], s[3], s[4], 4);
  }
  EXPECT(moe_workspace_bytes(0, 1, 1, 1, 1, F32), 0);
  EXPECT(moe_backward_workspace_bytes(0, 4096, 14336, 8, 2, BF), 0);

  // moe_route
  EXPECT(moe_route(F, F, 0, 0, 0, 8, 4, 2, BF, G0, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0), MOE_ERR_ARG);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 4, 5, BF, G0, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0), MOE_ERR_ARG);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 4, 0, BF, G0, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0), MOE_ERR_ARG);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 4, 2, BF, (moe_gating)3, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0),
         MOE_ERR_ARG);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 4, 2, (moe_dtype)7, G0, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0),
         MOE_ERR_ARG);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 4, 2, BF, G0, 4, Ff, Fi, Ff, 0, 0, 0, 0, 0), MOE_ERR_ARG);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 4, 2, BF, G0, 0, 0, Fi, Ff, 0, 0, 0, 0, 0), MOE_ERR_ARG);
  EXPECT(moe_route(0, F, 0, 0, 4, 8, 4, 2, BF, G0, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0), MOE_ERR_ARG);
  EXPECT(moe_route(F4, F, 0, 0, 4, 8, 4, 2, BF, G0, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0), MOE_ERR_ARG);
  EXPECT(moe_route(F, F, Ff, 0, 4, 8, 4, 2, BF, G0, 1, Ff, Fi, Ff, 0, 0, 0, 0, 0), MOE_ERR_ARG);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 2000, 2, BF, G0, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 64, 33, BF, G0, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_route(F, F, 0, 0, 4, 12, 4, 2, BF, G0, 0, Ff, Fi, Ff, 0, 0, 0, 0, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 4, 2, BF, G0, 0, Ff, Fi, Ff, Ff, 0, 0, 0, 0), MOE_ERR_ARG);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 4, 2, BF, G0, 0, Ff, Fi, Ff, Ff, 0, F, 4, 0),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_route(F, F, 0, 0, 4, 8, 4, 2, BF, G0, 0, Ff, Fi, Ff, 0, 0, F2, BIG, 0), MOE_ERR_ARG);

  // moe_dispatch and moe_dispatch_noalloc
  EXPECT(moe_dispatch(Fi, 0, 4, 2, 0, Fi, Fi, Fi, Fi, Fi, F, 1 << 20, 0), MOE_ERR_ARG);
  EXPECT(moe_dispatch(Fi, 4, 4, 5, 0, Fi, Fi, Fi, Fi, Fi, F, 1 << 20, 0), MOE_ERR_ARG);
  EXPECT(moe_dispatch(Fi, 4, 4, 2, 0, Fi, Fi, Fi, Fi, Fi, 0, 1 << 20, 0), MOE_ERR_ARG);
  EXPECT(moe_dispatch(Fi, 4, 1025, 2, 0, Fi, Fi, Fi, Fi, Fi, F, 1 << 20, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_dispatch(Fi, 4, 4, 2, 0, Fi, Fi, Fi, Fi, Fi, F, 8, 0), MOE_ERR_WORKSPACE);
  EXPECT(moe_dispatch(Fi, 1 << 30, 4, 4, 0, Fi, Fi, Fi, Fi, Fi, F, BIG, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_dispatch_noalloc(0, 4, 4, 2, 0, Fi, Fi, Fi, Fi, Fi, 0), MOE_ERR_ARG);
  EXPECT(moe_dispatch_noalloc(Fi, 4, 4, 2, 0, Fi, Fi, 0, Fi, Fi, 0), MOE_ERR_ARG);
  EXPECT(moe_dispatch_noalloc(Fi, 4, 2000, 2, 0, Fi, Fi, Fi, Fi, Fi, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_dispatch_noalloc(Fi, 600000, 1024, 1, 0, Fi, Fi, Fi, Fi, Fi, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_dispatch_noalloc(Fi, 1 << 30, 8, 4, 0, Fi, Fi, Fi, Fi, Fi, 0), MOE_ERR_UNSUPPORTED);

  // moe_expert_ffn and its halves
  EXPECT(moe_expert_ffn(F, 0, Fi, 4, 8, 16, 4, 2, F, F, F, BF, F, F, 1 << 30, 0), MOE_ERR_ARG);
  EXPECT(moe_expert_ffn(F, Fi, Fi, 4, 12, 16, 4, 2, F, F, F, BF, F, F, 1 << 30, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_ffn(F, Fi, Fi, 4, 8, 20, 4, 2, F, F, F, BF, F, F, 1 << 30, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_ffn(F, Fi, Fi, 4, 8, 16, 4, 2, F, F, F, BF, F, F, 16, 0), MOE_ERR_WORKSPACE);
  EXPECT(moe_expert_ffn(F, Fi, Fi, 4, 8, 16, 4, 2, F, F, F, BF, F2, F, 1 << 30, 0), MOE_ERR_ARG);
  EXPECT(moe_expert_ffn(F, Fi, Fi, 4, 8, 16, 4, 2, F, F, F, (moe_dtype)5, F, F, 1 << 30, 0),
         MOE_ERR_ARG);
  EXPECT(moe_expert_ffn(F, Fi, Fi, 1 << 28, 4096, 14336, 8, 2, F, F, F, BF, F, F, BIG, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_up(F, Fi, Fi, 0, 8, 16, 4, 2, F, F, BF, F, F, 1 << 30, 0), MOE_ERR_ARG);
  EXPECT(moe_expert_up(F, Fi, Fi, 4, 8, 16, 4, 2, F, F, BF, F, F2, 1 << 30, 0), MOE_ERR_ARG);
  EXPECT(moe_expert_down(F, Fi, 4, 12, 16, 4, 2, F, BF, F, F, 1 << 30, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_down(F, Fi, 4, 8, 16, 4, 2, F, BF, F4, F, 1 << 30, 0), MOE_ERR_ARG);
  EXPECT(moe_expert_ffn_save(F, Fi, Fi, 4, 8, 16, 4, 2, F, F, F, F32, F, F, F, 1 << 30, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_ffn_save(F, Fi, Fi, 4, 8, 16, 4, 2, F, F, F, BF, F, 0, F, 1 << 30, 0),
         MOE_ERR_ARG);

  // combine, losses, balancing, transpose
  EXPECT(moe_combine(F, Fi, Ff, 0, 8, 2, BF, 0, F, 0), MOE_ERR_ARG);
  EXPECT(moe_combine(F, Fi, Ff, 4, 12, 2, BF, 0, F, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_combine(F, Fi, Ff, 4, 8, 2000, BF, 0, F, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_combine(0, Fi, Ff, 4, 8, 2, BF, 0, F, 0), MOE_ERR_ARG);
  EXPECT(moe_combine(F, Fi, Ff, 4, 8, 2, BF, F8, F, 0), MOE_ERR_ARG);
  EXPECT(moe_aux_loss(Fi, Ff, Ff, 0, 4, 2, 0.01f, 1e-3f, Ff, Ff, 0), MOE_ERR_ARG);
  EXPECT(moe_aux_loss(Fi, 0, Ff, 4, 4, 2, 0.01f, 1e-3f, Ff, Ff, 0), MOE_ERR_ARG);
  EXPECT(moe_aux_loss(Fi, Ff, Ff, 4, 2000, 2, 0.01f, 1e-3f, Ff, Ff, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_update_select_bias(0, 4, 4, 2, 0.01f, Ff, 0), MOE_ERR_ARG);
  EXPECT(moe_update_select_bias(Fi, 4, 2000, 2, 0.01f, Ff, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_transpose(0, 1, 4, 4, BF, F, 0), MOE_ERR_ARG);
  EXPECT(moe_transpose(F, 1, 4, -1, BF, F, 0), MOE_ERR_ARG);
  EXPECT(moe_transpose(F, 70000, 4, 4, BF, F, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_transpose(F, 1, 64 * 65536, 4, BF, F, 0), MOE_ERR_UNSUPPORTED);

  // backward
  EXPECT(moe_combine_backward(F, F, Fi, Ff, 0, 16, 2, BF, F, Ff, 0), MOE_ERR_ARG);
  EXPECT(moe_combine_backward(F2, F, Fi, Ff, 4, 16, 2, BF, F, Ff, 0), MOE_ERR_ARG);
  EXPECT(moe_combine_backward(F, F, Fi, Ff, 4, 16, 2, F32, F, Ff, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_combine_backward(F, F, Fi, Ff, 4, 12, 2, BF, F, Ff, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_combine_backward(F, F, Fi, Ff, 4, 16, 33, BF, F, Ff, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_backward(F, Fi, 0, 4, 16, 32, 4, 2, F, F, F, F, BF, F, Ff, Ff, Ff, F, BIG, 0),
         MOE_ERR_ARG);
  EXPECT(moe_expert_backward(F, 0, Fi, 4, 16, 32, 4, 2, F, F, F, F, BF, F, Ff, Ff, Ff, F, BIG, 0),
         MOE_ERR_ARG);
  EXPECT(moe_expert_backward(F, Fi, Fi, 4, 16, 32, 4, 2, F, F, F, F, F32, F, Ff, Ff, Ff, F, BIG,
                             0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_backward(F, Fi, Fi, 4, 16, 36, 4, 2, F, F, F, F, BF, F, Ff, Ff, Ff, F, BIG, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_backward(F, Fi, Fi, 4, 16, 32, 4, 2, F, F, F, F, BF, F, Ff, Ff, Ff, F, 16, 0),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_expert_backward_saved(0, F, Fi, Fi, 4, 16, 32, 4, 2, F, F, F, F, BF, F, Ff, Ff, Ff,
                                   F, BIG, 0),
         MOE_ERR_ARG);
  EXPECT(moe_route_backward(F, F, Ff, Fi, Ff, Ff, Fi, 0, 16, 4, 2, BF, G0, 0.01f, 1e-3f, 0, Ff, Ff,
                            F, F, BIG, 0),
         MOE_ERR_ARG);
  EXPECT(moe_route_backward(F, F, Ff, Fi, Ff, Ff, 0, 4, 16, 4, 2, BF, G0, 0.01f, 1e-3f, 0, Ff, Ff,
                            F, F, BIG, 0),
         MOE_ERR_ARG);
  EXPECT(moe_route_backward(F, F, Ff, Fi, Ff, Ff, Fi, 4, 12, 4, 2, BF, G0, 0.01f, 1e-3f, 0, Ff,
                            Ff, F, F, BIG, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_route_backward(F, F, Ff, Fi, Ff, Ff, Fi, 4, 16, 4, 2, BF, G0, 0.01f, 1e-3f, 0, Ff,
                            Ff, F, F, 16, 0),
         MOE_ERR_WORKSPACE);

  // variants: Expert Choice, gathered rows, rerouting, quantized experts
  EXPECT(moe_expert_choice(Ff, 0, 4, 2, 0, Ff, Fi, Fi, Ff, Fi, 0), MOE_ERR_ARG);
  EXPECT(moe_expert_choice(Ff, 8, 4, 0, 0, Ff, Fi, Fi, Ff, Fi, 0), MOE_ERR_ARG);
  EXPECT(moe_expert_choice(Ff, 8, 4, 2, 2, Ff, Fi, Fi, Ff, Fi, 0), MOE_ERR_ARG);
  EXPECT(moe_expert_choice(Ff, 8, 2000, 2, 0, Ff, Fi, Fi, Ff, Fi, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_ffn_gathered(F, Fi, Fi, 8, 16, 32, 4, 0, F, F, F, BF, F, F, BIG, 0),
         MOE_ERR_ARG);
  EXPECT(moe_expert_ffn_gathered(F, Fi, Fi, 8, 12, 32, 4, 16, F, F, F, BF, F, F, BIG, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_ffn_gathered(F, Fi, Fi, 8, 16, 32, 4, 16, F, F, F, BF, F, F, 16, 0),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_reroute(Ff, 0, Fi, Ff, Fi, Fi, 0, 4, 2, 3, G0, Fi, Ff, Fi, Fi, Fi, Fi, F, BIG, 0),
         MOE_ERR_ARG);
  EXPECT(moe_reroute(Ff, 0, Fi, Ff, Fi, Fi, 8, 4, 2, 3, G0, Fi, Ff, Fi, Fi, Fi, Fi, 0, BIG, 0),
         MOE_ERR_ARG);
  EXPECT(moe_reroute(Ff, 0, Fi, Ff, Fi, Fi, 8, 2000, 2, 3, G0, Fi, Ff, Fi, Fi, Fi, Fi, F, BIG, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_reroute(Ff, 0, Fi, Ff, Fi, Fi, 8, 4, 2, 3, G0, Fi, Ff, Fi, Fi, Fi, Fi, F, 8, 0),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_quantize_weights(0, 1, 4, 8, BF, 8, F, Ff, 0), MOE_ERR_ARG);
  EXPECT(moe_quantize_weights(F, 1, 4, 8, BF, 5, F, Ff, 0), MOE_ERR_ARG);
  EXPECT(moe_quantize_weights(F, 1, 4, 8, F32, 8, F, Ff, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_quantize_weights(F, 1, 4, 7, BF, 4, F, Ff, 0), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_ffn_q(F, Fi, Fi, 8, 128, 256, 4, 2, 3, F, Ff, F, Ff, F, Ff, BF, F, F, BIG, 0),
         MOE_ERR_ARG);
  EXPECT(moe_expert_ffn_q(F, Fi, Fi, 8, 64, 256, 4, 2, 8, F, Ff, F, Ff, F, Ff, BF, F, F, BIG, 0),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_ffn_q(F, Fi, Fi, 8, 128, 256, 4, 2, 8, F, Ff, F, Ff, F, Ff, BF, F, F, 16, 0),
         MOE_ERR_WORKSPACE);

  // measurement helpers
  EXPECT(moe_peak_mfma(0, 4, 10, Ff, 0), MOE_ERR_ARG);
  EXPECT(moe_peak_mfma(F4, 4, 10, Ff, 0), MOE_ERR_ARG);
  EXPECT(moe_peak_copy(F, F, 40, 0), MOE_ERR_ARG);
  EXPECT(moe_peak_copy(F8, F, 64, 0), MOE_ERR_ARG);

  printf("abi_errors: %d failures (sizing checksum %zu)\n", failures, acc);
  return failures == 0 ? 0 : 1;
}
