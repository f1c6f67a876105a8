// Drives the host side of libqmoe (argument validation, workspace sizing,
// T = 0 no-ops, error strings) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU: every call below is answered by
// host code before any HIP call (built by tests/test_sanitizers.py).  The
// pointers are fake and never dereferenced.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int fails = 0;
#define EXPECT(call, code)                                                                          \
  do {                                                                                              \
    int rc_ = (call);                                                                               \
    if (rc_ != (code)) {                                                                            \
      printf("line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, rc_, (code),          \
             moe_last_error());                                                                     \
      fails++;                                                                                      \
    }                                                                                               \
  } while (0)

static moe_layer layer(int layout) {
  moe_layer L;
  memset(&L, 0, sizeof L);
  L.abi_version = MOE_ABI_VERSION;
  L.n_experts = 384; L.d_model = 4096; L.d_ff = 2048; L.top_k = 6;
  L.fmt_gate_up = MOE_FMT_IQ2XXS_L; L.fmt_down = MOE_FMT_Q2K_L; L.layout = layout;
  L.w_gate = (void*)(uintptr_t)(1ull << 40); L.w_up = (void*)(uintptr_t)(2ull << 40);
  L.w_down = (void*)(uintptr_t)(3ull << 40); L.iq2_grid = (const uint8_t*)(uintptr_t)(4ull << 40);
  L.w_router = (const float*)(uintptr_t)(5ull << 40);
  L.has_shared = 1; L.fmt_shared = MOE_FMT_Q8_0_L;
  L.s_gate = (void*)(uintptr_t)(6ull << 40); L.s_up = (void*)(uintptr_t)(7ull << 40);
  L.s_down = (void*)(uintptr_t)(8ull << 40);
  return L;
}

int main(void) {
  void* p = (void*)(uintptr_t)(9ull << 40);
  moe_layer L = layer(MOE_LAYOUT_DEVICE);
  size_t bytes = 0;
  EXPECT(moe_abi_version(), MOE_ABI_VERSION);
  for (int s = 0; s >= -5; s--) (void)strlen(moe_status_string(s));
  EXPECT(moe_matrix_bytes(MOE_FMT_IQ2XXS_L, 384, 2048, 4096, &bytes), MOE_OK);
  EXPECT(bytes == 384ull * 2162688ull ? 0 : 1, 0);
  EXPECT(moe_matrix_bytes(9, 1, 1, 256, &bytes), MOE_ERR_UNSUPPORTED);
  for (int op = 0; op < 4; op++)
    for (int T = 0; T <= 4096; T = T ? 2 * T : 1) EXPECT(moe_workspace_bytes(&L, T, op, &bytes), MOE_OK);
  EXPECT(moe_workspace_bytes(&L, 1, 7, &bytes), MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_forward(&L, p, MOE_F32, 0, (float*)p, NULL, NULL, 0, p, 0, NULL), MOE_OK);
  EXPECT(moe_layer_forward(&L, p, MOE_F32, 1, (float*)p, NULL, NULL, 0, p, 16, NULL), MOE_ERR_WORKSPACE);
  EXPECT(moe_layer_forward(&L, p, MOE_F32, 65536, (float*)p, NULL, NULL, 0, p, 1 << 20, NULL), MOE_ERR_WORKSPACE);
  moe_layer big = L;
  big.d_ff = 4096;
  EXPECT(moe_layer_forward(&big, p, MOE_F32, 65536, (float*)p, NULL, NULL, 0, p, (size_t)1 << 62, NULL),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_forward_noalloc(&L, p, MOE_F32, 4096, (float*)p, NULL, NULL, 0, NULL), MOE_ERR_WORKSPACE);
  EXPECT(moe_layer_forward_noalloc(&L, p, MOE_F32, 0, (float*)p, NULL, NULL, 0, NULL), MOE_OK);
  EXPECT(moe_expert_ffn_decode(&L, p, MOE_F32, 9, (const int32_t*)p, (const float*)p, (float*)p, p, 1 << 20, NULL),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_expert_ffn_prefill(&L, p, MOE_BF16, 8, (const int32_t*)p, (const float*)p, (float*)p, NULL, p, 0,
                                NULL), MOE_ERR_WORKSPACE);
  moe_layer bad = L;
  bad.abi_version = 1;
  EXPECT(moe_layer_forward(&bad, p, MOE_F32, 1, (float*)p, NULL, NULL, 0, p, 1 << 30, NULL), MOE_ERR_UNSUPPORTED);
  bad = L;
  bad.w_down = (void*)((uintptr_t)L.w_down + 8);
  EXPECT(moe_layer_forward(&bad, p, MOE_F32, 1, (float*)p, NULL, NULL, 0, p, 1 << 30, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk((const float*)p, NULL, 384, 4096, p, MOE_F32, 1, 0, (int32_t*)p, (float*)p, p, 1 << 20,
                        NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_bucket((const int32_t*)p, 0, 6, 384, NULL, NULL, NULL, NULL, NULL), MOE_OK);
  EXPECT(moe_repack(MOE_FMT_Q8_0_L, 1, 16, 32, p, p, MOE_REPACK_TO_DEVICE, NULL), MOE_ERR_INVALID_ARG);
  moe_layer canon = layer(MOE_LAYOUT_CANONICAL), out;
  memset(&out, 0, sizeof out);
  EXPECT(moe_prepare_weights(&canon, &out, NULL), MOE_ERR_INVALID_ARG);
  char names[48 * 4];
  int64_t launches[4];
  double ms[4];
  int32_t n = -1;
  EXPECT(moe_profile_collect(4, names, launches, ms, &n), MOE_OK);
  EXPECT(n, 0);
  if (fails) return 1;
  printf("OK\n");
  return 0;
}
