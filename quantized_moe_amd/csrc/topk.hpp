// Exact top-k of one token's router logits by one wave, and the mixing
// weights of the selected experts.  Shared by the top-k kernel and the decode
// kernels that fuse top-k into their prologue.
//
// Every (logit, expert) pair becomes one 64-bit key: the logit's bits mapped
// to an order-preserving unsigned integer (after folding -0 into +0, so equal
// logits compare equal as IEEE says) in the high word, and the bit-inverted
// expert index in the low word.  The largest key is then the largest logit,
// ties going to the lower index -- the selection rule of the layer.  Each of
// the k rounds takes the wave maximum of the lanes' best remaining keys with
// DPP row shifts and row broadcasts (no LDS round trips) and removes the
// winner.
#pragma once

#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace qmoe {

__device__ __forceinline__ uint32_t logit_order_bits(float z) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float logit_from_order_bits(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  // lanes without a source (or masked off) keep 0, the identity of max here
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, CTRL, ROW_MASK, 0xf, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, CTRL, ROW_MASK, 0xf, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > v ? o : v;
}

// Maximum of a 64-bit value over the 64 lanes of a wave (all lanes active),
// returned to every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0x111, 0xf>(v);  // row_shr:1
  v = dpp_max_step<0x112, 0xf>(v);  // row_shr:2
  v = dpp_max_step<0x114, 0xf>(v);  // row_shr:4
  v = dpp_max_step<0x118, 0xf>(v);  // row_shr:8   -> lane 15 of each row holds the row maximum
  v = dpp_max_step<0x142, 0xa>(v);  // row_bcast:15 -> rows 1, 3 take in rows 0, 2
  v = dpp_max_step<0x143, 0xc>(v);  // row_bcast:31 -> rows 2, 3 take in rows 0..1; lane 63 has all
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Top-k of zt[0..E) by one full wave.  out_idx / out_z (k entries, rank
// order) are written by lane 0 only; they are typically LDS arrays.
__device__ __forceinline__ void wave_topk(const float* __restrict__ zt, int E, int k, int* out_idx, float* out_z) {
  const int lane = threadIdx.x & 63;
  uint64_t key[TOPK_MAX_PER_LANE];
  float zv[TOPK_MAX_PER_LANE];
#pragma unroll
  for (int i = 0; i < TOPK_MAX_PER_LANE; i++) zv[i] = zt[min(lane + 64 * i, E - 1)];  // unconditional: one wait
#pragma unroll
  for (int i = 0; i < TOPK_MAX_PER_LANE; i++) {
    const int e = lane + 64 * i;
    key[i] = e < E ? (((uint64_t)logit_order_bits(zv[i]) << 32) | (uint32_t)~e) : 0ull;
  }
  for (int r = 0; r < k; r++) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < TOPK_MAX_PER_LANE; i++) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < TOPK_MAX_PER_LANE; i++)
      if (key[i] == best) key[i] = 0;
    if (lane == 0) {
      out_idx[r] = (int)~(uint32_t)best;
      out_z[r] = logit_from_order_bits((uint32_t)(best >> 32));
    }
  }
}

// Mixing weights from the selected logits: sigmoid in double precision,
// normalised by the rank-order sum, stored as fp32.
__device__ __forceinline__ void topk_weights(const float* zsel, int k, float* wt) {
  double s[TOPK_MAX_K];
  double sum = 0.0;
#pragma unroll
  for (int j = 0; j < TOPK_MAX_K; j++)
    if (j < k) s[j] = 1.0 / (1.0 + exp(-(double)zsel[j]));
#pragma unroll
  for (int j = 0; j < TOPK_MAX_K; j++)
    if (j < k) sum += s[j];
#pragma unroll
  for (int j = 0; j < TOPK_MAX_K; j++)
    if (j < k) wt[j] = (float)(s[j] / sum);
}

// The same weights computed by a whole wave: lane j < k takes sigmoid(z_j)
// in double precision, every lane sums s_0 .. s_{k-1} in rank order, and lane
// j returns its w_j (lanes >= k return 0).  zsel is read by every lane.
__device__ __forceinline__ float topk_weight_lane(const float* zsel, int k) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
  if (lane < k) s = 1.0 / (1.0 + exp(-(double)zsel[lane]));
  double sum = 0.0;
  for (int j = 0; j < k; j++) sum += __shfl(s, j, 64);
  return lane < k ? (float)(s / sum) : 0.0f;
}

}  // namespace qmoe
