// Exact top-k of one token's router logits (or of its biased selection keys)
// by one wave, and the mixing weights of the selected experts.  Shared by the top-k kernel and the decode
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

// The selection key of an expert under a router bias b: sigmoid32(z) + b in
// fp32, where sigmoid32 is the fixed sequence of IEEE fp32 operations that
// the interface defines (clamp z to [-80, 80]; t = -z; n = rint(t log2 e)
// by adding and subtracting 1.5 2^23; r = (t - n ln2_hi) - n ln2_lo; the
// degree-6 Taylor polynomial of e^r in Horner form, each step a product and
// then a sum; e = p 2^n with 2^n built from its bits; 1 / (1 + e)), so that
// every implementation performing these operations gets the same bits.
__device__ __forceinline__ float sigmoid32(float z) {
#pragma clang fp contract(off)  // every product and sum rounded on its own
  const float zc = fminf(fmaxf(z, -80.0f), 80.0f);
  const float t = -zc;
  const float kf = t * 0x1.715476p+0f;
  const float n = (kf + 0x1.8p+23f) - 0x1.8p+23f;
  const float r = (t - n * 0x1.62e400p-1f) - n * 0x1.7f7d1cp-20f;
  float p = 0x1.6c16c2p-10f;
  p = p * r + 0x1.111112p-7f;
  p = p * r + 0x1.555556p-5f;
  p = p * r + 0x1.555556p-3f;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  const float e = p * __uint_as_float((uint32_t)((int)n + 127) << 23);
  return 1.0f / (1.0f + e);
}

// The value a top-k ranks expert e on: its logit, or with a router bias its
// biased sigmoid key.
__device__ __forceinline__ float topk_rank_value(float z, const float* bias, int e) {
  return bias ? sigmoid32(z) + bias[e] : z;
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

// Top-k of zt[0..E) by one full wave, E <= 64 * SLOTS.  out_idx / out_z (k
// entries, rank order) are written by lane 0 only; they are typically LDS
// arrays.
template <int SLOTS>
__device__ __forceinline__ void wave_topk_n(const float* __restrict__ zt, int E, int k, int* out_idx, float* out_z,
                                            const float* bias, const float* zsrc) {
  const int lane = threadIdx.x & 63;
  uint64_t key[SLOTS];
  float zv[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; i++) zv[i] = zt[min(lane + 64 * i, E - 1)];  // unconditional: one wait
#pragma unroll
  for (int i = 0; i < SLOTS; i++) {
    const int e = lane + 64 * i;
    const float v = topk_rank_value(zv[i], bias, min(e, E - 1));
    key[i] = e < E ? (((uint64_t)logit_order_bits(v) << 32) | (uint32_t)~e) : 0ull;
  }
  for (int r = 0; r < k; r++) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < SLOTS; i++) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < SLOTS; i++)
      if (key[i] == best) key[i] = 0;
    if (lane == 0) {
      const int e = (int)~(uint32_t)best;
      out_idx[r] = e;
      out_z[r] = zsrc ? zsrc[e] : (bias ? zt[e] : logit_from_order_bits((uint32_t)(best >> 32)));
    }
  }
}

// Wave maximum / minimum of a 32-bit unsigned value, returned to every lane.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
  const int ident = MAX ? 0 : -1;
#define QMOE_DPP_STEP(CTRL, RM)                                                              \
  {                                                                                          \
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(ident, (int)v, CTRL, RM, 0xf, false); \
    v = MAX ? (o > v ? o : v) : (o < v ? o : v);                                             \
  }
  QMOE_DPP_STEP(0x111, 0xf)
  QMOE_DPP_STEP(0x112, 0xf)
  QMOE_DPP_STEP(0x114, 0xf)
  QMOE_DPP_STEP(0x118, 0xf)
  QMOE_DPP_STEP(0x142, 0xa)
  QMOE_DPP_STEP(0x143, 0xc)
#undef QMOE_DPP_STEP
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k with each lane's keys sorted first (a sorting network on (logit key
// descending, expert ascending)), so a round only compares list heads: the
// wave maximum of the heads' logit keys, then the smallest expert among the
// heads that reach it; the winner's lane pops its head.  Same result as
// wave_topk_n: largest logit first, equal logits to the smaller index.
template <int SLOTS>
__device__ __forceinline__ void wave_topk_sorted(const float* __restrict__ zt, int E, int k, int* out_idx,
                                                 float* out_z, const float* bias, const float* zsrc) {
  static_assert(SLOTS == 4 || SLOTS == 8, "network for 4 or 8 keys");
  const int lane = threadIdx.x & 63;
  uint32_t key[SLOTS];
  int ex[SLOTS];
  float zv[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; i++) zv[i] = zt[min(lane + 64 * i, E - 1)];  // unconditional: one wait
#pragma unroll
  for (int i = 0; i < SLOTS; i++) {
    ex[i] = lane + 64 * i;
    key[i] = ex[i] < E ? logit_order_bits(topk_rank_value(zv[i], bias, min(ex[i], E - 1))) : 0u;
  }
  auto cx = [&](int i, int j) {  // put the better of slots i < j first
    const bool swap = key[j] > key[i] || (key[j] == key[i] && ex[j] < ex[i]);
    const uint32_t ki = key[i], kj = key[j];
    const int ei = ex[i], ej = ex[j];
    key[i] = swap ? kj : ki;
    key[j] = swap ? ki : kj;
    ex[i] = swap ? ej : ei;
    ex[j] = swap ? ei : ej;
  };
  if constexpr (SLOTS == 4) {
    cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
  } else {
    cx(0, 1); cx(2, 3); cx(4, 5); cx(6, 7);
    cx(0, 2); cx(1, 3); cx(4, 6); cx(5, 7);
    cx(1, 2); cx(5, 6);
    cx(0, 4); cx(1, 5); cx(2, 6); cx(3, 7);
    cx(2, 4); cx(3, 5);
    cx(1, 2); cx(3, 4); cx(5, 6);
  }
  for (int r = 0; r < k; r++) {
    const uint32_t best = wave_ext_u32<true>(key[0]);
    const uint32_t cand = key[0] == best ? (uint32_t)ex[0] : 0xffffffffu;
    const uint32_t win = wave_ext_u32<false>(cand);
    if (cand == win) {  // this lane's head is taken
#pragma unroll
      for (int i = 0; i < SLOTS - 1; i++) {
        key[i] = key[i + 1];
        ex[i] = ex[i + 1];
      }
      key[SLOTS - 1] = 0u;
    }
    if (lane == 0) {
      out_idx[r] = (int)win;
      out_z[r] = zsrc ? zsrc[win] : (bias ? zt[win] : logit_from_order_bits(best));
    }
  }
}

// Any E <= MAX_EXPERTS.  bias (nullable, [E]): rank on the biased sigmoid
// keys of the logits zt instead of the logits.  zsrc (nullable): zt already
// holds the selection keys and zsrc the logits.  out_z always receives the
// selected logits.
__device__ __forceinline__ void wave_topk(const float* __restrict__ zt, int E, int k, int* out_idx, float* out_z,
                                          const float* bias, const float* zsrc = nullptr) {
  if (E <= 256)
    wave_topk_sorted<4>(zt, E, k, out_idx, out_z, bias, zsrc);
  else if (E <= 512)
    wave_topk_sorted<8>(zt, E, k, out_idx, out_z, bias, zsrc);
  else
    wave_topk_n<TOPK_MAX_PER_LANE>(zt, E, k, out_idx, out_z, bias, zsrc);
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
