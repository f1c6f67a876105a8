// Exact top-k of one token's router logits by one wave, and the mixing
// weights of the selected experts.  Shared by the top-k kernel and the
// decode kernels that fuse top-k into their prologue.
#pragma once

#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace qmoe {

// ---------------------------------------------------------------------------
// Exact top-k of one token's logits, by one wave.  Lane l holds experts
// l, l+64, ...; each round every lane offers its best untaken expert and a
// butterfly keeps the larger logit, equal logits going to the lower index
// (IEEE comparison, so -0 == +0).  All lanes end with the same idx/z lists.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_topk(const float* __restrict__ zt, int E, int k, int* out_idx, float* out_z) {
  const int lane = threadIdx.x & 63;
  float v[TOPK_MAX_PER_LANE];
#pragma unroll
  for (int i = 0; i < TOPK_MAX_PER_LANE; i++) {
    const int e = lane + 64 * i;
    v[i] = e < E ? zt[e] : 0.0f;
  }
  uint32_t taken = 0;
#pragma unroll
  for (int r = 0; r < TOPK_MAX_K; r++) {
    if (r >= k) continue;
    float bv = 0.0f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < TOPK_MAX_PER_LANE; i++) {
      const int e = lane + 64 * i;
      const bool ok = e < E && !((taken >> i) & 1u);
      // experts are visited in increasing index, so a strict '>' keeps the
      // lower index among equal logits
      if (ok && (bi == 0x7fffffff || v[i] > bv)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = shfl_xor(bv, off);
      const int oi = shfl_xor(bi, off);
      const bool other_valid = oi != 0x7fffffff;
      const bool mine_valid = bi != 0x7fffffff;
      if (other_valid && (!mine_valid || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    out_idx[r] = bi;
    out_z[r] = bv;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
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

}  // namespace qmoe
