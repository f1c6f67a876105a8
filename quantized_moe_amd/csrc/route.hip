// Router logits and exact top-k.
//
// The router scores every expert of the layer and the best top_k are kept
// per token (DeepSeek V4.1 Flash: 384 experts, 6 chosen -- "YoungAi --
// DeepSeek V4.1 Flash on one DGX Spark", section 2.2).  The pages give no
// summation order; bit-exact expert indices need one, so the fp32 order is
// fixed (include/moe.h): 64 partials, element i in partial (i/4) mod 64,
// consumed in increasing i with one fmaf each, then folded with
// s = 32, 16, ..., 1.  On the GPU partial l lives in lane l of a wave, which
// reads its four elements with one 16-byte load, and the fold is a chain of
// lane shuffles.  Contraction is off in this file: every multiply-add below
// is an explicit fmaf and every fold step a plain addition.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

#pragma clang fp contract(off)

namespace qmoe {

// Load elements 4c .. 4c+3 of an activation row as fp32.
__device__ __forceinline__ float4 load_x4(const void* x, int x_dtype, int64_t row_off, int c) {
  if (x_dtype == X_BF16) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + row_off + 4 * c);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                       __uint_as_float(v.y & 0xffff0000u));
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(x) + row_off + 4 * c);
}

__device__ __forceinline__ float fma4(float4 a, float4 b, float p) {
  p = __builtin_fmaf(a.x, b.x, p);
  p = __builtin_fmaf(a.y, b.y, p);
  p = __builtin_fmaf(a.z, b.z, p);
  p = __builtin_fmaf(a.w, b.w, p);
  return p;
}

// Fold the 64 lane partials: p[l] = p[l] + p[l + s] for s = 32 .. 1.  After
// the loop lane 0 holds the logit (other lanes hold partial garbage).
__device__ __forceinline__ float fold64(float p) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) p = p + __shfl_down(p, s, 64);
  return p;
}

// ---------------------------------------------------------------------------
// Small-T router: a wave per expert keeps its router row in registers and
// walks the tokens.  Block = 4 waves = 4 experts.
// ---------------------------------------------------------------------------
template <int CPL>  // 16-byte chunks per lane = d / 256
__global__ __launch_bounds__(256) void router_rows_kernel(const float* __restrict__ W, int E, int d,
                                                          const void* __restrict__ x, int x_dtype, int T,
                                                          float* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  float4 w[CPL];
#pragma unroll
  for (int m = 0; m < CPL; m++) w[m] = *reinterpret_cast<const float4*>(W + (int64_t)e * d + 4 * (lane + 64 * m));
  for (int t = 0; t < T; t++) {
    float p = 0.0f;
#pragma unroll
    for (int m = 0; m < CPL; m++) p = fma4(load_x4(x, x_dtype, (int64_t)t * d, lane + 64 * m), w[m], p);
    p = fold64(p);
    if (lane == 0) z[(int64_t)t * E + e] = p;
  }
}

// ---------------------------------------------------------------------------
// Large-T router: each wave owns 8 experts x 8 tokens (64 accumulators per
// lane, each the lane's partial of one (token, expert) pair), so every 16-byte
// chunk of W and x loaded feeds 32 fused multiply-adds.  Block = 4 waves
// covering 8 experts x 32 tokens; the 4 waves read the same router rows, which
// the L1 cache serves.
// ---------------------------------------------------------------------------
constexpr int RT_E = 8, RT_T = 8;

// x chunk of one lane as loaded (fp32: 4 floats, bf16: 4 values in 2 words),
// widened to fp32 where it is used, so no load waits on a conversion.
template <int XDT>
struct XRaw {
  uint4 v;
  __device__ __forceinline__ void load(const void* x, int64_t row_off, int c) {
    if constexpr (XDT == X_BF16) {
      const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + row_off + 4 * c);
      v = make_uint4(b.x, b.y, 0u, 0u);
    } else {
      v = *reinterpret_cast<const uint4*>(static_cast<const float*>(x) + row_off + 4 * c);
    }
  }
  __device__ __forceinline__ float4 f32() const {
    if constexpr (XDT == X_BF16)
      return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                         __uint_as_float(v.y & 0xffff0000u));
    else
      return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  }
};

template <int XDT>
__global__ __launch_bounds__(256) void router_tiled_kernel(const float* __restrict__ W, int E, int d,
                                                           const void* __restrict__ x, int T, float* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * RT_E;
  const int t0 = (blockIdx.y * 4 + wave) * RT_T;
  if (t0 >= T) return;
  float acc[RT_T][RT_E];
#pragma unroll
  for (int i = 0; i < RT_T; i++)
#pragma unroll
    for (int j = 0; j < RT_E; j++) acc[i][j] = 0.0f;
  // Chunk m + 1's operands are requested before chunk m's arithmetic (two
  // register sets), so the L2 latency overlaps the fused multiply-adds; the
  // per-lane summation order is unchanged.
  const int chunks = d / 256;
  float4 wv[2][RT_E];
  XRaw<XDT> xr[2][RT_T];
  auto fetch = [&](int set, int m) {
    const int c = lane + 64 * m;
#pragma unroll
    for (int j = 0; j < RT_E; j++) {
      const int e = min(e0 + j, E - 1);
      const float4 v = *reinterpret_cast<const float4*>(W + (int64_t)e * d + 4 * c);
      if (set) wv[1][j] = v;
      else wv[0][j] = v;
    }
#pragma unroll
    for (int i = 0; i < RT_T; i++) {
      const int t = min(t0 + i, T - 1);
      if (set) xr[1][i].load(x, (int64_t)t * d, c);
      else xr[0][i].load(x, (int64_t)t * d, c);
    }
  };
  auto fmas = [&](int set) {
#pragma unroll
    for (int i = 0; i < RT_T; i++) {
      const float4 xv = set ? xr[1][i].f32() : xr[0][i].f32();
#pragma unroll
      for (int j = 0; j < RT_E; j++) acc[i][j] = fma4(xv, set ? wv[1][j] : wv[0][j], acc[i][j]);
    }
  };
  fetch(0, 0);
  if (chunks == 1) {
    fmas(0);
  } else {  // d / 256 is a power of two: an even number of chunks
    for (int m = 0; m < chunks; m += 2) {
      fetch(1, m + 1);
      fmas(0);
      fetch(0, min(m + 2, chunks - 1));  // (after the last pair: a reload that is not used)
      fmas(1);
    }
  }
#pragma unroll
  for (int i = 0; i < RT_T; i++)
#pragma unroll
    for (int j = 0; j < RT_E; j++) {
      const float p = fold64(acc[i][j]);
      const int t = t0 + i, e = e0 + j;
      if (lane == 0 && t < T && e < E) z[(int64_t)t * E + e] = p;
    }
}

hipError_t launch_router(const float* W, int E, int d, const void* x, int x_dtype, int T, float* z, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= ROUTER_ROWS_MAX_T) {
    const dim3 grid((E + 3) / 4);
    switch (d / 256) {
      case 1: QMOE_LAUNCH(router_rows_kernel<1>, grid, dim3(256), 0, s, W, E, d, x, x_dtype, T, z); break;
      case 2: QMOE_LAUNCH(router_rows_kernel<2>, grid, dim3(256), 0, s, W, E, d, x, x_dtype, T, z); break;
      case 4: QMOE_LAUNCH(router_rows_kernel<4>, grid, dim3(256), 0, s, W, E, d, x, x_dtype, T, z); break;
      case 8: QMOE_LAUNCH(router_rows_kernel<8>, grid, dim3(256), 0, s, W, E, d, x, x_dtype, T, z); break;
      case 16: QMOE_LAUNCH(router_rows_kernel<16>, grid, dim3(256), 0, s, W, E, d, x, x_dtype, T, z); break;
      case 32: QMOE_LAUNCH(router_rows_kernel<32>, grid, dim3(256), 0, s, W, E, d, x, x_dtype, T, z); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    const dim3 grid((E + RT_E - 1) / RT_E, (T + 4 * RT_T - 1) / (4 * RT_T));
    if (x_dtype == X_BF16)
      QMOE_LAUNCH(router_tiled_kernel<X_BF16>, grid, dim3(256), 0, s, W, E, d, x, T, z);
    else
      QMOE_LAUNCH(router_tiled_kernel<X_F32>, grid, dim3(256), 0, s, W, E, d, x, T, z);
  }
  return hipGetLastError();
}

// One wave per token.  idx2/wt2 are optional second copies (may be null);
// bias (nullable) selects on the biased sigmoid keys.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ z, int T, int E, int k,
                                                   const float* __restrict__ bias, int32_t* __restrict__ idx,
                                                   float* __restrict__ wt, int32_t* __restrict__ idx2,
                                                   float* __restrict__ wt2) {
  __shared__ int s_sel[4][TOPK_MAX_K];
  __shared__ float s_z[4][TOPK_MAX_K];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  wave_topk(z + (int64_t)t * E, E, k, s_sel[wave], s_z[wave], bias);
  if (lane == 0) {  // lane 0 wrote the lists it reads back
    float w[TOPK_MAX_K];
    topk_weights(s_z[wave], k, w);
#pragma unroll
    for (int j = 0; j < TOPK_MAX_K; j++) {
      if (j >= k) continue;
      idx[(int64_t)t * k + j] = s_sel[wave][j];
      wt[(int64_t)t * k + j] = w[j];
      if (idx2) idx2[(int64_t)t * k + j] = s_sel[wave][j];
      if (wt2) wt2[(int64_t)t * k + j] = w[j];
    }
  }
}

hipError_t launch_topk(const float* z, int T, int E, int k, const float* bias, int32_t* idx, float* wt, int32_t* idx2,
                       float* wt2, hipStream_t s) {
  if (T == 0) return hipSuccess;
  QMOE_LAUNCH(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, z, T, E, k, bias, idx, wt, idx2, wt2);
  return hipGetLastError();
}

}  // namespace qmoe
