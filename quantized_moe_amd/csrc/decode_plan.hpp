// The planning step of the several-token decode path: every token's exact
// top-k (as the one-token path takes it), then the call's distinct experts
// in increasing id and, for each, its routes r = t k + j in increasing r.
// One block of PLAN_THREADS threads runs it, on its own (plan_kernel) or as
// block 0 of the launch that also runs the tokens' shared gate/up
// (decode_k1.hip).
#pragma once
#include "decode_rows.hpp"
#include "topk.hpp"

namespace qmoe {
namespace dec {

constexpr int PLAN_THREADS = THREADS;  // 512: the shared gate/up blocks' size
constexpr int MAX_ROUTES = DECODE_MAX_T * TOPK_MAX_K;
static_assert(MAX_ROUTES <= PLAN_THREADS && MAX_EXPERTS <= 2 * PLAN_THREADS, "plan block size");

// plan layout in the workspace (int32): [0] = U, [1, 1 + umax) distinct
// experts, [1 + umax, 2 + 2 umax) their first route slot (U + 1 entries),
// [2 + 2 umax, 2 + 2 umax + T k) the routes grouped by expert
struct PlanView {
  int* n;
  int* uexp;
  int* uoff;
  int* uroute;
};
__device__ __forceinline__ PlanView plan_view(const DecodeArgs& a) {
  PlanView p;
  p.n = a.plan;
  p.uexp = a.plan + 1;
  p.uoff = a.plan + 1 + a.umax;
  p.uroute = a.plan + 2 + 2 * a.umax;
  return p;
}

__device__ inline void plan_block(const DecodeArgs& a) {
  constexpr int NW = PLAN_THREADS / 64;
  __shared__ int s_sel[MAX_ROUTES];
  __shared__ float s_zs[MAX_ROUTES];
  __shared__ int s_rank[MAX_EXPERTS];  // 1 for a chosen expert, then its rank among the chosen
  __shared__ int s_wsum[2][NW];
  __shared__ int s_cnt[MAX_ROUTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = a.T * a.k;
  // ---- routes: the top-k of each token, one wave per token ----
  for (int t = wave; t < a.T; t += NW) {
    if (a.fused_topk) {
      if (a.router_bias)
        wave_topk(a.zkey + (int64_t)t * a.E, a.E, a.k, s_sel + t * a.k, s_zs + t * a.k, nullptr,
                  a.z + (int64_t)t * a.E);
      else
        wave_topk(a.z + (int64_t)t * a.E, a.E, a.k, s_sel + t * a.k, s_zs + t * a.k, nullptr);
    } else if (lane < a.k) {
      s_sel[t * a.k + lane] = a.idx[(int64_t)t * a.k + lane];
    }
  }
  for (int e = tid; e < a.E; e += PLAN_THREADS) s_rank[e] = 0;
  for (int i = tid; i < MAX_ROUTES; i += PLAN_THREADS) s_cnt[i] = 0;
  __syncthreads();
  if (a.fused_topk) {  // publish the routes and mixing weights
    for (int t = wave; t < a.T; t += NW) {
      const float w = topk_weight_lane(s_zs + t * a.k, a.k);
      if (lane < a.k) {
        const int64_t o = (int64_t)t * a.k + lane;
        a.idx[o] = s_sel[o];
        a.wt[o] = w;
        if (a.idx_out) a.idx_out[o] = s_sel[o];
        if (a.wt_out) a.wt_out[o] = w;
      }
    }
  }
  // ---- distinct experts (an out-of-range id, a caller error, has none) ----
  if (tid < R) {
    const int e = s_sel[tid];
    if ((unsigned)e < (unsigned)a.E) s_rank[e] = 1;
  }
  __syncthreads();
  // exclusive scan of the flags over the E <= 1024 experts, two per thread:
  // experts tid (the first half, in thread order) and tid + PLAN_THREADS
  const int e1 = tid + PLAN_THREADS;
  const int f0 = tid < a.E ? s_rank[tid] : 0, f1 = e1 < a.E ? s_rank[e1] : 0;
  int i0 = f0, i1 = f1;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int v0 = __shfl_up(i0, s, 64), v1 = __shfl_up(i1, s, 64);
    if (lane >= s) {
      i0 += v0;
      i1 += v1;
    }
  }
  if (lane == 63) {
    s_wsum[0][wave] = i0;
    s_wsum[1][wave] = i1;
  }
  __syncthreads();
  int b0 = 0, b1 = 0, t0 = 0, t1 = 0;
  for (int w = 0; w < NW; w++) {
    t0 += s_wsum[0][w];
    t1 += s_wsum[1][w];
    if (w < wave) {
      b0 += s_wsum[0][w];
      b1 += s_wsum[1][w];
    }
  }
  const int total = t0 + t1;
  const PlanView P = plan_view(a);
  __syncthreads();  // every flag read before the ranks overwrite them
  if (tid < a.E && f0) {
    const int rank = b0 + i0 - 1;
    s_rank[tid] = rank;
    P.uexp[rank] = tid;
  }
  if (e1 < a.E && f1) {
    const int rank = t0 + b1 + i1 - 1;
    s_rank[e1] = rank;
    P.uexp[rank] = e1;
  }
  if (tid == 0) P.n[0] = total;
  __syncthreads();
  // routes per distinct expert, then the routes grouped, in increasing r
  int pos = 0, u = -1;
  if (tid < R) {
    const int e = s_sel[tid];
    if ((unsigned)e < (unsigned)a.E) {
      u = s_rank[e];
      for (int r = 0; r < tid; r++) pos += s_sel[r] == e;
      atomicAdd(&s_cnt[u], 1);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    for (int v = 0; v < total; v++) {
      P.uoff[v] = off;
      off += s_cnt[v];
    }
    P.uoff[total] = off;
    for (int v = 0; v < total; v++) s_cnt[v] = P.uoff[v];  // (re-read below as first slots)
  }
  __syncthreads();
  if (u >= 0) P.uroute[s_cnt[u] + pos] = tid;
}

}  // namespace dec
}  // namespace qmoe
