// Decode path for several tokens: each chosen expert's down rows are read
// once per call, whatever the number of the call's tokens that chose it, and
// the shared expert's once for all tokens.
//
// "YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 4.4: the batch
// of tokens checked together runs a persistent expert kernel over (unique
// expert x rows) that reads each chosen expert's bits once; section 2.2
// counts 6 / 10 / 13.3 / 17.4 / 21.7 distinct experts for 1 .. 5 consecutive
// tokens, so a small batch reads far fewer expert bytes than its tokens
// times six.  Here, after the first launch (router logits, x quantized;
// none with the caller's routes):
//
//   plan   one block (decode_plan.hpp): the exact top-k of every token (as
//          the one-token path does it), then the list of distinct experts in
//          increasing id and, for each, its routes r = t k + j in increasing
//          r; the same launch's other blocks run every token's shared gate/up
//          and, with the caller's routes, quantize x (decode_k1.hip);
//   gate/up  the one-token kernel, per token, reading the plan's routes (a
//          version over (distinct expert, rows) that loaded each block's
//          codes once for all its routes was slower: 80 against 54 us for 8
//          tokens and 34 experts, its blocks bound by the latency of their
//          prologue and loads);
//   down   a block per 16 output rows: a task per (distinct expert, rows),
//          codes loaded once and run against every route's h; the shared
//          expert's rows once for all tokens; then the same fixed-order
//          combine per token.
//
// Every row result is computed by the same instructions on the same inputs
// as in the one-token path, so the output does not depend on the batch
// (bitwise).
#include "decode_plan.hpp"

namespace qmoe {
namespace dec {

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(DecodeArgs a) { plan_block(a); }

// The last launch over the distinct experts (d_ff <= 2048); FS is the shared
// expert's format.  8 waves: a routed task is 16 rows of one expert, a shared
// task 8 rows.  Where its rows' codes take at most 64 registers a task keeps
// them while it runs its routes, and requests all of them at once (one load
// round per task: a wave runs several tasks one after the other); otherwise
// it requests them again per route (L2-resident after the first), a few
// steps ahead.
constexpr int K3U_WAVES = 8;
template <int FMT, int K, int ROWS>
constexpr bool keep_codes() {
  return DownRows<FMT, K, ROWS, 1>::NS * Geo<FMT, K>::CPL * (int)sizeof(Piece<FMT>) <= 256;
}

template <int FR, int FS, int F>
__global__ __launch_bounds__(64 * K3U_WAVES) void k3u_kernel(DecodeArgs a) {
  constexpr int K3_WAVES = K3U_WAVES;
  constexpr int RT_PARTS = 1;
  constexpr int SH_PARTS = 2;

  constexpr int SH_ROWS = DN_ROWS / SH_PARTS;
  constexpr int RT_ROWS = DN_ROWS / RT_PARTS;
  constexpr int NG = F / 16;
  __shared__ Iq2Tab itab;
  __shared__ float ye[(MAX_ROUTES + DECODE_MAX_T) * DN_ROWS];  // [route][row], then [R + t][row] shared
  constexpr int SCL_R = RowScales<FR, F>::STAGE ? RT_ROWS * RowScales<FR, F>::BYTES : 16;
  constexpr int SCL_S = RowScales<FS, F>::STAGE ? SH_ROWS * RowScales<FS, F>::BYTES : 16;
  constexpr int SCL_BYTES = SCL_R > SCL_S ? SCL_R : SCL_S;
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[K3_WAVES * SCL_BYTES];
  const int wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * DN_ROWS;
  const int R = a.T * a.k;
  const PlanView P = plan_view(a);
  const int U = P.n[0];
  __shared__ int s_next;  // the first task no wave has taken yet
  if (threadIdx.x == 0) s_next = K3_WAVES;
  for (int i = threadIdx.x; i < R * DN_ROWS; i += 64 * K3_WAVES) ye[i] = 0.0f;  // routes with no expert
  if constexpr (FR == FMT_IQ2 || FS == FMT_IQ2) iq2_build(a.grid, threadIdx.x, &itab);
  __syncthreads();
  // The shared tasks (each runs every token) come first, then one task per
  // distinct expert; a wave that finishes a task takes the next one not yet
  // taken (the longest tasks start first, and the waves' chains come out
  // even whatever the experts' route counts).  Each task writes its own ye
  // entries, so the order changes no result.
  const int n_sh = a.has_shared ? SH_PARTS : 0;
  const int n_tasks = n_sh + U * RT_PARTS;
  for (int task = wave; task < n_tasks;) {
    if (task >= n_sh) {
      const int u = (task - n_sh) / RT_PARTS, part = (task - n_sh) % RT_PARTS;
      const int e = P.uexp[u], r0 = P.uoff[u], nr = P.uoff[u + 1] - r0;
      const float* gain = a.down_gain ? a.down_gain + (int64_t)e * a.d : nullptr;
      constexpr int NS = DownRows<FR, F, RT_ROWS, 1>::NS;
      constexpr int CPL = Geo<FR, F>::CPL;
      constexpr int PDMAX = keep_codes<FR, F, RT_ROWS>() ? NS : (FR == FMT_Q4K || FR == FMT_MX4 ? (CPL > 1 ? 1 : 2) : 3);
      using DR = DownRows<FR, F, RT_ROWS, (NS < PDMAX ? NS : PDMAX)>;
      uint8_t* my_scales = s_scl + wave * SCL_BYTES;
      if constexpr (keep_codes<FR, F, RT_ROWS>()) {
        DR dr;
        for (int i = 0; i < nr; i++) {
          const int r = P.uroute[r0 + i];
          dr.load_act(a.hq + (int64_t)r * NG * G16_BYTES, a.hs + (int64_t)r * NG);
          if (i == 0) dr.issue(a.down, e, a.E, row0 + part * RT_ROWS, my_scales, gain);
          dr.run(&itab, my_scales, ye + r * DN_ROWS + part * RT_ROWS, i == 0);
        }
      } else {
        for (int i = 0; i < nr; i++) {
          const int r = P.uroute[r0 + i];
          DR dr;
          dr.load_act(a.hq + (int64_t)r * NG * G16_BYTES, a.hs + (int64_t)r * NG);
          dr.issue(a.down, e, a.E, row0 + part * RT_ROWS, my_scales, gain);
          dr.run(&itab, my_scales, ye + r * DN_ROWS + part * RT_ROWS);
        }
      }
    } else {
      const int part = task;
      constexpr int NS = DownRows<FS, F, SH_ROWS, 1>::NS;
      constexpr int PDMAX = keep_codes<FS, F, SH_ROWS>() ? NS : 3;
      using DR = DownRows<FS, F, SH_ROWS, (NS < PDMAX ? NS : PDMAX)>;
      uint8_t* my_scales = s_scl + wave * SCL_BYTES;
      if constexpr (keep_codes<FS, F, SH_ROWS>()) {
        DR dr;
        for (int t = 0; t < a.T; t++) {
          dr.fetch_act_f32(a.hsh + (int64_t)t * F);
          if (t == 0) dr.issue(a.s_down, 0, 1, row0 + part * SH_ROWS, my_scales, nullptr);
          dr.quant_act_f32();
          dr.run(&itab, my_scales, ye + (R + t) * DN_ROWS + part * SH_ROWS, t == 0);
        }
      } else {
        for (int t = 0; t < a.T; t++) {
          DR dr;
          dr.fetch_act_f32(a.hsh + (int64_t)t * F);
          dr.issue(a.s_down, 0, 1, row0 + part * SH_ROWS, my_scales, nullptr);
          dr.quant_act_f32();
          dr.run(&itab, my_scales, ye + (R + t) * DN_ROWS + part * SH_ROWS);
        }
      }
    }
    int next = 0;
    if ((threadIdx.x & 63) == 0) next = atomicAdd(&s_next, 1);  // LDS
    task = __builtin_amdgcn_readfirstlane(next);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.T * DN_ROWS; i += 64 * K3_WAVES) {
    const int t = i / DN_ROWS, n = i % DN_ROWS;
    float acc = 0.0f;
    for (int q = 0; q < a.k; q++) acc = __builtin_fmaf(a.wt[(int64_t)t * a.k + q], ye[(t * a.k + q) * DN_ROWS + n], acc);
    if (a.has_shared) acc += ye[(R + t) * DN_ROWS + n];
    a.y[(int64_t)t * a.d + row0 + n] = acc;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_plan(const DecodeArgs& a, hipStream_t s) {
  QMOE_LAUNCH(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, s, a);
  return hipGetLastError();
}

template <int FR, int FS, int F>
static hipError_t run_k3u(const DecodeArgs& a, hipStream_t s) {
  QMOE_LAUNCH((k3u_kernel<FR, FS, F>), dim3(a.d / DN_ROWS), dim3(64 * K3U_WAVES), 0, s, a);
  return hipGetLastError();
}

template <int F>
static hipError_t run_k3u_f(const DecodeArgs& a, int fr, int fs, hipStream_t s) {
#define K3U_FS(FR)                                            \
  switch (fs) {                                               \
    case FMT_IQ2: return run_k3u<FR, FMT_IQ2, F>(a, s);       \
    case FMT_Q2K: return run_k3u<FR, FMT_Q2K, F>(a, s);       \
    default: return run_k3u<FR, FMT_Q8, F>(a, s);             \
  }
  switch (fr) {
    case FMT_IQ2: K3U_FS(FMT_IQ2)
    case FMT_Q2K: K3U_FS(FMT_Q2K)
    case FMT_Q4K: K3U_FS(FMT_Q4K)
    case FMT_MX4: K3U_FS(FMT_MX4)
    default: K3U_FS(FMT_Q8)
  }
#undef K3U_FS
}

// d_ff <= 2048 only (k3u_fits); longer rows take the one-token kernel per
// token, which reads the same h.
hipError_t launch_k3u(const DecodeArgs& a, int fmt_down, int fmt_shared, hipStream_t s) {
  switch (a.f) {
    case 256: return run_k3u_f<256>(a, fmt_down, fmt_shared, s);
    case 512: return run_k3u_f<512>(a, fmt_down, fmt_shared, s);
    case 1024: return run_k3u_f<1024>(a, fmt_down, fmt_shared, s);
    case 2048: return run_k3u_f<2048>(a, fmt_down, fmt_shared, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dec
}  // namespace qmoe
