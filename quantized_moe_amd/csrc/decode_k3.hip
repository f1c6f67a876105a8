// Third decode launch: down projections of the routed experts and of the
// shared expert, and the combine y = sum_j wt_j ye_j + ysh in that fixed
// order (the per-layer MoE sum of "YoungAi -- DeepSeek V4.1 Flash on one DGX
// Spark", section 4.2, with unit gains; ye is taken before the routing
// weight).
//
// Block = 16 output rows of one token.  Tasks: the k routed experts (16 rows
// each) and the shared expert in two halves of 8 rows; a wave runs one task
// at a time with that task's h slice in registers.  Row results meet in LDS.
#include "decode_common.hpp"

namespace qmoe {
namespace dec {

template <int FMT, int K>
struct DownAct {
  using type = ActNib<Geo<FMT, K>::CPL, true>;
};
template <int K>
struct DownAct<FMT_Q8, K> {
  using type = ActQ8N<Geo<FMT_Q8, K>::CPL>;
};

// ROWS rows of expert e's down matrix against one h vector (quantized in
// groups of 16 at hq / hs); row results to out[0 .. ROWS).  The h slice is
// requested before e is needed, so both loads are in flight together; an
// out-of-range expert id (a caller error) contributes zero.
template <int FMT, int K, int ROWS>
__device__ __forceinline__ void down_rows(const QMat& m, int e, int E, int r0, const uint8_t* hq, const float* hs,
                                          const Iq2Tab* tab, uint8_t* my_scales, float* out) {
  using G = Geo<FMT, K>;
  using SS = ScaleStage<FMT, K, 1, ROWS>;
  constexpr bool STAGE = SS::RS::STAGE;
  const int lane = threadIdx.x & 63, sub = lane / G::LPR, c = lane % G::LPR;
  typename DownAct<FMT, K>::type act;
  if constexpr (FMT == FMT_Q8) {
    act.template load<G::LPR, 16>(hq, hs, c);
  } else {
    act.template load<G::LPR>(hq, hs, c);
  }
  if ((unsigned)e >= (unsigned)E) {
    if (lane < ROWS) out[lane] = 0.0f;
    return;
  }
  const EPlanes Dp = expert_planes<FMT>(m, e);
  constexpr int NS = (ROWS + G::RPS - 1) / G::RPS;
  constexpr int PD = NS < 3 ? NS : 3;  // steps of loads kept in flight ahead of the compute
  Piece<FMT> w[NS][G::CPL];
  auto issue = [&](int s) {
    const int j = s * G::RPS + sub;
    const uint32_t n = (uint32_t)(r0 + (j < ROWS ? j : 0));
#pragma unroll
    for (int k = 0; k < G::CPL; k++) {
      w[s][k].template load<G::NB>(Dp, n, c + G::LPR * k);
      if constexpr (!STAGE) w[s][k].template scales_global<G::NB>(Dp, n, c + G::LPR * k);
    }
  };
  SS ss;
  if constexpr (STAGE)
    ss.issue([&](int, int j, EPlanes& P, uint32_t& row) {
      P = Dp;
      row = (uint32_t)(r0 + j);
    });
#pragma unroll
  for (int s = 0; s < PD; s++) issue(s);
  if constexpr (STAGE) ss.store(my_scales);
  if constexpr (FMT != FMT_Q8) act.sums();  // Q2K's min term, IQ2's 2u - 7 offset
#pragma unroll
  for (int s = 0; s < NS; s++) {
    if (s + PD < NS) issue(s + PD);
    const int j = s * G::RPS + sub;
    if constexpr (STAGE) {
#pragma unroll
      for (int k = 0; k < G::CPL; k++)
        w[s][k].template scales_lds<G::NB>(SS::row(my_scales, 0, j < ROWS ? j : 0), c + G::LPR * k);
    }
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < G::CPL; k++) v += piece_dot(w[s][k], act, k, tab);
    v = group_sum<G::LPR>(v);
    if (c == G::LPR - 1 && j < ROWS) out[j] = v;
  }
}

template <int FR, int FS, int F>
__global__ __launch_bounds__(THREADS) void k3_kernel(DecodeArgs a) {
  __shared__ Iq2Tab itab;
  __shared__ float ye[(TOPK_MAX_K + 1) * DN_ROWS];
  constexpr int SCL_R = RowScales<FR, F>::STAGE ? DN_ROWS * RowScales<FR, F>::BYTES : 16;
  constexpr int SCL_S = RowScales<FS, F>::STAGE ? (DN_ROWS / 2) * RowScales<FS, F>::BYTES : 16;
  constexpr int SCL_BYTES = SCL_R > SCL_S ? SCL_R : SCL_S;
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[WAVES * SCL_BYTES];
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.y;
  const int row0 = blockIdx.x * DN_ROWS;
  if constexpr (FR == FMT_IQ2 || FS == FMT_IQ2) {
    iq2_build(a.grid, threadIdx.x, &itab);
    __syncthreads();
  }
  constexpr int NG = F / 16;  // groups of 16 per h vector
  const int n_tasks = a.k + (a.has_shared ? 2 : 0);
  for (int task = wave; task < n_tasks; task += WAVES) {
    if (task < a.k) {
      const int64_t r = (int64_t)t * a.k + task;
      const int e = a.idx[r];
      down_rows<FR, F, DN_ROWS>(a.down, e, a.E, row0, a.hq + r * NG * G16_BYTES, a.hs + r * NG, &itab,
                                s_scl + wave * SCL_BYTES, ye + task * DN_ROWS);
    } else {
      const int half = task - a.k;
      const int64_t src = (int64_t)a.T * a.k + t;
      down_rows<FS, F, DN_ROWS / 2>(a.s_down, 0, 1, row0 + half * (DN_ROWS / 2), a.hq + src * NG * G16_BYTES,
                                    a.hs + src * NG, &itab, s_scl + wave * SCL_BYTES,
                                    ye + a.k * DN_ROWS + half * (DN_ROWS / 2));
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < DN_ROWS) {
    const int n = threadIdx.x;
    float acc = 0.0f;
    for (int q = 0; q < a.k; q++) acc = __builtin_fmaf(a.wt[(int64_t)t * a.k + q], ye[q * DN_ROWS + n], acc);
    if (a.has_shared) acc += ye[a.k * DN_ROWS + n];
    a.y[(int64_t)t * a.d + row0 + n] = acc;
  }
}

template <int FR, int FS, int F>
static hipError_t run_k3(const DecodeArgs& a, hipStream_t s) {
  QMOE_LAUNCH((k3_kernel<FR, FS, F>), dim3(a.d / DN_ROWS, a.T), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

template <int F>
static hipError_t run_k3_f(const DecodeArgs& a, int fr, int fs, hipStream_t s) {
#define K3_FS(FR)                                             \
  switch (fs) {                                               \
    case FMT_IQ2: return run_k3<FR, FMT_IQ2, F>(a, s);        \
    case FMT_Q2K: return run_k3<FR, FMT_Q2K, F>(a, s);        \
    default: return run_k3<FR, FMT_Q8, F>(a, s);              \
  }
  switch (fr) {
    case FMT_IQ2: K3_FS(FMT_IQ2)
    case FMT_Q2K: K3_FS(FMT_Q2K)
    default: K3_FS(FMT_Q8)
  }
#undef K3_FS
}

hipError_t launch_k3(const DecodeArgs& a, int fmt_down, int fmt_shared, hipStream_t s) {
  switch (a.f) {
    case 256: return run_k3_f<256>(a, fmt_down, fmt_shared, s);
    case 512: return run_k3_f<512>(a, fmt_down, fmt_shared, s);
    case 1024: return run_k3_f<1024>(a, fmt_down, fmt_shared, s);
    case 2048: return run_k3_f<2048>(a, fmt_down, fmt_shared, s);
    case 4096: return run_k3_f<4096>(a, fmt_down, fmt_shared, s);
    default: return run_k3_f<8192>(a, fmt_down, fmt_shared, s);
  }
}

}  // namespace dec
}  // namespace qmoe
