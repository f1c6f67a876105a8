// Second decode launch: exact top-k, routed gate/up + SwiGLU, and the
// quantization of the routed and shared SwiGLU outputs for the down
// projections.
//
// The routed h rows of all tokens (T * k * d_ff, route-major) are cut into
// groups of 16, the unit of h's quantization scale; a block takes GCNT
// consecutive groups of one token (8 waves, 2 GCNT rows each), so every block
// streams the same bytes and finishes whole groups.  Block prologue, in
// parallel: wave 0 selects the token's experts from the router logits (every
// block of the token does the same exact top-k; the token's first block
// publishes idx / wt); waves 1..7 build the IQ2 tables and (wave 7) quantize
// a share of the shared expert's h.  Then every wave requests its rows' scale
// bytes and first weights and the rows run software-pipelined (x comes
// quantized from the first launch).
#include "decode_common.hpp"
#include "topk.hpp"

namespace qmoe {
namespace dec {

template <int FMT, int D>
struct RoutedAct {
  using type = ActNib<Geo<FMT, D>::CPL, false>;
};
template <int D>
struct RoutedAct<FMT_Q8, D> {
  using type = ActQ8N<Geo<FMT_Q8, D>::CPL>;
};

template <int FMT, int D, int GCNT>
__global__ __launch_bounds__(THREADS) void k2_kernel(DecodeArgs a, int down_layout, int shared_layout) {
  __shared__ Iq2Tab itab;
  __shared__ __attribute__((aligned(16))) float hbuf[16 * GCNT];
  __shared__ int s_sel[TOPK_MAX_K];
  __shared__ float s_zs[TOPK_MAX_K];
  using G = Geo<FMT, D>;
  constexpr int RPW = 2 * GCNT;  // h rows per wave
  constexpr int NS = (RPW + G::RPS - 1) / G::RPS;
  constexpr int PD = NS < 3 ? NS : 3;  // steps of loads kept in flight ahead of the compute
  constexpr int SCL_BYTES = RowScales<FMT, D>::STAGE ? 2 * RPW * RowScales<FMT, D>::BYTES : 16;
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[WAVES * SCL_BYTES];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane / G::LPR, c = lane % G::LPR;
  const int g0 = blockIdx.x * GCNT;  // first group of 16 rows
  const int R0 = 16 * g0;            // first routed h row (route-major over all tokens)
  const int t = R0 / (a.k * a.f);

  // ---- prologue: only small loads, all issued before any weight load ----
  if (wave == 0) {
    if (a.fused_topk) {
      wave_topk(a.z + (int64_t)t * a.E, a.E, a.k, s_sel, s_zs);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      const float w = topk_weight_lane(s_zs, a.k);
      if (R0 % (a.k * a.f) == 0 && lane < a.k) {  // the token's first block publishes the routes
        const int64_t o = (int64_t)t * a.k + lane;
        a.idx[o] = s_sel[lane];
        a.wt[o] = w;
        if (a.idx_out) a.idx_out[o] = s_sel[lane];
        if (a.wt_out) a.wt_out[o] = w;
      }
    } else if (lane < a.k) {
      s_sel[lane] = a.idx[(int64_t)t * a.k + lane];
    }
  } else {
    if constexpr (FMT == FMT_IQ2) iq2_build(a.grid, threadIdx.x - 64, &itab);  // waves 1..7: 384 items
    if (a.has_shared && wave == WAVES - 1) {
      // the shared expert's h (from the first launch): 32 groups per pass,
      // the passes spread over the blocks
      const int NG = a.T * a.f / 16;
      const int64_t base = (int64_t)a.T * a.k * (a.f / 16);
      for (int g0s = 32 * blockIdx.x; g0s < NG; g0s += 32 * gridDim.x)
        quant_g32(a.hsh, NG, g0s, shared_layout, a.hq + base * G16_BYTES, a.hs + base);
    }
  }
  __syncthreads();

  // ---- this wave's rows, software-pipelined ----
  // The wave's RPW rows start at route r0 and cross at most one route
  // boundary (at wave row jb), so two plane sets cover them.
  using SS = ScaleStage<FMT, D, 2, RPW>;
  constexpr bool STAGE = SS::RS::STAGE;
  const int Rw = R0 + wave * RPW;   // first row of the wave
  const int r0 = Rw / a.f;          // its route (global index)
  const int n0 = Rw - r0 * a.f;     // its row inside the expert
  const int jb = a.f - n0;          // rows j >= jb belong to route r0 + 1
  const int r1 = min(r0 + 1, t * a.k + a.k - 1);  // (a block never leaves its token)
  const int e0 = s_sel[r0 - t * a.k], e1 = s_sel[r1 - t * a.k];
  const bool ok0 = (unsigned)e0 < (unsigned)a.E, ok1 = (unsigned)e1 < (unsigned)a.E;
  const EPlanes G0 = expert_planes<FMT>(a.gate, ok0 ? e0 : 0), U0 = expert_planes<FMT>(a.up, ok0 ? e0 : 0);
  const EPlanes G1 = expert_planes<FMT>(a.gate, ok1 ? e1 : 0), U1 = expert_planes<FMT>(a.up, ok1 ? e1 : 0);
  auto rowsrc = [&](int m, int j, EPlanes& P, uint32_t& row) {
    const bool second = j >= jb;
    P = m == 0 ? pick_planes(second, G0, G1) : pick_planes(second, U0, U1);
    row = (uint32_t)(second ? n0 + j - a.f : n0 + j);
  };
  Piece<FMT> wg[NS][G::CPL], wu[NS][G::CPL];
  int lr[NS];
  bool ok[NS];
  auto issue = [&](int s) {
    const int jj = s * G::RPS + sub;  // row within the wave
    const bool valid = jj < RPW;
    const int j = valid ? jj : 0;
    lr[s] = wave * RPW + j;
    const bool second = j >= jb;
    ok[s] = valid && (second ? ok1 : ok0);
    const uint32_t n = (uint32_t)(second ? n0 + j - a.f : n0 + j);
    const EPlanes Gp = pick_planes(second, G0, G1);
    const EPlanes Up = pick_planes(second, U0, U1);
#pragma unroll
    for (int k = 0; k < G::CPL; k++) {
      wg[s][k].template load<G::NB>(Gp, n, c + G::LPR * k);
      wu[s][k].template load<G::NB>(Up, n, c + G::LPR * k);
      if constexpr (!STAGE) {
        wg[s][k].template scales_global<G::NB>(Gp, n, c + G::LPR * k);
        wu[s][k].template scales_global<G::NB>(Up, n, c + G::LPR * k);
      }
    }
  };
  uint8_t* my_scales = s_scl + wave * SCL_BYTES;
  SS ss;
  if constexpr (STAGE) ss.issue(rowsrc);  // first: returns before the codes
#pragma unroll
  for (int s = 0; s < PD; s++) issue(s);
  if constexpr (STAGE) ss.store(my_scales);
  typename RoutedAct<FMT, D>::type act;
  {
    const uint8_t* xq = a.xq + (int64_t)t * (D / 64) * CHUNK_BYTES;
    const float* xs = a.xs + (int64_t)t * (D / 64);
    if constexpr (FMT == FMT_Q8) {
      act.template load<G::LPR, 64>(xq, xs, c);
    } else {
      act.template load<G::LPR>(xq, xs, c);
      act.sums();  // Q2K's min term, IQ2's 2u - 7 offset
    }
  }
#pragma unroll
  for (int s = 0; s < NS; s++) {
    if (s + PD < NS) issue(s + PD);
    if constexpr (STAGE) {
      const int j = min(s * G::RPS + sub, RPW - 1);
#pragma unroll
      for (int k = 0; k < G::CPL; k++) {
        wg[s][k].template scales_lds<G::NB>(SS::row(my_scales, 0, j), c + G::LPR * k);
        wu[s][k].template scales_lds<G::NB>(SS::row(my_scales, 1, j), c + G::LPR * k);
      }
    }
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int k = 0; k < G::CPL; k++) {
      g += piece_dot(wg[s][k], act, k, &itab);
      u += piece_dot(wu[s][k], act, k, &itab);
    }
    g = group_sum<G::LPR>(g);
    u = group_sum<G::LPR>(u);
    if (c == G::LPR - 1 && s * G::RPS + sub < RPW) hbuf[lr[s]] = ok[s] ? silu(g) * u : 0.0f;
  }
  __syncthreads();
  if (wave == 0) quant_g32(hbuf, GCNT, 0, down_layout, a.hq + (int64_t)g0 * G16_BYTES, a.hs + g0);
}

template <int FMT, int D, int GCNT>
static hipError_t run_k2(const DecodeArgs& a, int blocks, int down_layout, int shared_layout, hipStream_t s) {
  QMOE_LAUNCH((k2_kernel<FMT, D, GCNT>), dim3(blocks), dim3(THREADS), 0, s, a, down_layout, shared_layout);
  return hipGetLastError();
}

template <int FMT, int D>
static hipError_t run_k2_g(const DecodeArgs& a, int gcnt, int blocks, int dl, int sl, hipStream_t s) {
  switch (gcnt) {
    case 3: return run_k2<FMT, D, 3>(a, blocks, dl, sl, s);
    case 2: return run_k2<FMT, D, 2>(a, blocks, dl, sl, s);
    default: return run_k2<FMT, D, 1>(a, blocks, dl, sl, s);
  }
}

hipError_t launch_k2(const DecodeArgs& a, int fmt, int gcnt, int blocks, int down_layout, int shared_layout,
                     hipStream_t s) {
#define K2_FMT(D)                                                                              \
  switch (fmt) {                                                                               \
    case FMT_IQ2: return run_k2_g<FMT_IQ2, D>(a, gcnt, blocks, down_layout, shared_layout, s); \
    case FMT_Q2K: return run_k2_g<FMT_Q2K, D>(a, gcnt, blocks, down_layout, shared_layout, s); \
    default: return run_k2_g<FMT_Q8, D>(a, gcnt, blocks, down_layout, shared_layout, s);       \
  }
  switch (a.d) {
    case 256: K2_FMT(256)
    case 512: K2_FMT(512)
    case 1024: K2_FMT(1024)
    case 2048: K2_FMT(2048)
    case 4096: K2_FMT(4096)
    default: K2_FMT(8192)
  }
#undef K2_FMT
}

}  // namespace dec
}  // namespace qmoe
