// Second decode launch: exact top-k, routed gate/up + SwiGLU, and the
// quantization of the routed and shared SwiGLU outputs for the down
// projections.
//
// The routed h rows of all tokens (T * k * d_ff, route-major) are cut into
// groups of 16, the unit of h's quantization scale; a block takes GCNT
// consecutive groups of one token (8 waves, 2 GCNT rows each), so every block
// streams the same bytes and finishes whole groups.  Block prologue, all in
// parallel: wave 0 selects the token's experts from the router logits (every
// block of the token does the same exact top-k; the token's first block
// publishes idx / wt); waves 1..7 quantize x_t into LDS, load the IQ2 grid
// and (wave 7) quantize a share of the shared expert's h.  Then every wave
// issues its weight loads and the IQ2 table is written while they fly.
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
  extern __shared__ uint32_t dyn_tab[];
  __shared__ Iq2Aux aux;
  __shared__ __attribute__((aligned(16))) uint8_t s_xq[(D / 64) * CHUNK_BYTES];
  __shared__ float s_xs[D / 64];
  __shared__ float hbuf[16 * GCNT];
  __shared__ int s_sel[TOPK_MAX_K];
  __shared__ float s_zs[TOPK_MAX_K];
  using G = Geo<FMT, D>;
  constexpr int RPW = 2 * GCNT;  // h rows per wave
  constexpr int STEPS = (RPW + G::RPS - 1) / G::RPS;
  constexpr int BATCH_ = (FMT == FMT_Q8 ? 8 : 16) / (2 * G::CPL);
  constexpr int BATCH = BATCH_ < 1 ? 1 : (BATCH_ < STEPS ? BATCH_ : STEPS);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane / G::LPR, c = lane % G::LPR;
  const int g0 = blockIdx.x * GCNT;  // first group of 16 rows
  const int R0 = 16 * g0;            // first routed h row (route-major over all tokens)
  const int t = R0 / (a.k * a.f);

  // ---- prologue ----
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
    const int aux_item = threadIdx.x - 64;  // waves 1..7 prepare the 384 table items
    uint2 grow = make_uint2(0, 0);
    if constexpr (FMT == FMT_IQ2) grow = iq2_grid_row(a.grid, aux_item);
    float hv = 0.0f;
    const int NQ = a.T * a.f / 64;  // quads of shared h groups, spread over the blocks
    const bool do_sh = a.has_shared && wave == WAVES - 1 && (int)blockIdx.x < NQ;
    if (do_sh) hv = a.hsh[(int64_t)blockIdx.x * 64 + lane];
    quant_x_chunks<(D / 64 + WAVES - 2) / (WAVES - 1)>(a.x, a.x_dtype, (int64_t)t * D, D / 64, nib_layout(FMT), s_xq,
                                                     s_xs, 1);
    if constexpr (FMT == FMT_IQ2) iq2_aux_prepare(grow, aux_item, &aux);
    if (do_sh) {
      const int64_t base = (int64_t)a.T * a.k * (a.f / 16) + 4 * blockIdx.x;
      quant_wave<16>(hv, shared_layout, a.hq + base * G16_BYTES, a.hs + base, 4);
      for (int qd = blockIdx.x + gridDim.x; qd < NQ; qd += gridDim.x) {  // (only when blocks < quads)
        const float v = a.hsh[(int64_t)qd * 64 + lane];
        const int64_t b2 = (int64_t)a.T * a.k * (a.f / 16) + 4 * qd;
        quant_wave<16>(v, shared_layout, a.hq + b2 * G16_BYTES, a.hs + b2, 4);
      }
    }
  }
  __syncthreads();

  // ---- weights of this wave's rows ----
#pragma unroll
  for (int s0 = 0; s0 < STEPS; s0 += BATCH) {
    Piece<FMT> wg[BATCH][G::CPL], wu[BATCH][G::CPL];
    int lr[BATCH];
    bool ok[BATCH];
#pragma unroll
    for (int bb = 0; bb < BATCH; bb++) {
      const int j = (s0 + bb) * G::RPS + sub;  // row within the wave
      const bool valid = s0 + bb < STEPS && j < RPW;
      lr[bb] = wave * RPW + (valid ? j : 0);
      const int R = R0 + lr[bb];
      const int e = s_sel[R / a.f - t * a.k];
      const bool e_ok = (unsigned)e < (unsigned)a.E;
      ok[bb] = valid && e_ok;
      const uint32_t n = (uint32_t)(R % a.f);
      const EPlanes Gp = expert_planes(a.gate, e_ok ? e : 0), Up = expert_planes(a.up, e_ok ? e : 0);
#pragma unroll
      for (int k = 0; k < G::CPL; k++) {
        wg[bb][k].template load<G::NB>(Gp, n, c + G::LPR * k);
        wu[bb][k].template load<G::NB>(Up, n, c + G::LPR * k);
      }
    }
    if constexpr (FMT == FMT_IQ2) {
      if (s0 == 0) {  // the table is written while the first weights are in flight
        iq2_fill_table(dyn_tab, &aux);
        __syncthreads();
      }
    }
    typename RoutedAct<FMT, D>::type act;
    if constexpr (FMT == FMT_Q8) {
      act.template load<G::LPR, 64>(s_xq, s_xs, c);
    } else {
      act.template load<G::LPR>(s_xq, s_xs, c);
      if constexpr (FMT == FMT_Q2K) act.sums();
    }
#pragma unroll
    for (int bb = 0; bb < BATCH; bb++) {
      float g = 0.0f, u = 0.0f;
#pragma unroll
      for (int k = 0; k < G::CPL; k++) {
        g += piece_dot(wg[bb][k], act, k, dyn_tab);
        u += piece_dot(wu[bb][k], act, k, dyn_tab);
      }
      g = group_sum<G::LPR>(g);
      u = group_sum<G::LPR>(u);
      const int j = (s0 + bb) * G::RPS + sub;
      if (c == G::LPR - 1 && s0 + bb < STEPS && j < RPW) hbuf[lr[bb]] = ok[bb] ? silu(g) * u : 0.0f;
    }
  }
  __syncthreads();
  if (wave == 0)
    quant_wave<16>(lane < 16 * GCNT ? hbuf[lane] : 0.0f, down_layout, a.hq + (int64_t)g0 * G16_BYTES, a.hs + g0,
                   GCNT);
}

template <int FMT, int D, int GCNT>
static hipError_t run_k2(const DecodeArgs& a, int blocks, int down_layout, int shared_layout, hipStream_t s) {
  const size_t lds = FMT == FMT_IQ2 ? IQ2_TAB_BYTES : 0;
  static bool attr = false;
  if (!attr && lds) {
    hipError_t e = hipFuncSetAttribute((const void*)k2_kernel<FMT, D, GCNT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  k2_kernel<FMT, D, GCNT><<<dim3(blocks), THREADS, lds, s>>>(a, down_layout, shared_layout);
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
