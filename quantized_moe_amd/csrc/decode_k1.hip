// First decode launch: router logits, x quantized for the gate/up rows, and
// (for more than one token) the shared expert's gate/up + SwiGLU: everything
// that depends on x alone.  A single token's shared gate/up runs in the
// second launch instead, in the time its blocks wait for the routes.
//
// Blocks [0, n_rb) are router blocks: one expert per wave.  Blocks
// [n_rb, n_rb + n_sb) are shared-expert blocks: each takes spb consecutive
// wave steps of the shared gate/up; its waves issue their weight loads
// first, then quantize x into LDS together (once per token), then compute.
// epb and spb are chosen by the host so that all blocks stream about the same
// number of bytes.
#include "decode_rows.hpp"

namespace qmoe {
namespace dec {

// A lane's activation slice from x chunks quantized in LDS.
template <int FMT, int D>
__device__ __forceinline__ void load_x_act(typename RoutedAct<FMT, D>::type& act, const uint8_t* q, const float* sc) {
  using G = Geo<FMT, D>;
  const int c = (threadIdx.x & 63) % G::LPR;
  if constexpr (FMT == FMT_Q8) {
    act.template load<G::LPR, 64>(q, sc, c);
  } else {
    act.template load<G::LPR>(q, sc, c);
    act.sums();  // Q2K's min term, IQ2's 2u - 7 offset
  }
}

template <int FMT_S, int D>
__global__ __launch_bounds__(THREADS) void k1_kernel(DecodeArgs a, K1Plan pl, int gu_layout) {
  __shared__ Iq2Tab itab;
  __shared__ __attribute__((aligned(16))) uint8_t s_xq[(D / 64) * CHUNK_BYTES];
  __shared__ float s_xs[D / 64];
  constexpr int SCL_BYTES =
      RowScales<FMT_S, D>::STAGE ? 4 * Geo<FMT_S, D>::RPS * RowScales<FMT_S, D>::BYTES : 16;
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[WAVES * SCL_BYTES];
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch_all = a.T * (D / 64);       // x chunks of all tokens, for the routed gate/up
  const int n_oct = (nch_all + 7) / 8;      // ... in octets, one per wave call
  if (b < pl.n_rb || b >= pl.n_rb + pl.n_sb) {  // a router block, or the lone x block
    if (wave < pl.epb && b < pl.n_rb) {
      const int e = b * pl.epb + wave;
      if (e < a.E) router_item<D>(a, e);
    } else if (wave == WAVES - 1) {
      const int first = b < pl.n_rb ? b : 0, stride = pl.n_rb > 0 ? pl.n_rb : 1;
      for (int o = first; o < n_oct; o += stride) {
        quant_x8(a.x, a.x_dtype, nch_all, 8 * o, gu_layout, a.xq, a.xs);
        if (a.shared_k2) quant_x8(a.x, a.x_dtype, nch_all, 8 * o, nib_layout(FMT_S), a.xq_s, a.xs_s);
      }
    }
    return;
  }
  // shared-expert block: waves take steps s_lo + wave, s_lo + wave + 8 (two
  // per round).  Loads complete in order, so the x loads go out first, then
  // the scale bytes, then the weights; x is quantized into LDS (one octet of
  // chunks per wave) once it is back.
  using G = Geo<FMT_S, D>;
  constexpr int NOCT = (D / 64 + 7) / 8;    // octets of chunks of one token
  constexpr int OPW = (NOCT + WAVES - 1) / WAVES;
  const int sub = lane / G::LPR, c = lane % G::LPR;
  const int s_lo = (b - pl.n_rb) * pl.spb;
  const int s_hi = min(pl.n_steps, s_lo + pl.spb);
  const EPlanes Gp = expert_planes<FMT_S>(a.s_gate, 0), Up = expert_planes<FMT_S>(a.s_up, 0);
  XOctet xo[OPW];
  auto x_load = [&](int t) {
#pragma unroll
    for (int i = 0; i < OPW; i++)
      xo[i].load(static_cast<const uint8_t*>(a.x) + (int64_t)t * D * (a.x_dtype == X_BF16 ? 2 : 4), a.x_dtype,
                 D / 64, 8 * (wave + WAVES * i), nib_layout(FMT_S));
  };
  auto x_store = [&]() {
#pragma unroll
    for (int i = 0; i < OPW; i++) xo[i].store(D / 64, s_xq, s_xs, nib_layout(FMT_S));
  };
  x_load(0);
  if constexpr (FMT_S == FMT_IQ2) iq2_build(a.grid, threadIdx.x, &itab);  // published by the barrier below
  using SS = ScaleStage<FMT_S, D, 2, 2 * G::RPS>;  // gate/up x (2 steps x RPS rows)
  constexpr bool STAGE = SS::RS::STAGE;
  uint8_t* my_scales = s_scl + wave * SCL_BYTES;
  Piece<FMT_S> wg[2][G::CPL], wu[2][G::CPL];
  int st[2];
  auto issue = [&](int i, int base) {
    const int s = base + wave + WAVES * i;
    st[i] = s;
    const uint32_t n = (uint32_t)((s < s_hi ? s : s_lo) * G::RPS + sub);
#pragma unroll
    for (int k = 0; k < G::CPL; k++) {
      wg[i][k].template load<G::NB>(Gp, n, c + G::LPR * k);
      wu[i][k].template load<G::NB>(Up, n, c + G::LPR * k);
      if constexpr (!STAGE) {
        wg[i][k].template scales_global<G::NB>(Gp, n, c + G::LPR * k);
        wu[i][k].template scales_global<G::NB>(Up, n, c + G::LPR * k);
      }
    }
  };
  auto stage = [&](int base) {  // the scale bytes of this round's rows
    SS ss;
    ss.issue([&](int m, int j, EPlanes& P, uint32_t& row) {
      const int s = base + wave + WAVES * (j / G::RPS);
      P = m == 0 ? Gp : Up;
      row = (uint32_t)((s < s_hi ? s : s_lo) * G::RPS + j % G::RPS);
    });
    return ss;
  };
  auto compute = [&](int t) {
    typename RoutedAct<FMT_S, D>::type act;  // chunk-quantized x, as for the routed rows
    load_x_act<FMT_S, D>(act, s_xq, s_xs);
#pragma unroll
    for (int i = 0; i < 2; i++) {
      if constexpr (STAGE) {
#pragma unroll
        for (int k = 0; k < G::CPL; k++) {
          wg[i][k].template scales_lds<G::NB>(SS::row(my_scales, 0, i * G::RPS + sub), c + G::LPR * k);
          wu[i][k].template scales_lds<G::NB>(SS::row(my_scales, 1, i * G::RPS + sub), c + G::LPR * k);
        }
      }
      float g = 0.0f, u = 0.0f;
#pragma unroll
      for (int k = 0; k < G::CPL; k++) {
        g += piece_dot(wg[i][k], act, k, &itab);
        u += piece_dot(wu[i][k], act, k, &itab);
      }
      g = group_sum<G::LPR>(g);
      u = group_sum<G::LPR>(u);
      if (c == G::LPR - 1 && st[i] < s_hi) a.hsh[(int64_t)t * a.f + st[i] * G::RPS + sub] = silu(g) * u;
    }
  };
  // first round, first token: straight-line, so x is waited for alone
  {
    SS ss;
    if constexpr (STAGE) ss = stage(s_lo);
    issue(0, s_lo);
    issue(1, s_lo);
    if constexpr (STAGE) ss.store(my_scales);
    x_store();
    __syncthreads();
    compute(0);
  }
  // further tokens and rounds (more than one token, or a block with more
  // than 16 steps)
  for (int base = s_lo; base < s_hi; base += 2 * WAVES) {
    if (base != s_lo) {
      SS ss;
      if constexpr (STAGE) ss = stage(base);
      issue(0, base);
      issue(1, base);
      if constexpr (STAGE) ss.store(my_scales);
    }
    for (int t = (base == s_lo ? 1 : 0); t < a.T; t++) {
      __syncthreads();  // the previous token's chunks are no longer read
      x_load(t);
      x_store();
      __syncthreads();
      compute(t);
    }
  }
}

template <int FMT_S, int D>
static hipError_t run_k1(const DecodeArgs& a, const K1Plan& pl, int gu_layout, hipStream_t s) {
  QMOE_LAUNCH((k1_kernel<FMT_S, D>), dim3(pl.n_rb + pl.n_sb + pl.n_xb), dim3(THREADS), 0, s, a, pl, gu_layout);
  return hipGetLastError();
}

template <int D>
static hipError_t run_k1_f(const DecodeArgs& a, const K1Plan& pl, int fmt_s, int gl, hipStream_t s) {
  switch (fmt_s) {
    case FMT_IQ2: return run_k1<FMT_IQ2, D>(a, pl, gl, s);
    case FMT_Q2K: return run_k1<FMT_Q2K, D>(a, pl, gl, s);
    default: return run_k1<FMT_Q8, D>(a, pl, gl, s);
  }
}

hipError_t launch_k1(const DecodeArgs& a, const K1Plan& pl, int fmt_s, int gu_layout, hipStream_t s) {
  switch (a.d) {
    case 256: return run_k1_f<256>(a, pl, fmt_s, gu_layout, s);
    case 512: return run_k1_f<512>(a, pl, fmt_s, gu_layout, s);
    case 1024: return run_k1_f<1024>(a, pl, fmt_s, gu_layout, s);
    case 2048: return run_k1_f<2048>(a, pl, fmt_s, gu_layout, s);
    case 4096: return run_k1_f<4096>(a, pl, fmt_s, gu_layout, s);
    default: return run_k1_f<8192>(a, pl, fmt_s, gu_layout, s);
  }
}

}  // namespace dec
}  // namespace qmoe
