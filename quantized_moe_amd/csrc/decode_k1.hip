// First decode launch: router logits, x quantized for the gate/up rows, and
// (more than one token, VQ formats) the shared expert's gate/up + SwiGLU:
// everything that depends on x alone.  A single token's shared gate/up runs
// in the second launch instead, in the time its blocks wait for the routes;
// several tokens of the block formats run it in the planning launch
// (plan_shared_kernel below), beside the plan's single block.
//
// Blocks [0, n_rb) are router blocks: one expert per wave.  Blocks
// [n_rb, n_rb + n_sb) are shared-expert blocks: each takes spb consecutive
// wave steps of the shared gate/up; its waves issue their weight loads
// first, then quantize every token's x into LDS together (dynamic LDS,
// T x d/64 chunks and scales), then run every token against the weights in
// registers, with no barrier between tokens.
// epb and spb are chosen by the host so that all blocks stream about the same
// number of bytes.
#include "decode_plan.hpp"

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

// Dynamic LDS of the shared blocks for T tokens.
__host__ __device__ constexpr int k1_x_lds_bytes(int T, int D) { return T * (D / 64) * (CHUNK_BYTES + 4); }

// Static LDS of a shared gate/up block: the IQ2 nibble table and the
// waves' staged scale bytes.
template <int FMT_S, int D>
constexpr int k1_scl_bytes() {
  return RowScales<FMT_S, D>::STAGE ? 4 * Geo<FMT_S, D>::RPS * RowScales<FMT_S, D>::BYTES : 16;
}

// Shared gate/up block b of a launch whose plan pl lists pl.n_rb other
// blocks first (router or plan blocks): waves take steps s_lo + wave,
// s_lo + wave + 8 (two per round).  The scale bytes and weights of the first
// round are requested, then every token's x is quantized into LDS ((token,
// octet) items over the waves); one barrier; then every token runs against
// the round's weights.
template <int FMT_S, int D>
__device__ __forceinline__ void k1_shared_block(const DecodeArgs& a, const K1Plan& pl, int b, Iq2Tab& itab,
                                                uint8_t* s_scl, uint8_t* k1_dyn) {
  constexpr int SCL_BYTES = k1_scl_bytes<FMT_S, D>();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  using G = Geo<FMT_S, D>;
  constexpr int NOCT = (D / 64 + 7) / 8;    // octets of chunks of one token
  uint8_t* s_xq = k1_dyn;                                                          // [T][D/64][128]
  float* s_xs = reinterpret_cast<float*>(k1_dyn + (size_t)a.T * (D / 64) * CHUNK_BYTES);  // [T][D/64]
  const int sub = lane / G::LPR, c = lane % G::LPR;
  const int s_lo = (b - pl.n_rb) * pl.spb;
  const int s_hi = min(pl.n_steps, s_lo + pl.spb);
  const EPlanes Gp = expert_planes<FMT_S>(a.s_gate, 0), Up = expert_planes<FMT_S>(a.s_up, 0);
  if constexpr (FMT_S == FMT_IQ2) iq2_build(a.grid, threadIdx.x, &itab);  // published by the barrier below
  using SS = ScaleStage<FMT_S, D, 2, 2 * G::RPS>;  // gate/up x (2 steps x RPS rows)
  constexpr bool STAGE = SS::RS::STAGE;
  uint8_t* my_scales = s_scl + wave * SCL_BYTES;
  Piece<FMT_S> wg[2][G::CPL], wu[2][G::CPL];
  int st[2];
  auto issue = [&](int i, int base) {
    const int s = base + wave + WAVES * i;
    st[i] = s;
    if (s >= s_hi) return;  // (uniform per wave) no step: compute skips it too
    const uint32_t n = (uint32_t)(s * G::RPS + sub);
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
    load_x_act<FMT_S, D>(act, s_xq + (size_t)t * (D / 64) * CHUNK_BYTES, s_xs + (size_t)t * (D / 64));
#pragma unroll
    for (int i = 0; i < 2; i++) {
      if (st[i] >= s_hi) continue;  // (uniform per wave) a step past the block's share: nothing to compute
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
  for (int base = s_lo; base < s_hi; base += 2 * WAVES) {
    SS ss;
    if constexpr (STAGE) ss = stage(base);
    issue(0, base);
    issue(1, base);
    if constexpr (STAGE) ss.store(my_scales);
    if (base == s_lo) {
      if (a.xs_global) {  // quantized by the first launch (the same chunks, the same layout): copied
        const int n16 = a.T * (D / 64) * (CHUNK_BYTES / 16);
        for (int i = threadIdx.x; i < n16; i += THREADS)
          reinterpret_cast<uint4*>(s_xq)[i] = reinterpret_cast<const uint4*>(a.xq_s)[i];
        for (int i = threadIdx.x; i < a.T * (D / 64); i += THREADS) s_xs[i] = a.xs_s[i];
      } else {
        for (int item = wave; item < a.T * NOCT; item += WAVES) {
          const int t = item / NOCT, o = item % NOCT;
          XOctet xo;
          xo.load(static_cast<const uint8_t*>(a.x) + (int64_t)t * D * (a.x_dtype == X_BF16 ? 2 : 4), a.x_dtype,
                  D / 64, 8 * o, nib_layout(FMT_S));
          xo.store(D / 64, s_xq + (size_t)t * (D / 64) * CHUNK_BYTES, s_xs + (size_t)t * (D / 64), nib_layout(FMT_S));
        }
      }
      __syncthreads();
    }
    for (int t = 0; t < a.T; t++) compute(t);
  }
}

template <int FMT_S, int D>
__global__ __launch_bounds__(THREADS) void k1_kernel(DecodeArgs a, K1Plan pl, int gu_layout) {
  __shared__ Iq2Tab itab;
  extern __shared__ __align__(16) uint8_t k1_dyn[];  // shared blocks: x chunks [T][D/64], then scales [T][D/64]
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[WAVES * k1_scl_bytes<FMT_S, D>()];
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int nch_all = a.T * (D / 64);       // x chunks of all tokens, for the routed gate/up
  const int n_oct = (nch_all + 7) / 8;      // ... in octets, one per wave call
  if (b < pl.n_rb || b >= pl.n_rb + pl.n_sb) {  // a router block, or an x block
    int first = -1, stride = 1;
    if (b < pl.n_rb) {
      if (wave < pl.epb) {
        const int e = b * pl.epb + wave;
        if (e < a.E) router_item<D>(a, e);
      } else if (wave == WAVES - 1) {  // the last wave quantizes x
        first = b;
        stride = pl.n_rb;
      }
    } else {  // x blocks: every wave an octet
      first = (b - pl.n_rb - pl.n_sb) * WAVES + wave;
      stride = pl.n_xb * WAVES;
    }
    if (first >= 0) {
      for (int o = first; o < n_oct; o += stride) {
        quant_x8(a.x, a.x_dtype, nch_all, 8 * o, gu_layout, a.xq, a.xs);
        if (a.shared_k2 || a.xs_global) quant_x8(a.x, a.x_dtype, nch_all, 8 * o, nib_layout(FMT_S), a.xq_s, a.xs_s);
      }
    }
    return;
  }
  k1_shared_block<FMT_S, D>(a, pl, b, itab, s_scl, k1_dyn);
}

// Several tokens: block 0 takes the plan (decode_plan.hpp) while blocks
// 1 .. n_sb run the tokens' shared gate/up, whose weights do not depend on
// the routes, and (routes given by the caller, so no router launch before
// this one) the last n_xb blocks quantize x for the routed gate/up, one
// octet of chunks per wave.  The plan alone would leave every other CU idle.
template <int FMT_S, int D>
__global__ __launch_bounds__(THREADS) void plan_shared_kernel(DecodeArgs a, K1Plan pl, int gu_layout) {
  __shared__ Iq2Tab itab;
  extern __shared__ __align__(16) uint8_t k1_dyn[];  // shared blocks: x chunks [T][D/64], then scales [T][D/64]
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[WAVES * k1_scl_bytes<FMT_S, D>()];
  const int b = blockIdx.x;
  if (b == 0) {
    plan_block(a);
    return;
  }
  if (b >= pl.n_rb + pl.n_sb) {
    const int nch_all = a.T * (D / 64), n_oct = (nch_all + 7) / 8;
    for (int o = (b - pl.n_rb - pl.n_sb) * WAVES + (threadIdx.x >> 6); o < n_oct; o += pl.n_xb * WAVES)
      quant_x8(a.x, a.x_dtype, nch_all, 8 * o, gu_layout, a.xq, a.xs);
    return;
  }
  k1_shared_block<FMT_S, D>(a, pl, b, itab, s_scl, k1_dyn);
}

template <int FMT_S, int D>
static hipError_t run_k1(const DecodeArgs& a, const K1Plan& pl, int gu_layout, hipStream_t s) {
  const int dyn = pl.n_sb > 0 ? k1_x_lds_bytes(a.T, D) : 0;
  if (dyn > 0) {  // (raises the kernel's dynamic-LDS limit on first use)
    int per_cu = 0, n_cus = 0;
    if (hipError_t e = launch_shape((const void*)k1_kernel<FMT_S, D>, THREADS, dyn,
                                    k1_x_lds_bytes(DECODE_MAX_T, D), &per_cu, &n_cus);
        e != hipSuccess)
      return e;
  }
  QMOE_LAUNCH((k1_kernel<FMT_S, D>), dim3(pl.n_rb + pl.n_sb + pl.n_xb), dim3(THREADS), dyn, s, a, pl, gu_layout);
  return hipGetLastError();
}

template <int FMT_S, int D>
static hipError_t run_plan_shared(const DecodeArgs& a, const K1Plan& pl, int gu_layout, hipStream_t s) {
  const int dyn = pl.n_sb > 0 ? k1_x_lds_bytes(a.T, D) : 0;
  if (dyn > 0) {  // (raises the kernel's dynamic-LDS limit on first use)
    int per_cu = 0, n_cus = 0;
    if (hipError_t e = launch_shape((const void*)plan_shared_kernel<FMT_S, D>, THREADS, dyn,
                                    k1_x_lds_bytes(DECODE_MAX_T, D), &per_cu, &n_cus);
        e != hipSuccess)
      return e;
  }
  QMOE_LAUNCH((plan_shared_kernel<FMT_S, D>), dim3(pl.n_rb + pl.n_sb + pl.n_xb), dim3(THREADS), dyn, s, a, pl,
              gu_layout);
  return hipGetLastError();
}

template <int D>
static hipError_t run_plan_shared_f(const DecodeArgs& a, const K1Plan& pl, int fmt_s, int gl, hipStream_t s) {
  switch (fmt_s) {
    case FMT_IQ2: return run_plan_shared<FMT_IQ2, D>(a, pl, gl, s);
    case FMT_Q2K: return run_plan_shared<FMT_Q2K, D>(a, pl, gl, s);
    default: return run_plan_shared<FMT_Q8, D>(a, pl, gl, s);
  }
}

hipError_t launch_plan_shared(const DecodeArgs& a, const K1Plan& pl, int fmt_s, int gu_layout, hipStream_t s) {
  switch (a.d) {
    case 256: return run_plan_shared_f<256>(a, pl, fmt_s, gu_layout, s);
    case 512: return run_plan_shared_f<512>(a, pl, fmt_s, gu_layout, s);
    case 1024: return run_plan_shared_f<1024>(a, pl, fmt_s, gu_layout, s);
    case 2048: return run_plan_shared_f<2048>(a, pl, fmt_s, gu_layout, s);
    case 4096: return run_plan_shared_f<4096>(a, pl, fmt_s, gu_layout, s);
    default: return run_plan_shared_f<8192>(a, pl, fmt_s, gu_layout, s);
  }
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
