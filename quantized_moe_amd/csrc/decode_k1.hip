// First decode launch: router logits and the shared expert's gate/up +
// SwiGLU (everything that depends on x alone).
//
// Blocks [0, n_rb) are router blocks: one expert per wave.  Blocks
// [n_rb, n_rb + n_sb) are shared-expert blocks: each takes spb consecutive
// wave steps of the shared gate/up; its waves issue their weight loads
// first, then quantize x into LDS together (once per token), then compute.
// epb and spb are chosen by the host so that all blocks stream about the same
// number of bytes.
#include "decode_common.hpp"

namespace qmoe {
namespace dec {

// Router logits of expert e for every token, in the fixed fp32 order: lane l
// owns partial l, i.e. elements 4 (l + 64 m) + 0..3 for m = 0, 1, ...; it
// takes them in increasing order with one fmaf each; then the partials fold
// as p[l] += p[l + s] for s = 32, 16, ..., 1.
template <int D>
__device__ __forceinline__ void router_item(const DecodeArgs& a, int e) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  constexpr int CH = D / 256;
  float4 w[CH];
#pragma unroll
  for (int m = 0; m < CH; m++) {
    const uint4 v = ld16_stream(a.w_router + (int64_t)e * D + 4 * (lane + 64 * m));
    w[m] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
  }
  for (int t = 0; t < a.T; t++) {
    float4 xv[CH];
    if (a.x_dtype == X_BF16) {
      const uint16_t* xb = static_cast<const uint16_t*>(a.x) + (int64_t)t * D;
#pragma unroll
      for (int m = 0; m < CH; m++) {
        const uint2 bb = *reinterpret_cast<const uint2*>(xb + 4 * (lane + 64 * m));
        xv[m] = make_float4(__uint_as_float(bb.x << 16), __uint_as_float(bb.x & 0xffff0000u),
                            __uint_as_float(bb.y << 16), __uint_as_float(bb.y & 0xffff0000u));
      }
    } else {
      const float* xf = static_cast<const float*>(a.x) + (int64_t)t * D;
#pragma unroll
      for (int m = 0; m < CH; m++) xv[m] = *reinterpret_cast<const float4*>(xf + 4 * (lane + 64 * m));
    }
    float p = 0.0f;
#pragma unroll
    for (int m = 0; m < CH; m++) {
      p = __builtin_fmaf(xv[m].x, w[m].x, p);
      p = __builtin_fmaf(xv[m].y, w[m].y, p);
      p = __builtin_fmaf(xv[m].z, w[m].z, p);
      p = __builtin_fmaf(xv[m].w, w[m].w, p);
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) p = p + __shfl_down(p, s, 64);
    if (lane == 0) a.z[(int64_t)t * a.E + e] = p;
  }
}

template <int FMT, int D>
struct XAct {
  using type = ActNib<Geo<FMT, D>::CPL, false>;
};
template <int D>
struct XAct<FMT_Q8, D> {
  using type = ActQ8N<Geo<FMT_Q8, D>::CPL>;
};

// A lane's activation slice from x chunks quantized in LDS.
template <int FMT, int D>
__device__ __forceinline__ void load_x_act(typename XAct<FMT, D>::type& act, const uint8_t* q, const float* sc) {
  using G = Geo<FMT, D>;
  const int c = (threadIdx.x & 63) % G::LPR;
  if constexpr (FMT == FMT_Q8) {
    act.template load<G::LPR, 64>(q, sc, c);
  } else {
    act.template load<G::LPR>(q, sc, c);
    if constexpr (FMT == FMT_Q2K) act.sums();
  }
}

template <int FMT_S, int D>
__global__ __launch_bounds__(THREADS) void k1_kernel(DecodeArgs a, K1Plan pl) {
  extern __shared__ uint32_t dyn_tab[];
  __shared__ Iq2Aux aux;
  __shared__ __attribute__((aligned(16))) uint8_t s_xq[(D / 64) * CHUNK_BYTES];
  __shared__ float s_xs[D / 64];
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (b < pl.n_rb) {
    const int e = b * pl.epb + wave;
    if (wave < pl.epb && e < a.E) router_item<D>(a, e);
    return;
  }
  // shared-expert block: waves take steps s_lo + wave, s_lo + wave + 8 (two at a time)
  using G = Geo<FMT_S, D>;
  const int sub = lane / G::LPR, c = lane % G::LPR;
  const int s_lo = (b - pl.n_rb) * pl.spb;
  const int s_hi = min(pl.n_steps, s_lo + pl.spb);
  const EPlanes Gp = expert_planes(a.s_gate, 0), Up = expert_planes(a.s_up, 0);
  uint2 grow = make_uint2(0, 0);
  if constexpr (FMT_S == FMT_IQ2) grow = iq2_grid_row(a.grid, threadIdx.x);
  bool table_ready = false;
  for (int base = s_lo; base < s_hi; base += 2 * WAVES) {
    Piece<FMT_S> wg[2][G::CPL], wu[2][G::CPL];
    int st[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int s = base + wave + WAVES * i;
      st[i] = s;
      const uint32_t n = (uint32_t)((s < s_hi ? s : s_lo) * G::RPS + sub);
#pragma unroll
      for (int k = 0; k < G::CPL; k++) {
        wg[i][k].template load<G::NB>(Gp, n, c + G::LPR * k);
        wu[i][k].template load<G::NB>(Up, n, c + G::LPR * k);
      }
    }
    if constexpr (FMT_S == FMT_IQ2) {
      if (!table_ready) {  // block-uniform
        iq2_aux_prepare(grow, threadIdx.x, &aux);
        __syncthreads();
        iq2_fill_table(dyn_tab, &aux);
        table_ready = true;
      }
    }
    for (int t = 0; t < a.T; t++) {
      __syncthreads();  // the previous token's chunks are no longer read
      quant_x_chunks<(D / 64 + WAVES - 1) / WAVES>(a.x, a.x_dtype, (int64_t)t * D, D / 64, nib_layout(FMT_S), s_xq,
                                                   s_xs, 0);
      __syncthreads();
      typename XAct<FMT_S, D>::type act;
      load_x_act<FMT_S, D>(act, s_xq, s_xs);
#pragma unroll
      for (int i = 0; i < 2; i++) {
        float g = 0.0f, u = 0.0f;
#pragma unroll
        for (int k = 0; k < G::CPL; k++) {
          g += piece_dot(wg[i][k], act, k, dyn_tab);
          u += piece_dot(wu[i][k], act, k, dyn_tab);
        }
        g = group_sum<G::LPR>(g);
        u = group_sum<G::LPR>(u);
        if (c == G::LPR - 1 && st[i] < s_hi) a.hsh[(int64_t)t * a.f + st[i] * G::RPS + sub] = silu(g) * u;
      }
    }
  }
}

template <int FMT_S, int D>
static hipError_t run_k1(const DecodeArgs& a, const K1Plan& pl, hipStream_t s) {
  const size_t lds = FMT_S == FMT_IQ2 ? IQ2_TAB_BYTES : 0;
  static bool attr = false;
  if (!attr && lds) {
    hipError_t e = hipFuncSetAttribute((const void*)k1_kernel<FMT_S, D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  k1_kernel<FMT_S, D><<<dim3(pl.n_rb + pl.n_sb), THREADS, lds, s>>>(a, pl);
  return hipGetLastError();
}

template <int D>
static hipError_t run_k1_f(const DecodeArgs& a, const K1Plan& pl, int fmt_s, hipStream_t s) {
  switch (fmt_s) {
    case FMT_IQ2: return run_k1<FMT_IQ2, D>(a, pl, s);
    case FMT_Q2K: return run_k1<FMT_Q2K, D>(a, pl, s);
    default: return run_k1<FMT_Q8, D>(a, pl, s);
  }
}

hipError_t launch_k1(const DecodeArgs& a, const K1Plan& pl, int fmt_s, hipStream_t s) {
  if (pl.n_rb + pl.n_sb == 0) return hipSuccess;
  switch (a.d) {
    case 256: return run_k1_f<256>(a, pl, fmt_s, s);
    case 512: return run_k1_f<512>(a, pl, fmt_s, s);
    case 1024: return run_k1_f<1024>(a, pl, fmt_s, s);
    case 2048: return run_k1_f<2048>(a, pl, fmt_s, s);
    case 4096: return run_k1_f<4096>(a, pl, fmt_s, s);
    default: return run_k1_f<8192>(a, pl, fmt_s, s);
  }
}

}  // namespace dec
}  // namespace qmoe
