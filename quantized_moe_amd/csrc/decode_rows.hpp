// Row loops of the three decode kernels (decode_k1/k2/k3.hip): router
// logits of one expert, a wave's run of routed gate/up rows, and a wave's
// down-projection rows.
#pragma once

#include "decode_common.hpp"
#include "topk.hpp"
#include "vq.hpp"

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
    if (lane == 0) {
      a.z[(int64_t)t * a.E + e] = p;
      if (a.router_bias) a.zkey[(int64_t)t * a.E + e] = sigmoid32(p) + a.router_bias[e];
    }
  }
}

template <int FMT, int D>
struct RoutedAct {
  using type = ActNib<Geo<FMT, D>::CPL, false>;
};
template <int D>
struct RoutedAct<FMT_Q8, D> {
  using type = ActQ8B<Geo<FMT_Q8, D>::CPL>;
};
template <int D>
struct RoutedAct<FMT_MX4, D> {
  using type = ActMx4<Geo<FMT_MX4, D>::CPL>;
};

// Bytes of LDS scale staging one wave needs for RPW gate/up rows.
template <int FMT, int D, int RPW>
constexpr int gateup_scale_bytes() {
  return RowScales<FMT, D>::STAGE ? 2 * RPW * RowScales<FMT, D>::BYTES : 16;
}

// One wave's RPW consecutive h rows starting at global row Rw (rows are
// route-major: route r = t k + j covers rows r f .. r f + f - 1) of token t:
// gate and up rows (matrices gm, um of E experts with f rows each) of the
// route's expert (s_sel[j], or fixed_e when fixed_e >= 0) against x
// (chunk-quantized at xq / xs, global memory or LDS), SwiGLU, results to
// out[0 .. RPW) (0 for an out-of-range expert id).  The rows cross at most
// one route boundary, so two plane sets cover them.  The scale bytes (staged
// in my_scales) and x are requested first, then PD steps of weight codes; the
// steps run software-pipelined.
template <int FMT, int D, int RPW, int PD>
__device__ __forceinline__ void gateup_rows(const QMat& gm, const QMat& um, int E, int f, int k, int Rw, int t,
                                            const int* s_sel, int fixed_e, const uint8_t* xq, const float* xs,
                                            const Iq2Tab* tab, uint8_t* my_scales, float* out) {
  using G = Geo<FMT, D>;
  constexpr int NS = (RPW + G::RPS - 1) / G::RPS;
  using SS = ScaleStage<FMT, D, 2, RPW>;
  constexpr bool STAGE = SS::RS::STAGE;
  const int lane = threadIdx.x & 63, sub = lane / G::LPR, c = lane % G::LPR;
  const int r0 = Rw / f;          // route of the first row (global index)
  const int n0 = Rw - r0 * f;     // its row inside the expert
  const int jb = f - n0;          // rows j >= jb belong to route r0 + 1
  const int r1 = min(r0 + 1, t * k + k - 1);  // (a wave never leaves its token)
  const int e0 = fixed_e >= 0 ? fixed_e : s_sel[r0 - t * k], e1 = fixed_e >= 0 ? fixed_e : s_sel[r1 - t * k];
  const bool ok0 = (unsigned)e0 < (unsigned)E, ok1 = (unsigned)e1 < (unsigned)E;
  const EPlanes G0 = expert_planes<FMT>(gm, ok0 ? e0 : 0), U0 = expert_planes<FMT>(um, ok0 ? e0 : 0);
  const EPlanes G1 = expert_planes<FMT>(gm, ok1 ? e1 : 0), U1 = expert_planes<FMT>(um, ok1 ? e1 : 0);
  Piece<FMT> wg[NS][G::CPL], wu[NS][G::CPL];
  int lr[NS];
  bool ok[NS];
  auto issue = [&](int s) {
    const int jj = s * G::RPS + sub;  // row within the run
    const bool valid = jj < RPW;
    const int j = valid ? jj : 0;
    lr[s] = j;
    const bool second = j >= jb;
    ok[s] = valid && (second ? ok1 : ok0);
    const uint32_t n = (uint32_t)(second ? n0 + j - f : n0 + j);
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
  SS ss;
  if constexpr (STAGE) {  // first: returns before the codes
    ss.issue([&](int m, int j, EPlanes& P, uint32_t& row) {
      const bool second = j >= jb;
      P = m == 0 ? pick_planes(second, G0, G1) : pick_planes(second, U0, U1);
      row = (uint32_t)(second ? n0 + j - f : n0 + j);
    });
  }
  // x before the codes: loads complete in issue order, so the first step
  // then waits only for its own codes
  typename RoutedAct<FMT, D>::type act;
  if constexpr (FMT == FMT_Q8 || FMT == FMT_MX4) {
    act.template load<G::LPR, 64>(xq, xs, c);
  } else {
    act.template load<G::LPR>(xq, xs, c);
  }
#pragma unroll
  for (int s = 0; s < PD; s++) issue(s);
  if constexpr (STAGE) ss.store(my_scales);
  if constexpr (FMT != FMT_Q8 && FMT != FMT_MX4) act.sums();  // Q2K's min term, IQ2's 2u - 7 offset
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
      g += piece_dot(wg[s][k], act, k, tab);
      u += piece_dot(wu[s][k], act, k, tab);
    }
    g = group_sum<G::LPR>(g);
    u = group_sum<G::LPR>(u);
    if (c == G::LPR - 1 && s * G::RPS + sub < RPW) out[lr[s]] = ok[s] ? silu(g) * u : 0.0f;
  }
}

template <int FMT, int K>
struct DownAct {
  using type = ActNib<Geo<FMT, K>::CPL, true>;
};
template <int K>
struct DownAct<FMT_Q8, K> {
  using type = ActQ8B<Geo<FMT_Q8, K>::CPL>;
};
template <int K>
struct DownAct<FMT_MX4, K> {
  using type = ActMx4<Geo<FMT_MX4, K>::CPL>;
};

// ROWS rows of one expert's down matrix against one h vector (quantized in
// groups of 16), in three steps that the caller may order as it needs:
// load_act() reads the h slice, issue() stages the rows' scale bytes and
// requests the first PD steps of codes, run() computes (requesting the rest)
// and writes the row results to out[0 .. ROWS).  An out-of-range expert id (a
// caller error) contributes zero.
template <int FMT, int K, int ROWS, int PD>
struct DownRows {
  using G = Geo<FMT, K>;
  using SS = ScaleStage<FMT, K, 1, ROWS>;
  static constexpr bool STAGE = SS::RS::STAGE;
  static constexpr int NS = (ROWS + G::RPS - 1) / G::RPS;
  static constexpr int SCALE_BYTES = STAGE ? ROWS * SS::RS::BYTES : 16;
  static_assert(PD >= 1 && PD <= NS, "steps in flight");
  typename DownAct<FMT, K>::type act;
  Piece<FMT> w[NS][G::CPL];
  EPlanes Dp;
  int r0;
  bool valid;
  const float* grow;  // nullable: this expert's per-channel output gains, [d]
  float gv[NS];       // the gains of the rows this lane writes

  __device__ __forceinline__ void load_act(const uint8_t* hq, const float* hs) {
    const int c = (threadIdx.x & 63) % G::LPR;
    if constexpr (FMT == FMT_Q8 || FMT == FMT_MX4) {
      act.template load<G::LPR, 16>(hq, hs, c);
    } else {
      act.template load<G::LPR>(hq, hs, c);
    }
  }
  // the same from the fp32 h vector, quantized here in groups of 16: the
  // values are requested first (fetch_act_f32, ahead of the codes) and
  // quantized once they are back (quant_act_f32)
  float hraw[G::CPL][FMT == FMT_Q8 ? 16 : 64];
  __device__ __forceinline__ void fetch_act_f32(const float* h) {
    const int c = (threadIdx.x & 63) % G::LPR;
    act.template fetch_f32<G::LPR>(h, c, hraw);
  }
  __device__ __forceinline__ void quant_act_f32() {
    if constexpr (FMT == FMT_Q8)
      act.quant_f32(hraw);
    else
      act.quant_f32(hraw, nib_layout(FMT));
  }
  __device__ __forceinline__ void issue_step(int s) {
    const int lane = threadIdx.x & 63, sub = lane / G::LPR, c = lane % G::LPR;
    const int j = s * G::RPS + sub;
    const uint32_t n = (uint32_t)(r0 + (j < ROWS ? j : 0));
#pragma unroll
    for (int k = 0; k < G::CPL; k++) {
      w[s][k].template load<G::NB>(Dp, n, c + G::LPR * k);
      if constexpr (!STAGE) w[s][k].template scales_global<G::NB>(Dp, n, c + G::LPR * k);
    }
  }
  __device__ __forceinline__ void issue(const QMat& m, int e, int E, int row0, uint8_t* my_scales,
                                        const float* gain = nullptr) {
    valid = (unsigned)e < (unsigned)E;
    if (!valid) return;
    Dp = expert_planes<FMT>(m, e);
    r0 = row0;
    grow = gain;
    if (gain) {  // requested first: the oldest loads are back first
      const int lane = threadIdx.x & 63, sub = lane / G::LPR;
#pragma unroll
      for (int s = 0; s < NS; s++) {
        const int j = s * G::RPS + sub;
        gv[s] = gain[r0 + (j < ROWS ? j : 0)];
      }
    }
    SS ss;
    if constexpr (STAGE)
      ss.issue([&](int, int j, EPlanes& P, uint32_t& row) {
        P = Dp;
        row = (uint32_t)(r0 + j);
      });
#pragma unroll
    for (int s = 0; s < PD; s++) issue_step(s);
    if constexpr (STAGE) ss.store(my_scales);
  }
  // issue_more = false: every step's codes are already in registers (a
  // later h vector against the same rows, after a first run)
  __device__ __forceinline__ void run(const Iq2Tab* tab, const uint8_t* my_scales, float* out,
                                      bool issue_more = true) {
    const int lane = threadIdx.x & 63, sub = lane / G::LPR, c = lane % G::LPR;
    if (!valid) {
      if (lane < ROWS) out[lane] = 0.0f;
      return;
    }
    if constexpr (FMT != FMT_Q8 && FMT != FMT_MX4) act.sums();  // Q2K's min term, IQ2's 2u - 7 offset
#pragma unroll
    for (int s = 0; s < NS; s++) {
      if (issue_more && s + PD < NS) issue_step(s + PD);
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
      if (grow) v *= gv[s];
      if (c == G::LPR - 1 && j < ROWS) out[j] = v;
    }
  }
};

// ---------------------------------------------------------------------------
// VQ rows (MOE_FMT_VQ12_L / VQ13_L)
// ---------------------------------------------------------------------------
// The activations stay fp32 (x as given, h as the gate/up rows wrote it) and
// each codeword is converted to fp32 from the LDS codebook: 8 fused
// multiply-adds per index, no fixed point.  A row of K inputs is K / 64
// pieces; lane (sub, c) with sub = lane / LPR, c = lane % LPR takes pieces
// c + LPR * k (k < CPL) of row sub of each step.
template <int K>
struct VqGeo {
  static constexpr int PR = K / 64;
  static constexpr int LPR = PR < 64 ? PR : 64;
  static constexpr int CPL = PR / LPR;
  static constexpr int RPS = 64 / LPR;
};

// A lane's activation slice: CPL pieces of 64 fp32 values.
template <int K>
struct VqAct {
  using G = VqGeo<K>;
  float v[G::CPL][64];
  // from an fp32 (x_dtype X_F32) or bf16 vector of K values
  __device__ __forceinline__ void load(const void* src, int x_dtype, int c) {
#pragma unroll
    for (int k = 0; k < G::CPL; k++) {
      const int i0 = 64 * (c + G::LPR * k);
      if (x_dtype == X_BF16) {
        const uint16_t* p = static_cast<const uint16_t*>(src) + i0;
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const uint4 b = ld16(p + 8 * u);
          const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
          for (int i = 0; i < 4; i++) {
            v[k][8 * u + 2 * i] = __uint_as_float(bw[i] << 16);
            v[k][8 * u + 2 * i + 1] = __uint_as_float(bw[i] & 0xffff0000u);
          }
        }
      } else {
        const float* p = static_cast<const float*>(src) + i0;
#pragma unroll
        for (int u = 0; u < 16; u++) {
          const float4 f = *reinterpret_cast<const float4*>(p + 4 * u);
          v[k][4 * u] = f.x;
          v[k][4 * u + 1] = f.y;
          v[k][4 * u + 2] = f.z;
          v[k][4 * u + 3] = f.w;
        }
      }
    }
  }
};

// sum over the piece's 64 inputs of codeword value * activation, in a fixed
// order (two chains: even and odd indices, added at the end)
template <bool B13>
__device__ __forceinline__ float vq_dot(const VqPiece& p, const float* x, const uint8_t* cb) {
  float acc[2] = {0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < 8; q++) {
    float w[8];
    vq_to_f32(vq_codeword(cb, vq_index<B13>(p, q)), w);
#pragma unroll
    for (int i = 0; i < 8; i++) acc[q & 1] = __builtin_fmaf(w[i], x[8 * q + i], acc[q & 1]);
  }
  return acc[0] + acc[1];
}

__device__ __forceinline__ float vq_gain(const QMat& m, int64_t row) {
  return half_bits_to_float(reinterpret_cast<const uint16_t*>(m.p_scale)[row]);
}

// One wave's RPW consecutive h rows starting at global row Rw (route-major,
// as gateup_rows) of token t against the fp32 slice act of x:
// h = silu(g_G (C x)) * (g_U (C x)) per row, to out[0 .. RPW) (0 for an
// out-of-range expert id).  PD steps of codes are kept in flight.
template <int FMT, int D, int RPW, int PD>
__device__ __forceinline__ void vq_gateup_rows(const QMat& gm, const QMat& um, int E, int f, int k, int Rw, int t,
                                               const int* s_sel, const VqAct<D>& act, const uint8_t* cb,
                                               float* out) {
  using G = VqGeo<D>;
  constexpr bool B13 = FMT == FMT_VQ13;
  constexpr int NS = (RPW + G::RPS - 1) / G::RPS;
  const int lane = threadIdx.x & 63, sub = lane / G::LPR, c = lane % G::LPR;
  const int r0 = Rw / f;
  const int n0 = Rw - r0 * f;
  const int jb = f - n0;
  const int r1 = min(r0 + 1, t * k + k - 1);
  const int e0 = s_sel[r0 - t * k], e1 = s_sel[r1 - t * k];
  const bool ok0 = (unsigned)e0 < (unsigned)E, ok1 = (unsigned)e1 < (unsigned)E;
  VqPiece pg[NS][G::CPL], pu[NS][G::CPL];
  float gg[NS], gu[NS];
  bool ok[NS];
  int lr[NS];
  auto issue = [&](int s) {
    const int jj = s * G::RPS + sub;
    const bool valid = jj < RPW;
    const int j = valid ? jj : 0;
    lr[s] = j;
    const bool second = j >= jb;
    ok[s] = valid && (second ? ok1 : ok0);
    const int e = second ? (ok1 ? e1 : 0) : (ok0 ? e0 : 0);
    const int64_t row = (int64_t)e * f + (second ? n0 + j - f : n0 + j);
    gg[s] = vq_gain(gm, row);
    gu[s] = vq_gain(um, row);
#pragma unroll
    for (int kk = 0; kk < G::CPL; kk++) {
      pg[s][kk] = vq_load_piece<B13>(gm.p_a, gm.p_b, row, D, c + G::LPR * kk);
      pu[s][kk] = vq_load_piece<B13>(um.p_a, um.p_b, row, D, c + G::LPR * kk);
    }
  };
#pragma unroll
  for (int s = 0; s < PD && s < NS; s++) issue(s);
#pragma unroll
  for (int s = 0; s < NS; s++) {
    if (s + PD < NS) issue(s + PD);
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int kk = 0; kk < G::CPL; kk++) {
      g += vq_dot<B13>(pg[s][kk], act.v[kk], cb);
      u += vq_dot<B13>(pu[s][kk], act.v[kk], cb);
    }
    g = group_sum<G::LPR>(g);
    u = group_sum<G::LPR>(u);
    if (c == G::LPR - 1 && s * G::RPS + sub < RPW) out[lr[s]] = ok[s] ? silu(g * gg[s]) * (u * gu[s]) : 0.0f;
  }
}

// ROWS rows r0 .. r0 + ROWS - 1 of expert e's VQ down matrix against the
// fp32 h vector hf (K values): out[j] = gain_row * (C h) (times the
// expert's per-channel output gain when given; 0 for an out-of-range e).
template <int FMT, int K, int ROWS>
__device__ __forceinline__ void vq_down_rows(const QMat& m, int e, int E, int r0, const float* hf,
                                             const float* gain, const uint8_t* cb, float* out) {
  using G = VqGeo<K>;
  constexpr bool B13 = FMT == FMT_VQ13;
  constexpr int NS = (ROWS + G::RPS - 1) / G::RPS;
  constexpr int PD = G::CPL > 1 ? 2 : 4;  // steps of codes in flight
  const int lane = threadIdx.x & 63, sub = lane / G::LPR, c = lane % G::LPR;
  if ((unsigned)e >= (unsigned)E) {
    if (lane < ROWS) out[lane] = 0.0f;
    return;
  }
  VqPiece p[NS][G::CPL];
  float gr[NS], gc[NS];
  auto issue = [&](int s) {
    const int j = min(s * G::RPS + sub, ROWS - 1);
    const int64_t row = (int64_t)e * m.rows + r0 + j;
    gr[s] = vq_gain(m, row);
    gc[s] = gain ? gain[r0 + j] : 1.0f;
#pragma unroll
    for (int kk = 0; kk < G::CPL; kk++) p[s][kk] = vq_load_piece<B13>(m.p_a, m.p_b, row, K, c + G::LPR * kk);
  };
  VqAct<K> act;
  act.load(hf, X_F32, c);  // requested before the codes
#pragma unroll
  for (int s = 0; s < PD && s < NS; s++) issue(s);
#pragma unroll
  for (int s = 0; s < NS; s++) {
    if (s + PD < NS) issue(s + PD);
    float v = 0.0f;
#pragma unroll
    for (int kk = 0; kk < G::CPL; kk++) v += vq_dot<B13>(p[s][kk], act.v[kk], cb);
    v = group_sum<G::LPR>(v);
    const int j = s * G::RPS + sub;
    if (c == G::LPR - 1 && j < ROWS) out[j] = (v * gr[s]) * gc[s];
  }
}

}  // namespace dec
}  // namespace qmoe
