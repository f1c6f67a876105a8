// Decode path: streaming GEMVs over the selected experts' packed weights.
//
// Decode reads every selected weight once per token and is bound by HBM
// bytes ("YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 4.4:
// decoding is memory-bound; the engine's expert kernel streams whole cache
// lines and decodes codes in registers).  Here every lane owns 64
// consecutive inputs of a row (one 16-byte chunk of 2-bit codes, or 64 bytes
// of int8 codes); LPR = K/64 lanes share a row and reduce with a fixed
// butterfly.  Every wave issues the loads of all its rows before decoding any
// of them, so a wave waits for memory once, not once per row.
//
// Integer inner products.  Weights are exact small integers times fp16 block
// scales (IQ2: (2s+1) * grid * sign; Q2K: sc * q - m; Q8: q).  Activations
// (x and the SwiGLU output h) are carried as 16-bit fixed point with one fp32
// scale per 64-element chunk, split into two int8 planes (v ~ s * (256 H + L),
// |error| <= s/2 = max|v|/65024), so each 4 weights x 4 activations is one
// v_dot4_i32_i8 per plane, accumulated exactly in int32 and converted to fp32
// once per chunk.  The relative error this adds to a dot product is ~1e-5,
// far inside the layer's 1e-3 tolerance, and the VALU cost per weight is a
// third of an fp32 dequantise-and-FMA.
//
// Three launches per layer:
//   K1  router logits, quantized x for K2, and the shared expert's
//       gate/up+SwiGLU (all depend only on x);
//   K2  routed gate/up + SwiGLU; with routing fused, each block first runs
//       the exact top-k of its token from the logits K1 wrote;
//   K3  down projections of the routed experts and the shared expert, and
//       the fixed-order combine y = sum_j wt_j ye_j + ysh (the per-layer sum
//       of the YoungAi page, section 4.2).
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace qmoe {

constexpr int DEC_WAVES = 8;                 // waves per block (all three kernels)
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int GU_ROWS_PER_WAVE = 8;          // gate/up rows per wave
constexpr int GU_ROWS_PER_BLOCK = DEC_WAVES * GU_ROWS_PER_WAVE;  // = 64 = one quantization chunk of h
constexpr int DN_ROWS_PER_BLOCK = 16;        // down rows per block
constexpr int CHUNK_BYTES = 128;             // quantized 64-element chunk: 64 B hi plane + 64 B lo plane

// Activation byte orders inside a quantized chunk.  NAT: element e at byte e
// (IQ2 and Q8 consumers).  T16: within each 16-element sub-block, element
// 4j + k at byte 4k + j, so that the k-th 2-bit field of each Q2K quant byte
// (extracted as one 0x03030303-masked word) meets its activations in one dot4.
enum : int { ACT_NAT = 0, ACT_T16 = 1 };

__host__ __device__ constexpr int act_layout(int fmt) { return fmt == FMT_Q2K ? ACT_T16 : ACT_NAT; }

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// ---------------------------------------------------------------------------
// cross-lane sums and maxima with DPP (register-speed, fixed order)
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
  // lanes without a source (or masked off) read 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Sum of v over each aligned group of LPR lanes; the group's total lands in
// its last lane (c == LPR - 1).  Windows double each step (row_shr 1, 2, 4,
// 8 inside 16-lane rows, then row broadcasts), so the order is fixed.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR >= 2) v += dpp_f<0x111, 0xf>(v);
  if constexpr (LPR >= 4) v += dpp_f<0x112, 0xf>(v);
  if constexpr (LPR >= 8) v += dpp_f<0x114, 0xf>(v);
  if constexpr (LPR >= 16) v += dpp_f<0x118, 0xf>(v);
  if constexpr (LPR >= 32) v += dpp_f<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  if constexpr (LPR >= 64) v += dpp_f<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Maximum of v over the wave, returned to every lane (v >= 0).
__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = fmaxf(v, dpp_f<0x111, 0xf>(v));
  v = fmaxf(v, dpp_f<0x112, 0xf>(v));
  v = fmaxf(v, dpp_f<0x114, 0xf>(v));
  v = fmaxf(v, dpp_f<0x118, 0xf>(v));
  v = fmaxf(v, dpp_f<0x142, 0xa>(v));
  v = fmaxf(v, dpp_f<0x143, 0xc>(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ---------------------------------------------------------------------------
// activation quantization (one 64-element chunk per wave, one element per lane)
// ---------------------------------------------------------------------------
__device__ __forceinline__ void quant_chunk_wave(float v, int layout, uint8_t* __restrict__ out,
                                                 float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const float m = wave_max_nonneg(fabsf(v));
  const float inv = m > 0.0f ? 32512.0f / m : 0.0f;
  const int X = (int)rintf(v * inv);  // |X| <= 32512
  const int H = (X + 128) >> 8;       // floor((X + 128) / 256): H in [-127, 127]
  const int Lo = X - (H << 8);        // in [-128, 127]
  const int pos = layout == ACT_NAT ? lane : ((lane & ~15) | ((lane & 3) << 2) | ((lane >> 2) & 3));
  out[pos] = (uint8_t)(int8_t)H;
  out[64 + pos] = (uint8_t)(int8_t)Lo;
  if (lane == 0) *scale = m / 32512.0f;
}

// The same quantization done by one lane over its own 64 values (used where a
// wave needs its chunk before anyone could have written it).
__device__ __forceinline__ void quant_chunk_lane(const float* v, int layout, uint32_t* H, uint32_t* L, float& s) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; i++) m = fmaxf(m, fabsf(v[i]));
  const float inv = m > 0.0f ? 32512.0f / m : 0.0f;
  s = m / 32512.0f;
#pragma unroll
  for (int w = 0; w < 16; w++) {
    uint32_t hw = 0, lw = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int pos = 4 * w + b;  // byte position; which element lands here depends on the layout
      const int e = layout == ACT_NAT ? pos : ((pos & ~15) | ((pos & 3) << 2) | ((pos >> 2) & 3));
      const int X = (int)rintf(v[e] * inv);
      const int Hh = (X + 128) >> 8;
      const int Ll = X - (Hh << 8);
      hw |= ((uint32_t)Hh & 255u) << (8 * b);
      lw |= ((uint32_t)Ll & 255u) << (8 * b);
    }
    H[w] = hw;
    L[w] = lw;
  }
}

// A lane's quantized activation slice: chunk c (and c + LPR when CPL = 2).
template <int CPL>
struct ASlice {
  uint32_t H[16 * CPL], L[16 * CPL];
  float s[CPL];
  int SH[4 * CPL], SL[4 * CPL];  // per 16-element sub-block sums (Q2K min term)

  __device__ __forceinline__ void load(const uint8_t* q, const float* scales, int c, int LPR) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const uint8_t* p = q + (int64_t)(c + LPR * k) * CHUNK_BYTES;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint4 h = ld16(p + 16 * i), l = ld16(p + 64 + 16 * i);
        H[16 * k + 4 * i + 0] = h.x; H[16 * k + 4 * i + 1] = h.y; H[16 * k + 4 * i + 2] = h.z; H[16 * k + 4 * i + 3] = h.w;
        L[16 * k + 4 * i + 0] = l.x; L[16 * k + 4 * i + 1] = l.y; L[16 * k + 4 * i + 2] = l.z; L[16 * k + 4 * i + 3] = l.w;
      }
      s[k] = scales[c + LPR * k];
    }
  }
  __device__ __forceinline__ void sums() {
#pragma unroll
    for (int u = 0; u < 4 * CPL; u++) {
      int a = 0, b = 0;
#pragma unroll
      for (int w = 0; w < 4; w++) {
        a = dot4(H[4 * u + w], 0x01010101u, a);
        b = dot4(L[4 * u + w], 0x01010101u, b);
      }
      SH[u] = a;
      SL[u] = b;
    }
  }
};

// ---------------------------------------------------------------------------
// weight chunks: raw bytes of one lane's 64 weights of one row.  Addresses are
// one expert's plane bases (uniform per wave) plus 32-bit offsets whose row
// stride is a compile-time constant (NB blocks per row).
// ---------------------------------------------------------------------------
struct EPlanes {  // one expert's planes of a weight tensor in the device layout
  const uint8_t* scale;
  const uint8_t* a;
  const uint8_t* b;
};

__device__ __forceinline__ EPlanes expert_planes(const QMat& m, int e) {
  const int64_t r = (int64_t)e * m.rows * m.nb;  // blocks before this expert
  EPlanes p;
  if (m.fmt == FMT_IQ2) {
    p.scale = m.p_scale + r * 2;
    p.a = m.p_a + r * 64;
    p.b = nullptr;
  } else if (m.fmt == FMT_Q2K) {
    p.scale = m.p_scale + r * 4;
    p.a = m.p_a + r * 16;
    p.b = m.p_b + r * 64;
  } else {
    p.scale = m.p_scale + r * 2;
    p.a = m.p_a + r * 32;
    p.b = nullptr;
  }
  return p;
}

template <int FMT>
struct WChunk;

template <>
struct WChunk<FMT_IQ2> {  // words A0 B0 A1 B1 of sub-blocks 2(c%4), 2(c%4)+1 of superblock c/4
  uint4 v;
  uint32_t d;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t c) {
    v = ld16_stream(p.a + (row * NB * 64 + c * 16));
    d = reinterpret_cast<const uint16_t*>(p.scale)[row * NB + c / 4];
  }
};

template <>
struct WChunk<FMT_Q2K> {  // quants of sub-blocks 4(c%4) .. +3 of superblock c/4
  uint4 q;
  uint32_t sc, dm;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t c) {
    q = ld16_stream(p.b + (row * NB * 64 + c * 16));
    sc = *reinterpret_cast<const uint32_t*>(p.a + (row * NB * 16 + c * 4));
    dm = reinterpret_cast<const uint32_t*>(p.scale)[row * NB + c / 4];
  }
};

template <>
struct WChunk<FMT_Q8> {  // blocks 2c, 2c+1: 64 int8 quants, two fp16 scales
  uint4 q[4];
  uint32_t dd;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t c) {
    const uint8_t* src = p.a + (row * NB * 32 + c * 64);
#pragma unroll
    for (int i = 0; i < 4; i++) q[i] = ld16_stream(src + 16 * i);
    dd = reinterpret_cast<const uint32_t*>(p.scale)[row * (NB / 2) + c];
  }
};

// blocks per row of K = 64 * LPR * CPL inputs
template <int FMT, int LPR, int CPL>
struct Geo {
  static constexpr int K = 64 * LPR * CPL;
  static constexpr int NB = K / block_weights(FMT);
  static constexpr int RPS = 64 / LPR;  // rows per wave step
};

// IQ2 LDS tables: grid magnitudes as int8 (8 bytes per row) and, per 7 stored
// sign bits, the 0xFF byte mask of the negative elements (parity included).
struct Iq2Lds {
  uint2 mag[256];
  uint2 neg[128];
};

__device__ __forceinline__ void build_iq2_lds(const uint8_t* grid, Iq2Lds* t) {
  if (grid) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) t->mag[i] = reinterpret_cast<const uint2*>(grid)[i];
    for (int b = threadIdx.x; b < 128; b += blockDim.x) {
      const uint32_t s8 = b | ((__popc(b) & 1u) << 7);
      uint32_t w[2] = {0, 0};
#pragma unroll
      for (int p = 0; p < 8; p++)
        if ((s8 >> p) & 1u) w[p >> 2] |= 0xFFu << (8 * (p & 3));
      t->neg[b] = make_uint2(w[0], w[1]);
    }
  }
  __syncthreads();
}

// Dot of one weight chunk with the matching activation chunk (slice index k):
// returns sum w * (256 H + L) in fp32, i.e. the dot product divided by the
// activation scale.
template <int CPL>
__device__ __forceinline__ float chunk_dot(const WChunk<FMT_IQ2>& w, const ASlice<CPL>& a, int k, const Iq2Lds* t) {
  int ah = 0, al = 0;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const uint32_t A = h ? w.v.z : w.v.x;
    const uint32_t B = h ? w.v.w : w.v.y;
    int sh = 0, sl = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint2 mag = t->mag[(A >> (8 * i)) & 255u];
      const uint2 neg = t->neg[(B >> (7 * i)) & 127u];
      const uint32_t w0 = (mag.x ^ neg.x) + (neg.x & 0x01010101u);  // bytewise two's-complement negation
      const uint32_t w1 = (mag.y ^ neg.y) + (neg.y & 0x01010101u);
      const int g = 4 * h + i;  // group of 8 inside the chunk
      sh = dot4(w0, a.H[16 * k + 2 * g], sh);
      sh = dot4(w1, a.H[16 * k + 2 * g + 1], sh);
      sl = dot4(w0, a.L[16 * k + 2 * g], sl);
      sl = dot4(w1, a.L[16 * k + 2 * g + 1], sl);
    }
    const int mul = 2 * (int)(B >> 28) + 1;
    ah += mul * sh;
    al += mul * sl;
  }
  return (float)((ah << 8) + al) * half_bits_to_float(w.d);
}

template <int CPL>
__device__ __forceinline__ float chunk_dot(const WChunk<FMT_Q2K>& w, const ASlice<CPL>& a, int k, const Iq2Lds*) {
  int dh = 0, dl = 0, mh = 0, ml = 0;
  const uint32_t W[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
#pragma unroll
  for (int u = 0; u < 4; u++) {
    int qh = 0, ql = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t qd = (W[u] >> (2 * j)) & 0x03030303u;  // field j of each of the sub-block's 4 quant bytes
      qh = dot4(qd, a.H[16 * k + 4 * u + j], qh);
      ql = dot4(qd, a.L[16 * k + 4 * u + j], ql);
    }
    const int sc = (w.sc >> (8 * u)) & 15, m = (w.sc >> (8 * u + 4)) & 15;
    dh += sc * qh;
    dl += sc * ql;
    mh += m * a.SH[4 * k + u];
    ml += m * a.SL[4 * k + u];
  }
  return (float)((dh << 8) + dl) * half_bits_to_float(w.dm & 0xffffu) -
         (float)((mh << 8) + ml) * half_bits_to_float(w.dm >> 16);
}

template <int CPL>
__device__ __forceinline__ float chunk_dot(const WChunk<FMT_Q8>& w, const ASlice<CPL>& a, int k, const Iq2Lds*) {
  int h0 = 0, l0 = 0, h1 = 0, l1 = 0;
  const uint32_t Q[16] = {w.q[0].x, w.q[0].y, w.q[0].z, w.q[0].w, w.q[1].x, w.q[1].y, w.q[1].z, w.q[1].w,
                          w.q[2].x, w.q[2].y, w.q[2].z, w.q[2].w, w.q[3].x, w.q[3].y, w.q[3].z, w.q[3].w};
#pragma unroll
  for (int i = 0; i < 8; i++) {
    h0 = dot4(Q[i], a.H[16 * k + i], h0);
    l0 = dot4(Q[i], a.L[16 * k + i], l0);
    h1 = dot4(Q[8 + i], a.H[16 * k + 8 + i], h1);
    l1 = dot4(Q[8 + i], a.L[16 * k + 8 + i], l1);
  }
  return (float)((h0 << 8) + l0) * half_bits_to_float(w.dd & 0xffffu) +
         (float)((h1 << 8) + l1) * half_bits_to_float(w.dd >> 16);
}


// ---------------------------------------------------------------------------
// arguments
// ---------------------------------------------------------------------------
struct DecodeArgs {
  QMat gate, up, down;        // routed experts
  QMat s_gate, s_up, s_down;  // shared expert
  const uint8_t* grid;
  const float* w_router;
  int E, d, f, k, T;
  int has_shared;
  const void* x;
  int x_dtype;
  float* z;          // [T][E] logits (fused routing)
  int32_t* idx;      // [T][k] routes
  float* wt;         // [T][k]
  int32_t* idx_out;  // nullable user copies
  float* wt_out;
  uint8_t* xq;       // [T][d/64] quantized x chunks (layout of the routed gate/up format)
  float* xs;         // [T][d/64] their scales
  uint8_t* hq;       // [T*k + T][f/64] quantized SwiGLU outputs (layout of the consuming down format)
  float* hs;         // [T*k + T][f/64]
  float* y;          // [T][d]
  int fused_topk;
};

// gate/up + SwiGLU of GU_ROWS_PER_WAVE rows of one expert, by one wave; the
// resulting h values go to LDS (hrow[r]).  Loads of a whole batch of rows are
// issued before any is decoded (8 rows of 2-bit codes, 4 of Q8 codes, whose
// chunks are four times larger).
template <int FMT, int LPR, int CPL>
__device__ __forceinline__ void gateup_rows(const EPlanes& G, const EPlanes& U, int r0, const ASlice<CPL>& a,
                                            const Iq2Lds* t, float* hrow) {
  using Gm = Geo<FMT, LPR, CPL>;
  constexpr int RPS = Gm::RPS;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, c = lane % LPR;
  constexpr int STEPS = (GU_ROWS_PER_WAVE + RPS - 1) / RPS;
  constexpr int BATCH_ = (FMT == FMT_Q8 ? 4 : GU_ROWS_PER_WAVE) / CPL;
  constexpr int BATCH = BATCH_ < STEPS ? BATCH_ : STEPS;
  const bool lane_row_ok = RPS <= GU_ROWS_PER_WAVE || sub < GU_ROWS_PER_WAVE;  // rows of the last step
#pragma unroll
  for (int s0 = 0; s0 < STEPS; s0 += BATCH) {
    WChunk<FMT> wg[BATCH][CPL], wu[BATCH][CPL];
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
      const uint32_t n = r0 + (s0 + b) * RPS + (lane_row_ok ? sub : 0);
#pragma unroll
      for (int k = 0; k < CPL; k++) {
        wg[b][k].template load<Gm::NB>(G, n, c + LPR * k);
        wu[b][k].template load<Gm::NB>(U, n, c + LPR * k);
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
      float g = 0.0f, u = 0.0f;
#pragma unroll
      for (int k = 0; k < CPL; k++) {
        g += chunk_dot<CPL>(wg[b][k], a, k, t) * a.s[k];
        u += chunk_dot<CPL>(wu[b][k], a, k, t) * a.s[k];
      }
      g = group_sum<LPR>(g);
      u = group_sum<LPR>(u);
      if (c == LPR - 1 && lane_row_ok) hrow[(s0 + b) * RPS + sub] = silu(g) * u;
    }
  }
}

// ---------------------------------------------------------------------------
// K1: router logits | x quantization for K2 | shared gate/up
// ---------------------------------------------------------------------------
template <int FMT_S, int LPR, int CPL>
__global__ __launch_bounds__(DEC_THREADS) void decode_k1_kernel(DecodeArgs a, int n_router_blocks,
                                                                int n_quant_blocks, int gate_up_layout,
                                                                int down_layout_shared) {
  __shared__ Iq2Lds tab;
  __shared__ float hbuf[GU_ROWS_PER_BLOCK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int b = blockIdx.x;
  if (b < n_router_blocks) {
    // router: a wave per expert, tokens in a loop, fixed fp32 order (route.hip)
    const int e = b * DEC_WAVES + wave;
    if (e >= a.E) return;
    constexpr int CH = LPR * CPL / 4;  // d / 256 float4 chunks per lane
    float4 w[CH];
#pragma unroll
    for (int m = 0; m < CH; m++) w[m] = *reinterpret_cast<const float4*>(a.w_router + (int64_t)e * a.d + 4 * (lane + 64 * m));
    for (int t = 0; t < a.T; t++) {
      float4 xv[CH];
      if (a.x_dtype == X_BF16) {
        const uint16_t* xb = static_cast<const uint16_t*>(a.x) + (int64_t)t * a.d;
#pragma unroll
        for (int m = 0; m < CH; m++) {
          const uint2 bb = *reinterpret_cast<const uint2*>(xb + 4 * (lane + 64 * m));
          xv[m] = make_float4(__uint_as_float(bb.x << 16), __uint_as_float(bb.x & 0xffff0000u),
                              __uint_as_float(bb.y << 16), __uint_as_float(bb.y & 0xffff0000u));
        }
      } else {
        const float* xf = static_cast<const float*>(a.x) + (int64_t)t * a.d;
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
    return;
  }
  b -= n_router_blocks;
  if (b < n_quant_blocks) {
    // x quantization for K2: a wave per 64-element chunk
    const int nch = a.d / 64;
    const int task = b * DEC_WAVES + wave;
    if (task >= a.T * nch) return;
    const int t = task / nch, c = task % nch;
    float v;
    if (a.x_dtype == X_BF16)
      v = bf16_bits_to_float(static_cast<const uint16_t*>(a.x)[(int64_t)t * a.d + 64 * c + lane]);
    else
      v = static_cast<const float*>(a.x)[(int64_t)t * a.d + 64 * c + lane];
    quant_chunk_wave(v, gate_up_layout, a.xq + ((int64_t)t * nch + c) * CHUNK_BYTES, a.xs + (int64_t)t * nch + c);
    return;
  }
  b -= n_quant_blocks;
  // shared gate/up: 64 rows (one h chunk) of one token
  build_iq2_lds(a.grid, &tab);
  const int tiles = a.f / GU_ROWS_PER_BLOCK;
  const int tile = b % tiles, t = b / tiles;
  const int c = lane % LPR;
  ASlice<CPL> xs;
#pragma unroll
  for (int k = 0; k < CPL; k++) {
    const int cc = c + LPR * k;
    float v[64];
    if (a.x_dtype == X_BF16) {
      const uint16_t* xb = static_cast<const uint16_t*>(a.x) + (int64_t)t * a.d + 64 * cc;
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const uint4 bb = *reinterpret_cast<const uint4*>(xb + 8 * j);
        const uint32_t w4[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          v[8 * j + 2 * i] = __uint_as_float(w4[i] << 16);
          v[8 * j + 2 * i + 1] = __uint_as_float(w4[i] & 0xffff0000u);
        }
      }
    } else {
      const float* xf = static_cast<const float*>(a.x) + (int64_t)t * a.d + 64 * cc;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const float4 f4 = *reinterpret_cast<const float4*>(xf + 4 * j);
        v[4 * j] = f4.x;
        v[4 * j + 1] = f4.y;
        v[4 * j + 2] = f4.z;
        v[4 * j + 3] = f4.w;
      }
    }
    quant_chunk_lane(v, act_layout(FMT_S), xs.H + 16 * k, xs.L + 16 * k, xs.s[k]);
  }
  if constexpr (FMT_S == FMT_Q2K) xs.sums();
  gateup_rows<FMT_S, LPR, CPL>(expert_planes(a.s_gate, 0), expert_planes(a.s_up, 0),
                               tile * GU_ROWS_PER_BLOCK + wave * GU_ROWS_PER_WAVE, xs, &tab,
                               hbuf + wave * GU_ROWS_PER_WAVE);
  __syncthreads();
  if (wave == 0) {
    const int nfc = a.f / 64;
    const int src = a.T * a.k + t;
    quant_chunk_wave(hbuf[lane], down_layout_shared, a.hq + ((int64_t)src * nfc + tile) * CHUNK_BYTES,
                     a.hs + (int64_t)src * nfc + tile);
  }
}

// ---------------------------------------------------------------------------
// K2: routed gate/up.  grid = (f / 64, T * k).
// ---------------------------------------------------------------------------
template <int FMT, int LPR, int CPL>
__global__ __launch_bounds__(DEC_THREADS) void decode_k2_kernel(DecodeArgs a, int down_layout) {
  __shared__ Iq2Lds tab;
  __shared__ float hbuf[GU_ROWS_PER_BLOCK];
  __shared__ int s_expert;
  __shared__ int s_sel[TOPK_MAX_K];
  __shared__ float s_zs[TOPK_MAX_K];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int route = blockIdx.y, t = route / a.k, j = route % a.k;
  if (a.fused_topk) {
    if (wave == 0) {
      wave_topk(a.z + (int64_t)t * a.E, a.E, a.k, s_sel, s_zs);
      if (lane == 0) {  // lane 0 wrote the lists it reads back
        s_expert = s_sel[j];
        if (blockIdx.x == 0 && j == 0) {
          float w[TOPK_MAX_K];
          topk_weights(s_zs, a.k, w);
#pragma unroll
          for (int q = 0; q < TOPK_MAX_K; q++) {
            if (q >= a.k) continue;
            a.idx[(int64_t)t * a.k + q] = s_sel[q];
            a.wt[(int64_t)t * a.k + q] = w[q];
            if (a.idx_out) a.idx_out[(int64_t)t * a.k + q] = s_sel[q];
            if (a.wt_out) a.wt_out[(int64_t)t * a.k + q] = w[q];
          }
        }
      }
    }
  } else if (threadIdx.x == 0) {
    s_expert = a.idx[route];
  }
  build_iq2_lds(a.grid, &tab);  // includes the barrier that publishes s_expert
  const int e = s_expert;
  const int nfc = a.f / 64;
  if ((unsigned)e >= (unsigned)a.E) {  // caller route with an out-of-range expert id: contributes zero
    if (wave == 0) quant_chunk_wave(0.0f, down_layout, a.hq + ((int64_t)route * nfc + blockIdx.x) * CHUNK_BYTES,
                                    a.hs + (int64_t)route * nfc + blockIdx.x);
    return;
  }
  ASlice<CPL> xs;
  xs.load(a.xq + (int64_t)t * (a.d / 64) * CHUNK_BYTES, a.xs + (int64_t)t * (a.d / 64), lane % LPR, LPR);
  if constexpr (FMT == FMT_Q2K) xs.sums();
  gateup_rows<FMT, LPR, CPL>(expert_planes(a.gate, e), expert_planes(a.up, e),
                             blockIdx.x * GU_ROWS_PER_BLOCK + wave * GU_ROWS_PER_WAVE, xs, &tab,
                             hbuf + wave * GU_ROWS_PER_WAVE);
  __syncthreads();
  if (wave == 0)
    quant_chunk_wave(hbuf[lane], down_layout, a.hq + ((int64_t)route * nfc + blockIdx.x) * CHUNK_BYTES,
                     a.hs + (int64_t)route * nfc + blockIdx.x);
}

// ---------------------------------------------------------------------------
// K3: down + combine.  grid = (d / DN_ROWS_PER_BLOCK, T).  Tasks: routed
// route j (all rows of the tile), then the shared expert in two row halves.
// Each task's row dots go to LDS; then y = sum_j wt_j ye_j + ysh in that
// fixed order.
// ---------------------------------------------------------------------------
template <int FMT, int LPR, int CPL, int ROWS>
__device__ __forceinline__ void down_task(const EPlanes& D, int r0, const uint8_t* hq, const float* hs,
                                          const Iq2Lds* t, float* out) {
  using Gm = Geo<FMT, LPR, CPL>;
  constexpr int RPS = Gm::RPS;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, c = lane % LPR;
  ASlice<CPL> hsl;
  hsl.load(hq, hs, c, LPR);
  if constexpr (FMT == FMT_Q2K) hsl.sums();
  constexpr int STEPS = (ROWS + RPS - 1) / RPS;
  constexpr int BATCH_ = (FMT == FMT_Q8 ? 4 : 8) / CPL;
  constexpr int BATCH = BATCH_ < STEPS ? BATCH_ : STEPS;
  const bool lane_row_ok = RPS <= ROWS || sub < ROWS;
#pragma unroll
  for (int s0 = 0; s0 < STEPS; s0 += BATCH) {
    WChunk<FMT> w[BATCH][CPL];
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
      const uint32_t n = r0 + (s0 + b) * RPS + (lane_row_ok ? sub : 0);
#pragma unroll
      for (int k = 0; k < CPL; k++) w[b][k].template load<Gm::NB>(D, n, c + LPR * k);
    }
#pragma unroll
    for (int b = 0; b < BATCH; b++) {
      float v = 0.0f;
#pragma unroll
      for (int k = 0; k < CPL; k++) v += chunk_dot<CPL>(w[b][k], hsl, k, t) * hsl.s[k];
      v = group_sum<LPR>(v);
      if (c == LPR - 1 && lane_row_ok) out[(s0 + b) * RPS + sub] = v;
    }
  }
}

template <int FMT_R, int FMT_S, int LPR, int CPL>
__global__ __launch_bounds__(DEC_THREADS) void decode_k3_kernel(DecodeArgs a) {
  __shared__ Iq2Lds tab;
  __shared__ float ye[(TOPK_MAX_K + 1) * DN_ROWS_PER_BLOCK];
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.y;
  const int row0 = blockIdx.x * DN_ROWS_PER_BLOCK;
  build_iq2_lds(a.grid, &tab);
  const int nfc = a.f / 64;
  const int n_tasks = a.k + (a.has_shared ? 2 : 0);
  for (int task = wave; task < n_tasks; task += DEC_WAVES) {
    if (task < a.k) {
      const int src = t * a.k + task;
      const int e = a.idx[src];
      if ((unsigned)e >= (unsigned)a.E) {  // out-of-range caller route: contributes zero
        if ((threadIdx.x & 63) < DN_ROWS_PER_BLOCK) ye[task * DN_ROWS_PER_BLOCK + (threadIdx.x & 63)] = 0.0f;
        continue;
      }
      down_task<FMT_R, LPR, CPL, DN_ROWS_PER_BLOCK>(expert_planes(a.down, e), row0,
                                                   a.hq + (int64_t)src * nfc * CHUNK_BYTES, a.hs + (int64_t)src * nfc,
                                                   &tab, ye + task * DN_ROWS_PER_BLOCK);
    } else {
      const int src = a.T * a.k + t;
      const int half = task - a.k;
      down_task<FMT_S, LPR, CPL, DN_ROWS_PER_BLOCK / 2>(
          expert_planes(a.s_down, 0), row0 + half * (DN_ROWS_PER_BLOCK / 2), a.hq + (int64_t)src * nfc * CHUNK_BYTES,
          a.hs + (int64_t)src * nfc, &tab, ye + a.k * DN_ROWS_PER_BLOCK + half * (DN_ROWS_PER_BLOCK / 2));
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < DN_ROWS_PER_BLOCK) {
    const int n = threadIdx.x;
    float acc = 0.0f;
    for (int q = 0; q < a.k; q++) acc = __builtin_fmaf(a.wt[(int64_t)t * a.k + q], ye[q * DN_ROWS_PER_BLOCK + n], acc);
    if (a.has_shared) acc += ye[a.k * DN_ROWS_PER_BLOCK + n];
    a.y[(int64_t)t * a.d + row0 + n] = acc;
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
#define FMT_SWITCH(fmt, F, ...)                                      \
  switch (fmt) {                                                     \
    case FMT_IQ2: { constexpr int F = FMT_IQ2; __VA_ARGS__; } break; \
    case FMT_Q2K: { constexpr int F = FMT_Q2K; __VA_ARGS__; } break; \
    default: { constexpr int F = FMT_Q8; __VA_ARGS__; } break;       \
  }

// (lanes per row, chunks per lane) for a row of K inputs: K = 64 * LPR * CPL
#define GEO_SWITCH(K, LPR, CPL, ...)                                                   \
  switch (K) {                                                                         \
    case 256: { constexpr int LPR = 4, CPL = 1; __VA_ARGS__; } break;                  \
    case 512: { constexpr int LPR = 8, CPL = 1; __VA_ARGS__; } break;                  \
    case 1024: { constexpr int LPR = 16, CPL = 1; __VA_ARGS__; } break;                \
    case 2048: { constexpr int LPR = 32, CPL = 1; __VA_ARGS__; } break;                \
    case 4096: { constexpr int LPR = 64, CPL = 1; __VA_ARGS__; } break;                \
    default: { constexpr int LPR = 64, CPL = 2; __VA_ARGS__; } break;                  \
  }

size_t decode_quant_bytes(int T, int k, int d, int f) {
  return (size_t)T * (d / 64) * (CHUNK_BYTES + 4) + (size_t)(T * k + T) * (f / 64) * (CHUNK_BYTES + 4);
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t s) {
  DecodeArgs a;
  a.gate = make_qmat(L.w_gate, L.fmt_gate_up, L.E, L.f, L.d);
  a.up = make_qmat(L.w_up, L.fmt_gate_up, L.E, L.f, L.d);
  a.down = make_qmat(L.w_down, L.fmt_down, L.E, L.d, L.f);
  if (L.has_shared) {
    a.s_gate = make_qmat(L.s_gate, L.fmt_shared, 1, L.f, L.d);
    a.s_up = make_qmat(L.s_up, L.fmt_shared, 1, L.f, L.d);
    a.s_down = make_qmat(L.s_down, L.fmt_shared, 1, L.d, L.f);
  } else {
    a.s_gate = a.s_up = a.s_down = a.gate;
  }
  a.grid = L.grid;
  a.w_router = L.w_router;
  a.E = L.E; a.d = L.d; a.f = L.f; a.k = L.k; a.T = L.T;
  a.has_shared = L.has_shared;
  a.x = L.x; a.x_dtype = L.x_dtype;
  a.z = L.z; a.idx = L.idx; a.wt = L.wt; a.idx_out = L.idx_out; a.wt_out = L.wt_out;
  uint8_t* q = static_cast<uint8_t*>(L.quant);
  a.xq = q;
  a.xs = reinterpret_cast<float*>(q + (size_t)L.T * (L.d / 64) * CHUNK_BYTES);
  uint8_t* q2 = reinterpret_cast<uint8_t*>(a.xs + (size_t)L.T * (L.d / 64));
  a.hq = q2;
  a.hs = reinterpret_cast<float*>(q2 + (size_t)(L.T * L.k + L.T) * (L.f / 64) * CHUNK_BYTES);
  a.y = L.y;
  a.fused_topk = L.fused_topk;
  if (L.T == 0) return hipSuccess;
  const int nrb = L.fused_topk ? (L.E + DEC_WAVES - 1) / DEC_WAVES : 0;
  const int nqb = (L.T * (L.d / 64) + DEC_WAVES - 1) / DEC_WAVES;
  const int nsb = L.has_shared ? (L.f / GU_ROWS_PER_BLOCK) * L.T : 0;
  const int fs = L.has_shared ? L.fmt_shared : L.fmt_gate_up;
  const int gu_layout = act_layout(L.fmt_gate_up);
  const int sh_down_layout = act_layout(fs);
  const int dn_layout = act_layout(L.fmt_down);
  {
    const int pid = prof_begin("decode_router_shared_gateup", s);
    GEO_SWITCH(L.d, LPR, CPL, FMT_SWITCH(fs, F, (decode_k1_kernel<F, LPR, CPL><<<dim3(nrb + nqb + nsb), DEC_THREADS, 0, s>>>(
                                                     a, nrb, nqb, gu_layout, sh_down_layout))))
    prof_end(pid, s);
  }
  {
    const int pid = prof_begin("decode_gateup", s);
    GEO_SWITCH(L.d, LPR, CPL, FMT_SWITCH(L.fmt_gate_up, F, (decode_k2_kernel<F, LPR, CPL><<<dim3(L.f / GU_ROWS_PER_BLOCK, L.T * L.k), DEC_THREADS, 0, s>>>(a, dn_layout))))
    prof_end(pid, s);
  }
  {
    const int pid = prof_begin("decode_down_combine", s);
    GEO_SWITCH(L.f, LPR, CPL, FMT_SWITCH(L.fmt_down, FR, FMT_SWITCH(fs, FS, (decode_k3_kernel<FR, FS, LPR, CPL><<<dim3(L.d / DN_ROWS_PER_BLOCK, L.T), DEC_THREADS, 0, s>>>(a)))))
    prof_end(pid, s);
  }
  return hipGetLastError();
}

}  // namespace qmoe
