// Pieces shared by the three decode kernels (decode_k1/k2/k3.hip).
//
// Decode reads every selected weight once per token and is bound by HBM
// bytes ("YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 4.4:
// decoding is memory-bound and the expert kernel streams whole cache lines,
// decoding the codes in registers).  On gfx950 the 2-bit formats are close to
// a second ceiling as well: at HBM speed a CU must consume ~50 IQ2 weights per
// clock, which leaves ~1.3 vector instructions per weight.  Everything below
// is shaped by that budget:
//
//   * Activations (x, and the SwiGLU output h) are integers X, |X| <= 0x7777,
//     times one fp32 scale (per 64 inputs for x, per 16 for h).  X is kept as
//     four planes of balanced hex digits D_p in [-8, 7] (X = sum 16^p D_p),
//     packed 8 per dword as signed nibbles, so that 8 weights meet 8
//     activation digits in one v_dot8_i32_i4.  The digits come out of
//     Z = (X + 0x8888) ^ 0x8888, whose hex digits are the two's-complement
//     nibbles of D_p.  The quantization error is at most s/2 = max|v|/61166
//     per value: a relative error ~1e-5 on a dot product.
//   * IQ2 weights come from one LDS table of 32768 dwords indexed by (grid
//     row, 7 stored sign bits): the 8 signed magnitudes as nibbles, signs and
//     parity already applied.  One ds_read_b32 per 8 weights.
//   * Q2K quants are already 2-bit integers: (W & 0x33333333) and
//     ((W >> 2) & 0x33333333) are 8 nibble weights each.
//   * Q8 weights use v_dot4 against the activation digit planes widened to
//     bytes (16 D_p), or against 16-bit activations split into two byte
//     planes where a lane quantizes its own inputs.
//
// All integer sums are exact; each row's lanes reduce their fp32 partials
// with DPP in a fixed order, so results are deterministic.
//
// Loads: a row of K inputs is cut into 16-byte pieces (64 inputs of a 2-bit
// format, 16 of Q8) and the 64 lanes of a wave read consecutive pieces, so
// every load instruction reads 1 KB of consecutive bytes.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace qmoe {
namespace dec {

constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr int XMAX = 0x7777;      // |X| bound of the fixed-point activations
constexpr int G16_BYTES = 32;     // one quantized group of 16 activations: 2 halves x 4 planes x 4 B
constexpr int CHUNK_BYTES = 128;  // 64 activations (four groups)
constexpr int DN_ROWS = 16;       // down rows per block of the last kernel
constexpr uint32_t SPIN_LIMIT = 1u << 22;

// Order of the 16 activations of a group inside its two halves x 8 nibbles,
// chosen per consuming weight format so that weight words need no shuffling:
//   NAT (IQ2): half hh holds elements 8 hh .. 8 hh + 7, nibble n = element n;
//   Q2K      : half hh holds the elements of parity hh, nibble n = element 2n + hh
//              (Q2K fields 0/2 and 1/3 of each quant byte);
//   Q8       : half hh holds elements 8 hh + 0..7 with nibble 2i = element i and
//              nibble 2i + 1 = element 4 + i (so the even and odd nibbles widen
//              to the bytes of two consecutive int8 weight words).
enum : int { NIB_NAT = 0, NIB_Q2K = 1, NIB_Q8 = 2 };

__host__ __device__ constexpr int nib_layout(int fmt) {
  return fmt == FMT_Q2K ? NIB_Q2K : (fmt == FMT_Q8 ? NIB_Q8 : NIB_NAT);
}

__host__ __device__ constexpr int nib_elem(int layout, int hh, int n) {
  return layout == NIB_Q2K ? 2 * n + hh : (layout == NIB_Q8 ? 8 * hh + ((n & 1) ? 4 + (n >> 1) : (n >> 1)) : 8 * hh + n);
}

// A row of K inputs in format FMT: 16-byte pieces, lanes per row, pieces per
// lane, rows per wave step.  Lane (sub, c) with sub = lane / LPR, c = lane %
// LPR reads pieces c + LPR * k (k < CPL) of row sub of the step.
template <int FMT, int K>
struct Geo {
  static constexpr int PW = FMT == FMT_Q8 ? 16 : 64;  // inputs per piece
  static constexpr int PR = K / PW;                   // pieces per row
  static constexpr int LPR = PR < 64 ? PR : 64;
  static constexpr int CPL = PR / LPR;
  static constexpr int RPS = 64 / LPR;
  static constexpr int NB = K / block_weights(FMT);   // blocks per row
};

__device__ __forceinline__ int dot8(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}
// sum_p 16^p acc[p]
__device__ __forceinline__ int combine4(const int* acc) { return ((acc[3] * 16 + acc[2]) * 16 + acc[1]) * 16 + acc[0]; }

// ---------------------------------------------------------------------------
// cross-lane sums and maxima with DPP (fixed order)
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Sum of v over each aligned group of LPR lanes; the total lands in the
// group's last lane (c == LPR - 1).
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

// Maximum of v >= 0 over each 16-lane row (GROUP = 16) or the wave (GROUP =
// 64), returned to every lane of the row / wave.
template <int GROUP>
__device__ __forceinline__ float group_max_nonneg(float v) {
  v = fmaxf(v, dpp_f<0x111, 0xf>(v));
  v = fmaxf(v, dpp_f<0x112, 0xf>(v));
  v = fmaxf(v, dpp_f<0x114, 0xf>(v));
  v = fmaxf(v, dpp_f<0x118, 0xf>(v));  // lane 15 of each row holds the row maximum
  if constexpr (GROUP == 16) {
    return __shfl(v, (int)((threadIdx.x & 63) | 15), 64);
  } else {
    v = fmaxf(v, dpp_f<0x142, 0xa>(v));
    v = fmaxf(v, dpp_f<0x143, 0xc>(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  }
}

__device__ __forceinline__ uint32_t to_digits(float v, float inv) {
  const int X = (int)rintf(v * inv);  // |X| <= XMAX
  return ((uint32_t)(X + 0x8888) ^ 0x8888u) & 0xffffu;
}

// Quantize 64 values (lane e holds element e of 4 consecutive groups of 16)
// with one scale per GROUP lanes, and write the groups' nibble planes in
// `layout`: 32 bytes per group at out, scales at scale_out[e / GROUP].  Only
// the first n_groups groups are written.
template <int GROUP>
__device__ __forceinline__ void quant_wave(float v, int layout, uint8_t* __restrict__ out,
                                           float* __restrict__ scale_out, int n_groups) {
  const int lane = threadIdx.x & 63;
  const float m = group_max_nonneg<GROUP>(fabsf(v));
  const float inv = m > 0.0f ? (float)XMAX / m : 0.0f;
  const uint32_t Z = to_digits(v, inv);
  const int q = (lane >> 3) & 3, hh = (lane >> 2) & 1, p = lane & 3;  // word of lanes 0..31
  uint32_t word = 0;
#pragma unroll
  for (int n = 0; n < 8; n++) {
    const uint32_t z = (uint32_t)__shfl((int)Z, 16 * q + nib_elem(layout, hh, n), 64);
    word |= ((z >> (4 * p)) & 15u) << (4 * n);
  }
  if (lane < 32 && q < n_groups) reinterpret_cast<uint32_t*>(out)[lane] = word;
  if ((lane % GROUP) == 0 && lane / 16 < n_groups) scale_out[lane / GROUP] = m / (float)XMAX;
}

// ---------------------------------------------------------------------------
// activation slices held by a lane: CPL pieces
// ---------------------------------------------------------------------------
// 2-bit pieces (64 inputs = 4 groups of 16): digit planes, one scale per piece
// (chunk-quantized x) or per group (PER16, group-quantized h), and for Q2K the
// per-group sums of X (the min term).
template <int CPL, bool PER16>
struct ActNib {
  uint32_t w[CPL][4][2][4];
  float s[CPL][PER16 ? 4 : 1];
  int Ai[CPL][4];    // sum of X over each group (chunk-scaled)
  float As[CPL][4];  // scale * sum of X (group-scaled)

  // quantized groups at q (32 bytes each), scales at sc
  template <int LPR>
  __device__ __forceinline__ void load(const uint8_t* q, const float* sc, int c) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int pc = c + LPR * k;
      const uint8_t* p = q + (int64_t)pc * CHUNK_BYTES;
#pragma unroll
      for (int u = 0; u < 4; u++)
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const uint4 v = ld16(p + 32 * u + 16 * hh);
          w[k][u][hh][0] = v.x;
          w[k][u][hh][1] = v.y;
          w[k][u][hh][2] = v.z;
          w[k][u][hh][3] = v.w;
        }
      if constexpr (PER16) {
        const float4 s4 = *reinterpret_cast<const float4*>(sc + 4 * pc);
        s[k][0] = s4.x;
        s[k][1] = s4.y;
        s[k][2] = s4.z;
        s[k][3] = s4.w;
      } else {
        s[k][0] = sc[pc];
      }
    }
  }
  // per-group sums of X (needed by Q2K's min term)
  __device__ __forceinline__ void sums() {
#pragma unroll
    for (int k = 0; k < CPL; k++)
#pragma unroll
      for (int u = 0; u < 4; u++) {
        int acc[4];
#pragma unroll
        for (int p = 0; p < 4; p++) acc[p] = dot8(w[k][u][1][p], 0x11111111u, dot8(w[k][u][0][p], 0x11111111u, 0));
        Ai[k][u] = combine4(acc);
        if constexpr (PER16) As[k][u] = s[k][u] * (float)Ai[k][u];
      }
  }
  // lane-local quantization of 64 consecutive fp32 inputs per piece (chunk
  // scaled): v points at input 0 of the row
  template <int LPR>
  __device__ __forceinline__ void from_f32(const float* v, int c, int layout) {
    static_assert(!PER16, "lane-local quantization is chunk-scaled");
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int pc = c + LPR * k;
      float x[64];
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const float4 f = *reinterpret_cast<const float4*>(v + 64 * pc + 4 * j);
        x[4 * j] = f.x;
        x[4 * j + 1] = f.y;
        x[4 * j + 2] = f.z;
        x[4 * j + 3] = f.w;
      }
      quantize_local(x, k, layout);
    }
  }
  template <int LPR>
  __device__ __forceinline__ void from_bf16(const uint16_t* v, int c, int layout) {
    static_assert(!PER16, "lane-local quantization is chunk-scaled");
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int pc = c + LPR * k;
      float x[64];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const uint4 b = ld16(v + 64 * pc + 8 * j);
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          x[8 * j + 2 * i] = __uint_as_float(bw[i] << 16);
          x[8 * j + 2 * i + 1] = __uint_as_float(bw[i] & 0xffff0000u);
        }
      }
      quantize_local(x, k, layout);
    }
  }
  __device__ __forceinline__ void quantize_local(const float* x, int k, int layout) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; i++) m = fmaxf(m, fabsf(x[i]));
    const float inv = m > 0.0f ? (float)XMAX / m : 0.0f;
    s[k][0] = m / (float)XMAX;
    uint32_t Z[64];
#pragma unroll
    for (int i = 0; i < 64; i++) Z[i] = to_digits(x[i], inv);
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int p = 0; p < 4; p++) {
          uint32_t word = 0;
#pragma unroll
          for (int n = 0; n < 8; n++) {
            const int e = 16 * u + (layout == NIB_Q2K ? 2 * n + hh : 8 * hh + n);
            word |= ((Z[e] >> (4 * p)) & 15u) << (4 * n);
          }
          w[k][u][hh][p] = word;
        }
  }
};

// Q8 pieces (16 inputs = one group) from quantized groups: the digit planes
// widened to bytes 16 D_p (even nibbles -> the first weight word of a half,
// odd nibbles -> the second).  One scale per piece.
template <int CPL>
struct ActQ8N {
  uint32_t e[CPL][2][4][2];
  float s[CPL];
  // GSCALE: 16 for group-quantized h (scale per piece), 64 for chunk-quantized x
  template <int LPR, int GSCALE>
  __device__ __forceinline__ void load(const uint8_t* q, const float* sc, int c) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int pc = c + LPR * k;
      const uint8_t* p = q + (int64_t)pc * G16_BYTES;
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        const uint4 v = ld16(p + 16 * hh);
        const uint32_t N[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int pl = 0; pl < 4; pl++) {
          e[k][hh][pl][0] = (N[pl] << 4) & 0xf0f0f0f0u;
          e[k][hh][pl][1] = N[pl] & 0xf0f0f0f0u;
        }
      }
      s[k] = sc[GSCALE == 16 ? pc : pc / 4] * 0.0625f;  // bytes carry 16 D_p
    }
  }
};

// Q8 pieces from lane-local 16-bit quantization of fp32 inputs: two byte
// planes H, L with X = 256 H + L, |X| <= 32512, one scale per piece.
template <int CPL>
struct ActQ8B {
  uint32_t H[CPL][4], L[CPL][4];
  float s[CPL];
  __device__ __forceinline__ void quantize_piece(const float* x, int k) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) m = fmaxf(m, fabsf(x[i]));
    const float inv = m > 0.0f ? 32512.0f / m : 0.0f;
    s[k] = m / 32512.0f;
#pragma unroll
    for (int wd = 0; wd < 4; wd++) {
      uint32_t hw = 0, lw = 0;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const int X = (int)rintf(x[4 * wd + b] * inv);
        const int Hh = (X + 128) >> 8;  // floor((X + 128) / 256), in [-127, 127]
        const int Ll = X - (Hh << 8);   // in [-128, 127]
        hw |= ((uint32_t)Hh & 255u) << (8 * b);
        lw |= ((uint32_t)Ll & 255u) << (8 * b);
      }
      H[k][wd] = hw;
      L[k][wd] = lw;
    }
  }
  template <int LPR>
  __device__ __forceinline__ void from_f32(const float* v, int c) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int pc = c + LPR * k;
      float x[16];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float4 f = *reinterpret_cast<const float4*>(v + 16 * pc + 4 * j);
        x[4 * j] = f.x;
        x[4 * j + 1] = f.y;
        x[4 * j + 2] = f.z;
        x[4 * j + 3] = f.w;
      }
      quantize_piece(x, k);
    }
  }
  template <int LPR>
  __device__ __forceinline__ void from_bf16(const uint16_t* v, int c) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int pc = c + LPR * k;
      float x[16];
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const uint4 b = ld16(v + 16 * pc + 8 * j);
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          x[8 * j + 2 * i] = __uint_as_float(bw[i] << 16);
          x[8 * j + 2 * i + 1] = __uint_as_float(bw[i] & 0xffff0000u);
        }
      }
      quantize_piece(x, k);
    }
  }
};

// ---------------------------------------------------------------------------
// weight pieces: one lane's 16 bytes of codes of one row plus its scales
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
struct Piece;

template <>
struct Piece<FMT_IQ2> {  // words A0 B0 A1 B1 of sub-blocks 2 (pc % 4), +1 of superblock pc / 4
  uint4 v;
  uint32_t d;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t pc) {
    v = ld16_stream(p.a + (row * NB * 64 + pc * 16));
    d = reinterpret_cast<const uint16_t*>(p.scale)[row * NB + pc / 4];
  }
};

template <>
struct Piece<FMT_Q2K> {  // quants of sub-blocks 4 (pc % 4) .. +3 of superblock pc / 4
  uint4 q;
  uint32_t sc, dm;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t pc) {
    q = ld16_stream(p.b + (row * NB * 64 + pc * 16));
    sc = *reinterpret_cast<const uint32_t*>(p.a + (row * NB * 16 + pc * 4));
    dm = reinterpret_cast<const uint32_t*>(p.scale)[row * NB + pc / 4];
  }
};

template <>
struct Piece<FMT_Q8> {  // 16 int8 quants: half of block pc / 2
  uint4 q;
  uint32_t d;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t pc) {
    q = ld16_stream(p.a + (row * NB * 32 + pc * 16));
    d = reinterpret_cast<const uint16_t*>(p.scale)[row * NB + pc / 2];
  }
};

// ---------------------------------------------------------------------------
// IQ2 nibble table: entry (g, b) = the 8 weights of grid row g with stored
// sign bits b (and the parity sign), as signed nibbles (element n in nibble
// n).  128 KB of LDS, built per block.
// ---------------------------------------------------------------------------
constexpr int IQ2_TAB_WORDS = 256 * 128;
constexpr size_t IQ2_TAB_BYTES = (size_t)IQ2_TAB_WORDS * 4;

struct Iq2Aux {
  uint2 pm[256];       // per grid row: magnitudes as nibbles, and their negations
  uint32_t mask[128];  // per stored sign pattern: 0xF in every negative nibble
};

// The table is built in two steps so that the global loads it needs (the
// grid) can be in flight together with other loads: iq2_aux_prepare() for
// items 0..383 (grid row i for i < 256, sign pattern i - 256 below 384), each
// item by one thread with the grid row it loaded, then, after a barrier,
// iq2_fill_table() by all 512 threads, then another barrier.
__device__ __forceinline__ uint2 iq2_grid_row(const uint8_t* __restrict__ grid, int item) {
  return (item >= 0 && item < 256) ? reinterpret_cast<const uint2*>(grid)[item] : make_uint2(0, 0);
}

__device__ __forceinline__ void iq2_aux_prepare(uint2 g, int item, Iq2Aux* aux) {
  if (item >= 0 && item < 256) {
    uint32_t pos = 0, neg = 0;
#pragma unroll
    for (int n = 0; n < 8; n++) {
      const uint32_t m = ((n < 4 ? g.x : g.y) >> (8 * (n & 3))) & 255u;
      pos |= (m & 15u) << (4 * n);
      neg |= ((16u - m) & 15u) << (4 * n);
    }
    aux->pm[item] = make_uint2(pos, neg);
  } else if (item >= 256 && item < 384) {
    const uint32_t b = item - 256;
    const uint32_t s8 = b | ((__popc(b) & 1u) << 7);
    uint32_t mk = 0;
#pragma unroll
    for (int n = 0; n < 8; n++) mk |= ((s8 >> n) & 1u) ? (0xfu << (4 * n)) : 0u;
    aux->mask[b] = mk;
  }
}

__device__ __forceinline__ void iq2_fill_table(uint32_t* tab, const Iq2Aux* aux) {
  const int t = threadIdx.x;
#pragma unroll 4
  for (int it = 0; it < IQ2_TAB_WORDS / 4 / THREADS; it++) {
    const int u = t + THREADS * it;  // entries 4u .. 4u + 3: grid row u / 32, sign patterns 4 (u % 32) + 0..3
    const uint2 pm = aux->pm[u >> 5];
    const uint4 mk = *reinterpret_cast<const uint4*>(&aux->mask[4 * (u & 31)]);
    uint4 o;
    o.x = (mk.x & pm.y) | (~mk.x & pm.x);
    o.y = (mk.y & pm.y) | (~mk.y & pm.x);
    o.z = (mk.z & pm.y) | (~mk.z & pm.x);
    o.w = (mk.w & pm.y) | (~mk.w & pm.x);
    reinterpret_cast<uint4*>(tab)[u] = o;
  }
}

// Whole build by all 512 threads of the block, with its barriers.
__device__ __forceinline__ void build_iq2_table(const uint8_t* __restrict__ grid, uint32_t* tab, Iq2Aux* aux) {
  iq2_aux_prepare(iq2_grid_row(grid, threadIdx.x), threadIdx.x, aux);
  __syncthreads();
  iq2_fill_table(tab, aux);
  __syncthreads();
}

// Quantize x_t (d values, fp32 or bf16) into chunks of 64 in `layout` at
// q / sc (LDS or global), with the waves w0 .. WAVES-1 of the block: every
// wave first issues the loads of all its chunks, then quantizes them.
template <int MAXC>
__device__ __forceinline__ void quant_x_chunks(const void* x, int x_dtype, int64_t off, int nch, int layout,
                                               uint8_t* q, float* sc, int w0) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = WAVES - w0;
  if (wave < w0) return;
  float v[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; j++) {
    const int ch = (wave - w0) + nw * j;
    const int chc = ch < nch ? ch : nch - 1;
    v[j] = x_dtype == X_BF16 ? bf16_bits_to_float(static_cast<const uint16_t*>(x)[off + 64 * chc + lane])
                             : static_cast<const float*>(x)[off + 64 * chc + lane];
  }
#pragma unroll
  for (int j = 0; j < MAXC; j++) {
    const int ch = (wave - w0) + nw * j;
    if (ch < nch) quant_wave<64>(v[j], layout, q + (int64_t)ch * CHUNK_BYTES, sc + ch, 4);
  }
}

// ---------------------------------------------------------------------------
// dot products of one weight piece with the matching activation slice k;
// each returns the piece's contribution in real units
// ---------------------------------------------------------------------------
template <int CPL, bool PER16>
__device__ __forceinline__ float piece_dot(const Piece<FMT_IQ2>& w, const ActNib<CPL, PER16>& a, int k,
                                           const uint32_t* tab) {
  const uint32_t AB[4] = {w.v.x, w.v.y, w.v.z, w.v.w};
  int itot = 0;
  float ftot = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const uint32_t A = AB[2 * h], B = AB[2 * h + 1];
    const int mul = 2 * (int)(B >> 28) + 1;
    int acc[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t e = tab[(((A >> (8 * i)) & 255u) << 7) | ((B >> (7 * i)) & 127u)];
      const int q = 2 * h + (i >> 1), hh = i & 1, slot = PER16 ? (i >> 1) : 0;
#pragma unroll
      for (int p = 0; p < 4; p++) acc[slot][p] = dot8(e, a.w[k][q][hh][p], acc[slot][p]);
    }
    if constexpr (PER16) {
      ftot += (float)(combine4(acc[0]) * mul) * a.s[k][2 * h] + (float)(combine4(acc[1]) * mul) * a.s[k][2 * h + 1];
    } else {
      itot += combine4(acc[0]) * mul;
    }
  }
  const float d = half_bits_to_float(w.d);
  if constexpr (PER16)
    return ftot * d;
  else
    return (float)itot * (a.s[k][0] * d);
}

template <int CPL, bool PER16>
__device__ __forceinline__ float piece_dot(const Piece<FMT_Q2K>& w, const ActNib<CPL, PER16>& a, int k,
                                           const uint32_t*) {
  const uint32_t W[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
  int im = 0, in = 0;
  float fm = 0.0f, fn = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const uint32_t N0 = W[u] & 0x33333333u, N1 = (W[u] >> 2) & 0x33333333u;
    int acc[4];
#pragma unroll
    for (int p = 0; p < 4; p++) acc[p] = dot8(N1, a.w[k][u][1][p], dot8(N0, a.w[k][u][0][p], 0));
    const int D = combine4(acc);
    const int sc = (int)((w.sc >> (8 * u)) & 15u), m = (int)((w.sc >> (8 * u + 4)) & 15u);
    if constexpr (PER16) {
      fm += (float)(sc * D) * a.s[k][u];
      fn += (float)m * a.As[k][u];
    } else {
      im += sc * D;
      in += m * a.Ai[k][u];
    }
  }
  const float d = half_bits_to_float(w.dm & 0xffffu), dmin = half_bits_to_float(w.dm >> 16);
  if constexpr (PER16)
    return fm * d - fn * dmin;
  else
    return a.s[k][0] * ((float)im * d - (float)in * dmin);
}

template <int CPL>
__device__ __forceinline__ float piece_dot(const Piece<FMT_Q8>& w, const ActQ8N<CPL>& a, int k, const uint32_t*) {
  int acc[4];
#pragma unroll
  for (int p = 0; p < 4; p++)
    acc[p] = dot4(w.q.w, a.e[k][1][p][1],
                  dot4(w.q.z, a.e[k][1][p][0], dot4(w.q.y, a.e[k][0][p][1], dot4(w.q.x, a.e[k][0][p][0], 0))));
  return (float)combine4(acc) * (a.s[k] * half_bits_to_float(w.d));
}

template <int CPL>
__device__ __forceinline__ float piece_dot(const Piece<FMT_Q8>& w, const ActQ8B<CPL>& a, int k, const uint32_t*) {
  const int h = dot4(w.q.w, a.H[k][3], dot4(w.q.z, a.H[k][2], dot4(w.q.y, a.H[k][1], dot4(w.q.x, a.H[k][0], 0))));
  const int l = dot4(w.q.w, a.L[k][3], dot4(w.q.z, a.L[k][2], dot4(w.q.y, a.L[k][1], dot4(w.q.x, a.L[k][0], 0))));
  return (float)(h * 256 + l) * (a.s[k] * half_bits_to_float(w.d));
}

// ---------------------------------------------------------------------------
// arguments of the three kernels
// ---------------------------------------------------------------------------
struct DecodeArgs {
  QMat gate, up, down;        // routed experts
  QMat s_gate, s_up, s_down;  // shared expert
  const uint8_t* grid;
  const float* w_router;
  int E, d, f, k, T;
  int has_shared;
  int fused_topk;
  const void* x;
  int x_dtype;
  float* z;          // [T][E] logits (fused routing)
  int32_t* idx;      // [T][k] routes
  float* wt;         // [T][k]
  int32_t* idx_out;  // nullable caller copies
  float* wt_out;
  float* hsh;        // [T][f] shared SwiGLU output, fp32
  uint8_t* hq;       // [T*k + T][f/16] quantized SwiGLU outputs (routed, then shared)
  float* hs;         // [T*k + T][f/16]
  float* y;          // [T][d]
};

// Work split of the first kernel: blocks [0, n_rb) hold epb router experts
// each (one per wave), blocks [n_rb, n_rb + n_sb) hold spb consecutive
// shared gate/up steps each; epb and spb are chosen so that every block
// streams about the same number of bytes.
struct K1Plan {
  int n_rb, epb, n_sb, spb, n_steps;
};

}  // namespace dec
}  // namespace qmoe
