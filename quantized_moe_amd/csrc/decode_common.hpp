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
//   * IQ2 weights: the grid row's magnitudes and the stored signs come from
//     two small LDS tables as nibbles u with w = 2u - 7, combined by one XOR
//     (see Iq2Tab).
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
constexpr int G16_BYTES = 32;     // one quantized group of 16 activations (nibble or byte planes)
constexpr int CHUNK_BYTES = 128;  // 64 activations (four groups)
constexpr int DN_ROWS = 16;       // down rows per block of the last kernel

// How the 16 activations of a group are stored (32 bytes), chosen per
// consuming weight format so that weight words need no shuffling:
//   NAT (IQ2): 4-bit digit planes, half hh holds elements 8 hh .. 8 hh + 7,
//              nibble n = element n;
//   Q2K      : 4-bit digit planes, half hh holds the elements of parity hh,
//              nibble n = element 2n + hh (Q2K fields 0/2 and 1/3 of each
//              quant byte);
//   Q8       : two signed byte planes, X = 256 H + L with |X| <= 32512: bytes
//              0..15 are H of elements 0..15, bytes 16..31 their L (each plane
//              meets the int8 weight words directly, 8 dot4 per 16 weights).
enum : int { NIB_NAT = 0, NIB_Q2K = 1, Q8_BYTES = 2 };
constexpr int Q8_XMAX = 32512;  // |X| bound of the byte-plane activations

__host__ __device__ constexpr int nib_layout(int fmt) {
  return fmt == FMT_Q2K ? NIB_Q2K : (fmt == FMT_Q8 || fmt == FMT_MX4 ? Q8_BYTES : NIB_NAT);
}

// A row of K inputs in format FMT: 16-byte pieces, lanes per row, pieces per
// lane, rows per wave step.  Lane (sub, c) with sub = lane / LPR, c = lane %
// LPR reads pieces c + LPR * k (k < CPL) of row sub of the step.
template <int FMT, int K>
struct Geo {
  static constexpr int PW = FMT == FMT_Q8 ? 16 : FMT == FMT_MX4 ? 32 : 64;  // inputs per piece
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
// First link of a chain (zero accumulator): the clamping three-operand form
// takes the zero as an inline constant, where the two-operand form would need
// a register copied from zero.  The clamp never acts: 8 products of 4-bit
// values stay within +-512, 4 products of 8-bit values within +-65536.
__device__ __forceinline__ int dot8_0(uint32_t a, uint32_t b) { return __builtin_amdgcn_sdot8((int)a, (int)b, 0, true); }
__device__ __forceinline__ int dot4_0(uint32_t a, uint32_t b) { return __builtin_amdgcn_sdot4((int)a, (int)b, 0, true); }
// (a << S) + b in one instruction (the compiler splits it into a shift and
// a three-input add)
template <int S>
__device__ __forceinline__ int lshl_add(int a, int b) {
  int r;
  asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "i"(S), "v"(b));
  return r;
}
// sum_p 16^p acc[p]
__device__ __forceinline__ int combine4(const int* acc) {
  return lshl_add<4>(lshl_add<4>(lshl_add<4>(acc[3], acc[2]), acc[1]), acc[0]);
}

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

// Digit planes of 8 values: X_n = rint(v_n inv) (|X| <= XMAX) as four signed
// hex digits, Z = ((X + 0x8888) ^ 0x8888) mod 2^16; returns plane p's word
// (nibble n = digit p of Z_n) in component p.  The fp32 sum v inv + (1.5 2^23
// + 0x8888) is an integer in [2^23, 2^24), rounded as rint rounds, whose bit
// pattern holds X + 0x8888 in its low 16 bits; pairs of values share a word
// and the 4 x 8 nibble transpose is done with masks, shifts and byte
// permutes.
__device__ __forceinline__ uint4 nib_planes8(const float* v, float inv) {
#pragma clang fp contract(off)  // the product is rounded before the shift (rint of the fp32 product)
  uint32_t y[8];
#pragma unroll
  for (int n = 0; n < 8; n++) y[n] = __float_as_uint(v[n] * inv + 12617864.0f);
  uint32_t D[4], E[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const uint32_t A = __builtin_amdgcn_perm(y[2 * k + 1], y[2 * k], 0x05040100u) ^ 0x88888888u;  // Z_2k | Z_2k+1 << 16
    const uint32_t B = A & 0x0f0f0f0fu, C = (A >> 4) & 0x0f0f0f0fu;  // digits 0, 2 / 1, 3 of both, one per byte
    D[k] = B | (B >> 12);  // byte 0: digit 0 of Z_2k, Z_2k+1; byte 1: digit 2
    E[k] = C | (C >> 12);  // byte 0: digit 1; byte 1: digit 3
  }
  auto gather = [](const uint32_t* W, uint32_t b) {  // byte b of W[0..3]
    return __builtin_amdgcn_perm(W[1], W[0], 0x0c0c0400u + 0x0101u * b) |
           __builtin_amdgcn_perm(W[3], W[2], 0x04000c0cu + 0x01010000u * b);
  };
  return make_uint4(gather(D, 0), gather(E, 0), gather(D, 1), gather(E, 1));
}

// Maximum of |v[0..7]| over each aligned unit of GL lanes (GL = 8: a chunk
// of 64 values, GL = 2: a group of 16), returned to every lane of the unit.
template <int GL>
__device__ __forceinline__ float unit_max8(const float* v) {
  float m = 0.0f;
#pragma unroll
  for (int n = 0; n < 8; n++) m = fmaxf(m, fabsf(v[n]));
  if constexpr (GL >= 2) m = fmaxf(m, dpp_f<0x111, 0xf>(m));
  if constexpr (GL >= 4) m = fmaxf(m, dpp_f<0x112, 0xf>(m));
  if constexpr (GL >= 8) m = fmaxf(m, dpp_f<0x114, 0xf>(m));
  return __shfl(m, (int)((threadIdx.x & 63) | (GL - 1)), 64);  // the unit's last lane holds its maximum
}

// Lane-parallel quantization to digit planes: each lane turns 8 values (one
// half of a group of 16, already in the nibble order of the layout) into its
// 4 plane words; GL consecutive lanes share one scale.  Returns the 4 words;
// *scale is the unit's scale.
template <int GL>
__device__ __forceinline__ uint4 quant8(const float* v, float& scale) {
  const float m = unit_max8<GL>(v);
  const float inv = m > 0.0f ? (float)XMAX / m : 0.0f;
  scale = m / (float)XMAX;
  return nib_planes8(v, inv);
}

// Byte planes of 4 values: X_n = rint(v_n inv) (|X| <= 32512) = 256 H + L
// with H = floor((X + 128) / 256) and L in [-128, 127].  The fp32 sum
// v inv + (1.5 2^23 + 128) is an integer in [2^23, 2^24), rounded as rint
// rounds, whose bit pattern holds X + 128 in its low 16 bits: H is byte 1 of
// it and L is byte 0 with the top bit flipped.  H bytes to hw, L bytes to lw.
__device__ __forceinline__ void q8_planes4(const float* v, float inv, uint32_t& hw, uint32_t& lw) {
#pragma clang fp contract(off)  // the product is rounded before the shift (rint of the fp32 product)
  uint32_t y[4];
#pragma unroll
  for (int n = 0; n < 4; n++) y[n] = __float_as_uint(v[n] * inv + 12583040.0f);
  hw = __builtin_amdgcn_perm(y[1], y[0], 0x0c0c0501u) | __builtin_amdgcn_perm(y[3], y[2], 0x05010c0cu);
  lw = (__builtin_amdgcn_perm(y[1], y[0], 0x0c0c0400u) | __builtin_amdgcn_perm(y[3], y[2], 0x04000c0cu)) ^ 0x80808080u;
}

// The same to byte planes (Q8 consumers): 8 values in natural order become
// 8 H bytes and 8 L bytes, X = 256 H + L = rint(v 32512 / m).  Writes H to
// hq[0..8) and L to hq[16..24); *scale is the unit's scale.
template <int GL>
__device__ __forceinline__ void quant8_bytes(const float* v, uint8_t* hq, float& scale) {
  const float m = unit_max8<GL>(v);
  const float inv = m > 0.0f ? (float)Q8_XMAX / m : 0.0f;
  scale = m / (float)Q8_XMAX;
  uint32_t hw[2], lw[2];
  q8_planes4(v, inv, hw[0], lw[0]);
  q8_planes4(v + 4, inv, hw[1], lw[1]);
  if (hq) {
    *reinterpret_cast<uint2*>(hq) = make_uint2(hw[0], hw[1]);
    *reinterpret_cast<uint2*>(hq + 16) = make_uint2(lw[0], lw[1]);
  }
}

// The 8 values of half hh of the group of 16 starting at element e16 of an
// fp32 vector, in the nibble order of `layout`.
__device__ __forceinline__ void load_half_f32(const float* src, int64_t e16, int hh, int layout, float* v) {
  if (layout == NIB_Q2K) {
    float a[16];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float4 f = *reinterpret_cast<const float4*>(src + e16 + 4 * i);
      a[4 * i] = f.x;
      a[4 * i + 1] = f.y;
      a[4 * i + 2] = f.z;
      a[4 * i + 3] = f.w;
    }
#pragma unroll
    for (int n = 0; n < 8; n++) v[n] = hh ? a[2 * n + 1] : a[2 * n];
  } else {
    const float4 f0 = *reinterpret_cast<const float4*>(src + e16 + 8 * hh);
    const float4 f1 = *reinterpret_cast<const float4*>(src + e16 + 8 * hh + 4);
    const float a[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
    for (int n = 0; n < 8; n++) v[n] = a[n];
  }
}

__device__ __forceinline__ void load_half_bf16(const uint16_t* src, int64_t e16, int hh, int layout, float* v) {
  const uint4 b0 = ld16(src + e16), b1 = ld16(src + e16 + 8);
  const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  float a[16];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a[2 * i] = __uint_as_float(bw[i] << 16);
    a[2 * i + 1] = __uint_as_float(bw[i] & 0xffff0000u);
  }
  // every index below is a compile-time constant (hh only selects), so a[]
  // stays in registers
#pragma unroll
  for (int n = 0; n < 8; n++) {
    const float q2k = hh ? a[2 * n + 1] : a[2 * n];
    const float nat = hh ? a[8 + n] : a[n];
    v[n] = layout == NIB_Q2K ? q2k : nat;
  }
}

// Quantize chunks [c0, c0 + 8) of 64 values of x (fp32 or bf16, nch chunks
// in all, x taken as one flat vector) with one wave: lane L takes half L % 8
// of chunk c0 + L / 8.  Chunk ch goes to q + 128 ch (groups of 32 bytes in
// the layout's form), its scale to sc[ch].  load() only issues the loads.
struct XOctet {
  float v[8];
  int ch, hg;
  __device__ __forceinline__ void load(const void* x, int x_dtype, int nch, int c0, int layout) {
    const int lane = threadIdx.x & 63;
    ch = c0 + (lane >> 3);
    hg = lane & 7;
    const int chc = ch < nch ? ch : nch - 1;
    if (x_dtype == X_BF16)
      load_half_bf16(static_cast<const uint16_t*>(x), 64 * (int64_t)chc + 16 * (hg >> 1), hg & 1, layout, v);
    else
      load_half_f32(static_cast<const float*>(x), 64 * (int64_t)chc + 16 * (hg >> 1), hg & 1, layout, v);
  }
  // Digit planes (16 bytes per lane) or, for layout Q8_BYTES, byte planes
  // (8 H bytes and 8 L bytes per lane); one scale per chunk.
  __device__ __forceinline__ void store(int nch, uint8_t* q, float* sc, int layout) const {
    float s;
    uint8_t* g = q + (int64_t)(ch < nch ? ch : 0) * CHUNK_BYTES;
    if (layout == Q8_BYTES) {
      quant8_bytes<8>(v, ch < nch ? g + 32 * (hg >> 1) + 8 * (hg & 1) : nullptr, s);
    } else {
      const uint4 w = quant8<8>(v, s);
      if (ch < nch) *reinterpret_cast<uint4*>(g + 16 * hg) = w;
    }
    if (ch < nch && hg == 0) sc[ch] = s;
  }
};

__device__ __forceinline__ void quant_x8(const void* x, int x_dtype, int nch, int c0, int layout, uint8_t* q,
                                         float* sc) {
  XOctet o;
  o.load(x, x_dtype, nch, c0, layout);
  o.store(nch, q, sc, layout);
}

// Quantize groups [g0, g0 + 32) of 16 fp32 values (ng groups in all) with one
// wave: lane L takes half L % 2 of group g0 + L / 2.
__device__ __forceinline__ void quant_g32(const float* h, int ng, int g0, int layout, uint8_t* q, float* sc) {
  const int lane = threadIdx.x & 63;
  const int g = g0 + (lane >> 1), hh = lane & 1;
  const int gc = g < ng ? g : ng - 1;
  float v[8];
  load_half_f32(h, 16 * (int64_t)gc, hh, layout, v);
  float s;
  uint8_t* p = q + (int64_t)(g < ng ? g : 0) * G16_BYTES;
  if (layout == Q8_BYTES) {
    quant8_bytes<2>(v, g < ng ? p + 8 * hh : nullptr, s);
  } else {
    const uint4 w = quant8<2>(v, s);
    if (g < ng) *reinterpret_cast<uint4*>(p + 16 * hh) = w;
  }
  if (g < ng && hh == 0) sc[g] = s;
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
  // pieces c + LPR k quantized here from fp32 h (one scale per group of 16,
  // the same digits and scales as quant_g32 gives), digits in `layout`:
  // fetch_f32 only loads, so the caller can request other data before
  // quant_f32 waits for it
  template <int LPR>
  static __device__ __forceinline__ void fetch_f32(const float* h, int c, float (&raw)[CPL][64]) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int pc = c + LPR * k;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const float4 f = *reinterpret_cast<const float4*>(h + 64 * pc + 4 * j);
        raw[k][4 * j] = f.x;
        raw[k][4 * j + 1] = f.y;
        raw[k][4 * j + 2] = f.z;
        raw[k][4 * j + 3] = f.w;
      }
    }
  }
  __device__ __forceinline__ void quant_f32(const float (&raw)[CPL][64], int layout) {
    static_assert(PER16, "lane-local quantization is group-scaled");
#pragma unroll
    for (int k = 0; k < CPL; k++)
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const float* v = raw[k] + 16 * u;
        float m = 0.0f;
#pragma unroll
        for (int n = 0; n < 16; n++) m = fmaxf(m, fabsf(v[n]));
        const float inv = m > 0.0f ? (float)XMAX / m : 0.0f;
        s[k][u] = m / (float)XMAX;
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          float vh[8];
#pragma unroll
          for (int n = 0; n < 8; n++) vh[n] = layout == NIB_Q2K ? v[2 * n + hh] : v[8 * hh + n];
          const uint4 pw = nib_planes8(vh, inv);
          w[k][u][hh][0] = pw.x;
          w[k][u][hh][1] = pw.y;
          w[k][u][hh][2] = pw.z;
          w[k][u][hh][3] = pw.w;
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
        for (int p = 0; p < 4; p++) acc[p] = dot8(w[k][u][1][p], 0x11111111u, dot8_0(w[k][u][0][p], 0x11111111u));
        Ai[k][u] = combine4(acc);
        if constexpr (PER16) As[k][u] = s[k][u] * (float)Ai[k][u];
      }
  }
};

// Q8 pieces (16 inputs = one group) as two signed byte planes H, L with
// X = 256 H + L (layout Q8_BYTES), one scale per piece.
template <int CPL>
struct ActQ8B {
  uint32_t H[CPL][4], L[CPL][4];
  float s[CPL];
  // pieces c + LPR k of groups at q; GSCALE: 16 for group-quantized h
  // (scale per piece), 64 for chunk-quantized x (scale per four pieces)
  template <int LPR, int GSCALE>
  __device__ __forceinline__ void load(const uint8_t* q, const float* sc, int c) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int pc = c + LPR * k;
      const uint4 hv = ld16(q + (int64_t)pc * G16_BYTES);
      const uint4 lv = ld16(q + (int64_t)pc * G16_BYTES + 16);
      H[k][0] = hv.x;
      H[k][1] = hv.y;
      H[k][2] = hv.z;
      H[k][3] = hv.w;
      L[k][0] = lv.x;
      L[k][1] = lv.y;
      L[k][2] = lv.z;
      L[k][3] = lv.w;
      s[k] = sc[GSCALE == 16 ? pc : pc / 4];
    }
  }
  // pieces c + LPR k quantized here from fp32 h (one scale per piece, the
  // same bytes and scales as quant_g32 gives): fetch_f32 only loads, so the
  // caller can request other data before quant_f32 waits for it
  template <int LPR>
  static __device__ __forceinline__ void fetch_f32(const float* h, int c, float (&raw)[CPL][16]) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int pc = c + LPR * k;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float4 f = *reinterpret_cast<const float4*>(h + 16 * pc + 4 * j);
        raw[k][4 * j] = f.x;
        raw[k][4 * j + 1] = f.y;
        raw[k][4 * j + 2] = f.z;
        raw[k][4 * j + 3] = f.w;
      }
    }
  }
  __device__ __forceinline__ void quant_f32(const float (&raw)[CPL][16]) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      float m = 0.0f;
#pragma unroll
      for (int n = 0; n < 16; n++) m = fmaxf(m, fabsf(raw[k][n]));
      const float inv = m > 0.0f ? (float)Q8_XMAX / m : 0.0f;
      s[k] = m / (float)Q8_XMAX;
#pragma unroll
      for (int wd = 0; wd < 4; wd++) q8_planes4(raw[k] + 4 * wd, inv, H[k][wd], L[k][wd]);
    }
  }
};

// MXFP4 pieces (32 inputs = two groups of 16) as the two signed byte planes
// H, L of each group (layout Q8_BYTES, natural order), one scale per group
// (group-quantized h) or per 64-input chunk (x).
template <int CPL>
struct ActMx4 {
  uint32_t H[CPL][8], L[CPL][8];
  float s[CPL][2];
  // pieces c + LPR k of groups at q; GSCALE: 16 for group-quantized h, 64
  // for chunk-quantized x
  template <int LPR, int GSCALE>
  __device__ __forceinline__ void load(const uint8_t* q, const float* sc, int c) {
#pragma unroll
    for (int k = 0; k < CPL; k++) {
      const int g0 = 2 * (c + LPR * k);
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const uint4 hv = ld16(q + (int64_t)(g0 + j) * G16_BYTES);
        const uint4 lv = ld16(q + (int64_t)(g0 + j) * G16_BYTES + 16);
        H[k][4 * j] = hv.x;
        H[k][4 * j + 1] = hv.y;
        H[k][4 * j + 2] = hv.z;
        H[k][4 * j + 3] = hv.w;
        L[k][4 * j] = lv.x;
        L[k][4 * j + 1] = lv.y;
        L[k][4 * j + 2] = lv.z;
        L[k][4 * j + 3] = lv.w;
        s[k][j] = sc[GSCALE == 16 ? g0 + j : (g0 + j) / 4];
      }
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

// A or B, chosen field by field (a select of values, never of addresses, so
// that the planes stay in registers).
__device__ __forceinline__ EPlanes pick_planes(bool second, const EPlanes& A, const EPlanes& B) {
  // (the fields are read into values first: a conditional of two lvalues is
  // itself an lvalue, i.e. a select of their addresses)
  const uint8_t *as = A.scale, *aa = A.a, *ab = A.b;
  const uint8_t *bs = B.scale, *ba = B.a, *bb = B.b;
  EPlanes p;
  p.scale = second ? bs : as;
  p.a = second ? ba : aa;
  p.b = second ? bb : ab;
  return p;
}

// Expert e's planes of a tensor whose format is a compile-time FMT.
template <int FMT>
__device__ __forceinline__ EPlanes expert_planes(const QMat& m, int e) {
  const int64_t r = (int64_t)e * m.rows * m.nb;  // blocks before this expert
  EPlanes p;
  if constexpr (FMT == FMT_IQ2) {
    p.scale = m.p_scale + r * 2;
    p.a = m.p_a + r * 64;
    p.b = nullptr;
  } else if constexpr (FMT == FMT_Q2K) {
    p.scale = m.p_scale + r * 4;
    p.a = m.p_a + r * 16;
    p.b = m.p_b + r * 64;
  } else if constexpr (FMT == FMT_Q4K) {
    p.scale = m.p_scale + r * 4;
    p.a = m.p_a + r * 12;
    p.b = m.p_b + r * 128;
  } else if constexpr (FMT == FMT_MX4) {
    p.scale = m.p_scale + r;
    p.a = m.p_a + r * 16;
    p.b = nullptr;
  } else {
    p.scale = m.p_scale + r * 2;
    p.a = m.p_a + r * 32;
    p.b = nullptr;
  }
  return p;
}

// A piece: one lane's 16 bytes of codes of one row, plus the scales that
// belong to them.  load() reads the codes; the scales come either straight
// from their planes (scales_global) or from a copy of the rows' scale bytes
// that the wave staged in LDS (scales_lds; see ScaleStage).
template <int FMT>
struct Piece;

template <>
struct Piece<FMT_IQ2> {  // words A0 B0 A1 B1 of sub-blocks 2 (pc % 4), +1 of superblock pc / 4
  uint4 v;
  uint32_t d;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t pc) {
    v = ld16_stream(p.a + (row * NB * 64 + pc * 16));
  }
  template <int NB>
  __device__ __forceinline__ void scales_global(const EPlanes& p, uint32_t row, uint32_t pc) {
    d = reinterpret_cast<const uint16_t*>(p.scale)[row * NB + pc / 4];
  }
  template <int NB>
  __device__ __forceinline__ void scales_lds(const uint8_t* rp, uint32_t pc) {
    d = reinterpret_cast<const uint16_t*>(rp)[pc / 4];
  }
};

template <>
struct Piece<FMT_Q2K> {  // quants of sub-blocks 4 (pc % 4) .. +3 of superblock pc / 4
  uint4 q;
  uint32_t sc, dm;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t pc) {
    q = ld16_stream(p.b + (row * NB * 64 + pc * 16));
  }
  template <int NB>
  __device__ __forceinline__ void scales_global(const EPlanes& p, uint32_t row, uint32_t pc) {
    sc = *reinterpret_cast<const uint32_t*>(p.a + (row * NB * 16 + pc * 4));
    dm = reinterpret_cast<const uint32_t*>(p.scale)[row * NB + pc / 4];
  }
  template <int NB>
  __device__ __forceinline__ void scales_lds(const uint8_t* rp, uint32_t pc) {  // row: dm[NB] then sc[NB][16]
    dm = reinterpret_cast<const uint32_t*>(rp)[pc / 4];
    sc = reinterpret_cast<const uint32_t*>(rp + NB * 4)[pc];
  }
};

// Q4K: a piece is 64 inputs, the quants of sub-blocks 2 (pc % 4) and
// 2 (pc % 4) + 1 of superblock pc / 4 (32 bytes, two 16-byte loads);
// lo holds their two low-bit scale bytes, hi their top-bit byte.
template <>
struct Piece<FMT_Q4K> {
  uint4 q0, q1;
  uint32_t lo, hi, dm;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t pc) {
    const uint8_t* b = p.b + (row * NB * 128 + pc * 32);
    q0 = ld16_stream(b);
    q1 = ld16_stream(b + 16);
  }
  __device__ __forceinline__ void scale_bytes(const uint8_t* sb, uint32_t pc) {  // sb: the superblock's 12 bytes
    lo = *reinterpret_cast<const uint16_t*>(sb + 2 * (pc % 4));
    hi = sb[8 + pc % 4];
  }
  template <int NB>
  __device__ __forceinline__ void scales_global(const EPlanes& p, uint32_t row, uint32_t pc) {
    scale_bytes(p.a + (row * NB + pc / 4) * 12, pc);
    dm = reinterpret_cast<const uint32_t*>(p.scale)[row * NB + pc / 4];
  }
  template <int NB>
  __device__ __forceinline__ void scales_lds(const uint8_t* rp, uint32_t pc) {  // row: dm[NB] then sc[NB][12]
    dm = reinterpret_cast<const uint32_t*>(rp)[pc / 4];
    scale_bytes(rp + NB * 4 + (pc / 4) * 12, pc);
  }
};

template <>
struct Piece<FMT_Q8> {  // 16 int8 quants: half of block pc / 2
  uint4 q;
  uint32_t d;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t pc) {
    q = ld16_stream(p.a + (row * NB * 32 + pc * 16));
  }
  template <int NB>
  __device__ __forceinline__ void scales_global(const EPlanes& p, uint32_t row, uint32_t pc) {
    d = reinterpret_cast<const uint16_t*>(p.scale)[row * NB + pc / 2];
  }
  template <int NB>
  __device__ __forceinline__ void scales_lds(const uint8_t* rp, uint32_t pc) {
    d = reinterpret_cast<const uint16_t*>(rp)[pc / 2];
  }
};

// MXFP4: a piece is one block, 32 E2M1 codes (two per byte, the even weight
// in the low nibble), with its E8M0 scale byte.
template <>
struct Piece<FMT_MX4> {
  uint4 q;
  uint32_t e;
  template <int NB>
  __device__ __forceinline__ void load(const EPlanes& p, uint32_t row, uint32_t pc) {
    q = ld16_stream(p.a + (row * NB + pc) * 16);
  }
  template <int NB>
  __device__ __forceinline__ void scales_global(const EPlanes& p, uint32_t row, uint32_t pc) {
    e = p.scale[row * NB + pc];
  }
  template <int NB>
  __device__ __forceinline__ void scales_lds(const uint8_t* rp, uint32_t pc) {
    e = rp[pc];
  }
};

// Scale bytes of one row in format FMT with K inputs, as staged in LDS.
template <int FMT, int K>
struct RowScales {
  static constexpr int NB = K / block_weights(FMT);
  static constexpr bool KQ = FMT == FMT_Q2K || FMT == FMT_Q4K;
  static constexpr int DM = KQ ? NB * 4 : 0;                                  // K-quant (d, dmin) pairs
  static constexpr int BYTES = KQ ? NB * (4 + kq_scale_bytes(FMT)) : NB * (FMT == FMT_MX4 ? 1 : 2);  // + sub-block scales
  static constexpr bool STAGE = (BYTES % 16) == 0 && (DM % 16) == 0;    // whole 16-byte chunks
};

// The scale bytes of NM matrices x NR rows, copied by one wave into its LDS
// area (row (m, j) at m * NR + j, RowScales::BYTES each) with one 16-byte
// load per lane per 64 chunks.  issue() only loads (so these loads can be
// put ahead of the code loads, which then return after them); store()
// writes LDS.  Each lane maps its chunks to (row, plane) itself, so rows may
// belong to different experts.
template <int FMT, int K, int NM, int NR>
struct ScaleStage {
  using RS = RowScales<FMT, K>;
  static constexpr int CPR = RS::BYTES >= 16 ? RS::BYTES / 16 : 1;  // chunks per row (only staged rows use it)
  static constexpr int CH = NM * NR * CPR;
  static constexpr int NV = (CH + 63) / 64;
  uint4 v[NV];
  // rowsrc(m, j, planes, row) gives the expert planes and row index of (m, j)
  template <class RowSrc>
  __device__ __forceinline__ void issue(RowSrc rowsrc) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NV; i++) {
      int q = lane + 64 * i;
      q = q < CH ? q : CH - 1;
      const int r = q / CPR, cq = q % CPR;
      const int m = r / NR, j = r % NR;
      EPlanes P;
      uint32_t row;
      rowsrc(m, j, P, row);
      const uint8_t* src;
      if constexpr (RS::KQ) {
        src = cq * 16 < RS::DM ? P.scale + row * RS::DM + cq * 16
                               : P.a + row * (RS::NB * kq_scale_bytes(FMT)) + (cq * 16 - RS::DM);
      } else {
        src = P.scale + row * RS::BYTES + cq * 16;
      }
      v[i] = ld16(src);
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NV; i++)
      if (lane + 64 * i < CH) *reinterpret_cast<uint4*>(lds + 16 * (lane + 64 * i)) = v[i];
  }
  static __device__ __forceinline__ const uint8_t* row(const uint8_t* lds, int m, int j) {
    return lds + (m * NR + j) * RS::BYTES;
  }
};

// ---------------------------------------------------------------------------
// IQ2 tables.  A grid magnitude m (odd, 1..7) becomes the nibble u = (m + 7)
// / 2, so +m is u and -m is 7 - u = u ^ 7: pos[row] holds the 8 magnitudes
// of a grid row as such nibbles (element n in nibble n), neg[b] holds 0x7 in
// every nibble whose sign is negative for the 7 stored sign bits b (parity
// sign included).  A group's weights are w_n = 2 u_n - 7 with
// u = pos[row] ^ neg[b]: one XOR of two small-table words per 8 weights, and
// sum w x = 2 sum u x - 7 sum x.  1.5 KB of LDS.
// ---------------------------------------------------------------------------
struct Iq2Tab {
  uint32_t pos[256];
  uint32_t neg[128];
};

// Items 0..383 (grid row i < 256, sign pattern i - 256), one per thread
// `item`; the caller publishes the table with a barrier.
__device__ __forceinline__ void iq2_build(const uint8_t* __restrict__ grid, int item, Iq2Tab* t) {
  if (item >= 0 && item < 256) {
    const uint2 g = reinterpret_cast<const uint2*>(grid)[item];
    uint32_t w = 0;
#pragma unroll
    for (int n = 0; n < 8; n++) {
      const uint32_t m = ((n < 4 ? g.x : g.y) >> (8 * (n & 3))) & 255u;
      w |= (((m + 7u) >> 1) & 15u) << (4 * n);
    }
    t->pos[item] = w;
  } else if (item >= 256 && item < 384) {
    const uint32_t b = item - 256;
    const uint32_t s8 = b | ((__popc(b) & 1u) << 7);
    uint32_t mk = 0;
#pragma unroll
    for (int n = 0; n < 8; n++) mk |= ((s8 >> n) & 1u) ? (0x7u << (4 * n)) : 0u;
    t->neg[b] = mk;
  }
}

// ---------------------------------------------------------------------------
// dot products of one weight piece with the matching activation slice k;
// each returns the piece's contribution in real units
// ---------------------------------------------------------------------------
template <int CPL, bool PER16>
__device__ __forceinline__ float piece_dot(const Piece<FMT_IQ2>& w, const ActNib<CPL, PER16>& a, int k,
                                           const Iq2Tab* tab) {
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
      const uint32_t u = tab->pos[(A >> (8 * i)) & 255u] ^ tab->neg[(B >> (7 * i)) & 127u];
      const int q = 2 * h + (i >> 1), hh = i & 1, slot = PER16 ? (i >> 1) : 0;
#pragma unroll
      for (int p = 0; p < 4; p++)
        acc[slot][p] = (i == 0 || (PER16 && i == 2)) ? dot8_0(u, a.w[k][q][hh][p]) : dot8(u, a.w[k][q][hh][p], acc[slot][p]);
    }
    // sum w x = 2 sum u x - 7 sum x over each group of 16; |2 u - 7| <= 7
    // and |X| <= 0x7777 keep a half's sum within 24 bits
    if constexpr (PER16) {
      ftot += (float)__mul24(lshl_add<1>(combine4(acc[0]), -7 * a.Ai[k][2 * h]), mul) * a.s[k][2 * h] +
              (float)__mul24(lshl_add<1>(combine4(acc[1]), -7 * a.Ai[k][2 * h + 1]), mul) * a.s[k][2 * h + 1];
    } else {
      itot += __mul24(lshl_add<1>(combine4(acc[0]), -7 * (a.Ai[k][2 * h] + a.Ai[k][2 * h + 1])), mul);
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
                                           const Iq2Tab*) {
  const uint32_t W[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
  int im = 0, in = 0;
  float fm = 0.0f, fn = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const uint32_t N0 = W[u] & 0x33333333u, N1 = (W[u] >> 2) & 0x33333333u;
    int acc[4];
#pragma unroll
    for (int p = 0; p < 4; p++) acc[p] = dot8(N1, a.w[k][u][1][p], dot8_0(N0, a.w[k][u][0][p]));
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

// Q4K: the 4-bit quants q meet the signed digit planes as q - 8 (q ^ 8 read
// as a signed nibble); sum q x = sum (q - 8) x + 8 sum x.  A group's sum
// stays within 15 * 0x7777 * 16 < 2^23, so the 6-bit scale multiplies with
// a 24-bit integer multiply.
template <int CPL, bool PER16>
__device__ __forceinline__ float piece_dot(const Piece<FMT_Q4K>& w, const ActNib<CPL, PER16>& a, int k,
                                           const Iq2Tab*) {
  const uint32_t W[8] = {w.q0.x, w.q0.y, w.q0.z, w.q0.w, w.q1.x, w.q1.y, w.q1.z, w.q1.w};
  int im = 0, in = 0;
  float fm = 0.0f, fn = 0.0f;
#pragma unroll
  for (int sb = 0; sb < 2; sb++) {
    const int sc = (int)(((w.lo >> (8 * sb)) & 15u) | (((w.hi >> (4 * sb)) & 3u) << 4));
    const int m = (int)(((w.lo >> (8 * sb + 4)) & 15u) | (((w.hi >> (4 * sb + 2)) & 3u) << 4));
#pragma unroll
    for (int g = 0; g < 2; g++) {
      const int u = 2 * sb + g;
      const uint32_t N0 = W[2 * u] ^ 0x88888888u, N1 = W[2 * u + 1] ^ 0x88888888u;
      int acc[4];
#pragma unroll
      for (int p = 0; p < 4; p++) acc[p] = dot8(N1, a.w[k][u][1][p], dot8_0(N0, a.w[k][u][0][p]));
      const int D = lshl_add<3>(a.Ai[k][u], combine4(acc));
      if constexpr (PER16) {
        fm += (float)__mul24(sc, D) * a.s[k][u];
        fn += (float)m * a.As[k][u];
      } else {
        im += __mul24(sc, D);
        in += m * a.Ai[k][u];
      }
    }
  }
  const float d = half_bits_to_float(w.dm & 0xffffu), dmin = half_bits_to_float(w.dm >> 16);
  if constexpr (PER16)
    return fm * d - fn * dmin;
  else
    return a.s[k][0] * ((float)im * d - (float)in * dmin);
}

// Four E2M1 codes (one per byte, 0..15) -> four int8 values 2 w (exact
// integers: 0, 1, 2, 3, 4, 6, 8, 12 with the sign of bit 3).  Two byte
// permutes look the magnitude up in the positive and in the negative table
// (bytes 0..3 of the second operand, 4..7 of the first); a bitfield select
// keeps the negative entry where bit 3 is set.
__device__ __forceinline__ uint32_t mx4_bytes(uint32_t n) {
  const uint32_t m = n & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x0c080604u, 0x03020100u, m);
  const uint32_t neg = __builtin_amdgcn_perm(0xf4f8fafcu, 0xfdfeff00u, m);
  const uint32_t sgn = ((n >> 3) & 0x01010101u) * 0xffu;
  return (neg & sgn) | (pos & ~sgn);
}

// MXFP4 piece: sum 2w H and 2w L over each group of 16 (exact integers:
// |2w| <= 12, |H| <= 127, |L| <= 128), X = 256 H + L, times the group's
// scale and 2^(e - 128) (the block scale 2^(e - 127) over the factor 2).
template <int CPL>
__device__ __forceinline__ float piece_dot(const Piece<FMT_MX4>& w, const ActMx4<CPL>& a, int k, const Iq2Tab*) {
  const uint32_t W[4] = {w.q.x, w.q.y, w.q.z, w.q.w};
  int hs[2], ls[2];
#pragma unroll
  for (int i = 0; i < 4; i++) {  // word i: weights 8i .. 8i + 7 (group i / 2)
    const uint32_t lo = W[i] & 0x0f0f0f0fu, hi = (W[i] >> 4) & 0x0f0f0f0fu;
    const uint32_t b0 = mx4_bytes(__builtin_amdgcn_perm(hi, lo, 0x05010400u));  // weights 8i .. 8i + 3
    const uint32_t b1 = mx4_bytes(__builtin_amdgcn_perm(hi, lo, 0x07030602u));  // 8i + 4 .. 8i + 7
    const int g = i >> 1, j = 4 * g + 2 * (i & 1);
    if ((i & 1) == 0) {
      hs[g] = dot4(b1, a.H[k][j + 1], dot4_0(b0, a.H[k][j]));
      ls[g] = dot4(b1, a.L[k][j + 1], dot4_0(b0, a.L[k][j]));
    } else {
      hs[g] = dot4(b1, a.H[k][j + 1], dot4(b0, a.H[k][j], hs[g]));
      ls[g] = dot4(b1, a.L[k][j + 1], dot4(b0, a.L[k][j], ls[g]));
    }
  }
  const float v = (float)(hs[0] * 256 + ls[0]) * a.s[k][0] + (float)(hs[1] * 256 + ls[1]) * a.s[k][1];
  return __builtin_amdgcn_ldexpf(v, (int)w.e - 128);
}

template <int CPL>
__device__ __forceinline__ float piece_dot(const Piece<FMT_Q8>& w, const ActQ8B<CPL>& a, int k, const Iq2Tab*) {
  const int h = dot4(w.q.w, a.H[k][3], dot4(w.q.z, a.H[k][2], dot4(w.q.y, a.H[k][1], dot4_0(w.q.x, a.H[k][0]))));
  const int l = dot4(w.q.w, a.L[k][3], dot4(w.q.z, a.L[k][2], dot4(w.q.y, a.L[k][1], dot4_0(w.q.x, a.L[k][0]))));
  return (float)(h * 256 + l) * (a.s[k] * half_bits_to_float(w.d));
}

// ---------------------------------------------------------------------------
// arguments of the three kernels
// ---------------------------------------------------------------------------
struct DecodeArgs {
  QMat gate, up, down;        // routed experts
  QMat s_gate, s_up, s_down;  // shared expert
  const uint8_t* grid;
  const uint8_t* vq_cb;       // E4M3 codewords [n][8] (VQ routed formats)
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
  uint8_t* xq;       // [T][d/64] x in chunks (layout of the routed gate/up format), from the first launch
  float* xs;         // [T][d/64]
  uint8_t* xq_s;     // [T][d/64] x in the shared gate/up format's layout (when shared_k2)
  float* xs_s;       // [T][d/64]
  int shared_k2;     // the shared gate/up runs in the second launch (one token), not the first
  int xs_global;     // (several tokens) the first launch also quantizes x into xq_s / xs_s, which the
                     // shared gate/up blocks then copy instead of quantizing x themselves
  const float* router_bias;  // nullable [E]: selection on sigmoid32(z) + bias
  float* zkey;               // [T][E] the selection keys (fused routing with a bias), from the first launch
  const float* down_gain;    // nullable [E][d]: per-channel gains of the routed outputs
  float* hsh;        // [T][f] shared SwiGLU output, fp32
  uint8_t* hq;       // [T*k][f/16] quantized routed SwiGLU outputs
  float* hs;         // [T*k][f/16]
  float* hf;         // [T*k][f] routed SwiGLU outputs in fp32 (VQ routed formats)
  int* plan;         // several tokens: distinct experts and their routes (decode_unique.hip)
  int umax;          // the plan's capacity in distinct experts, min(E, T k)
  float* y;          // [T][d]
};

// Up to 2048 inputs per row and a Q8 shared expert: 16 waves, a routed
// expert's 16 rows as two tasks of 8 and the shared expert's as four tasks
// of 4 (16 tasks for k = 6, four per SIMD); longer rows, or a 2-bit shared
// expert (whose h slice is quantized from 64 fp32 values per piece), need
// more registers per wave: 8 waves, one task per routed expert and two for
// the shared expert.
// (Q4K routed rows, with twice the code registers per piece, and VQ rows,
// whose h slice is 64 fp32 values per piece, take 8 waves.)
constexpr int k3_waves(int FR, int FS, int F) {
  return F <= 2048 && FS == FMT_Q8 && FR != FMT_Q4K && !is_vq(FR) ? 16 : 8;
}

// Work split of the first kernel: blocks [0, n_rb) hold epb (< 8) router
// experts each (one per wave; the last wave quantizes x for the routed
// gate/up), blocks [n_rb, n_rb + n_sb) hold spb consecutive shared gate/up
// steps each; epb and spb are chosen so that every block streams about the
// same number of bytes.
struct K1Plan {
  int n_rb, epb, n_sb, spb, n_steps;
  int n_xb;  // blocks that only quantize x (one octet of chunks per wave), when no router runs
};

}  // namespace dec
}  // namespace qmoe
