// fp16 MFMA helpers and the IQ2 codebook tables of the prefill grouped GEMMs.
//
// "YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 4.4 feeds 16-bit
// matrix units with codewords that convert without rounding.  Here every IQ2
// B-operand value handed to v_mfma is the exact integer (2s+1) * g (s the
// 4-bit sub-block scale, g in {1,3,5,7} the grid magnitude, so <= 217) with
// its sign, in fp16; the fp16 superblock scale is applied to the fp32 result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int TAB_COPIES = 16;  // magnitude-table copies (one per lane of a 16-lane row)

__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0,
                                               0, 0);
}

// fp32 -> fp16 bits (round to nearest even) and back
__device__ __forceinline__ uint32_t to_h(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ __forceinline__ float from_h(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }

// IQ2 tables in LDS.  tm[row][c] = the 8 grid magnitudes of row as fp16, 16
// bytes, stored TAB_COPIES times (copy c at bank quad c, row stride 256
// bytes): the byte address row << 8 | c << 4 is one v_perm of the payload
// word and c << 4.  sgn[b7][c] = XOR masks of the 7 stored signs plus the
// parity sign, stored SGN copies times (16 or 8; row stride 16 SGN bytes).
// Lane l reads copy l % 16 of the magnitudes and copy l % SGN of the signs,
// so the 16 lanes of a row never meet in a bank on a magnitude read whatever
// rows they look up (a table indexed by the sub-block scale as well put every
// lane with the same scale on the same banks), nor on a sign read with 16
// copies (with 8, which 64-row M tiles take to fit the LDS, at most two
// meet).  The scale (2s+1) is one packed fp16 multiply per word:
// (2s+1) * g <= 217 is exact.
constexpr int IQ2_TM_BYTES = 256 * TAB_COPIES * 16;
template <int SGN>
constexpr int iq2_sgn_bytes() { return 128 * SGN * 16; }

// Both tables, built by threads t0 .. t0 + nt - 1 of the block: a thread
// that owns a grid row reads it once and writes its copies; the sign table
// needs no loads and is spread over all of them.
template <int SGN>
__device__ inline void build_iq2_tables(const uint8_t* grid, uint4* tm, uint4* sgn, int t0, int nt) {
  static_assert(SGN == 8 || SGN == 16, "sign-table copies");
  for (int row = t0; row < 256; row += nt) {
    const uint2 g = *reinterpret_cast<const uint2*>(grid + 8 * row);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t word = i < 2 ? g.x : g.y;
      const uint32_t v0 = (word >> (16 * (i & 1))) & 255u, v1 = (word >> (16 * (i & 1) + 8)) & 255u;
      w[i] = to_h((float)v0) | (to_h((float)v1) << 16);
    }
#pragma unroll 4
    for (int c = 0; c < TAB_COPIES; c++) tm[row * TAB_COPIES + c] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  for (int e = t0; e < 128 * SGN; e += nt) {
    const uint32_t b = e / SGN;
    const uint32_t s8 = b | ((__popc(b) & 1u) << 7);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) w[i] = (((s8 >> (2 * i)) & 1u) << 15) | (((s8 >> (2 * i + 1)) & 1u) << 31);
    sgn[e] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// IQ2 sub-block scale (2s+1) (s the top nibble of its B word) as a packed
// pair of fp16
__device__ __forceinline__ uint32_t iq2_scale_h2(uint32_t bword) {
  const uint32_t h = to_h((float)(2u * (bword >> 28) + 1u));
  return h | (h << 16);
}

// The 8 exact integers of group i (0..3) of a sub-block with payload words
// (A, B): SC = iq2_scale_h2(B), CB = (lane % 16) << 4, CS = (lane % SGN) << 4.
template <int SGN>
__device__ __forceinline__ uint4 iq2_frag_words(uint32_t A, uint32_t B, int i, uint32_t SC, uint32_t CB,
                                                uint32_t CS, const uint8_t* tm, const uint8_t* sgn) {
  // row << 8 | copy << 4: byte 0 from CB, byte 1 = byte i of A
  const uint32_t maddr = __builtin_amdgcn_perm(A, CB, 0x0c0c0000u | ((4u + i) << 8));
  // (7 sign bits) << 8 | copy << 4 (16 copies), or << 7 (8 copies)
  uint32_t saddr;
  if constexpr (SGN == 16) {
    const uint32_t sh = i == 0 ? (B << 8) : i == 1 ? (B << 1) : i == 2 ? (B >> 6) : (B >> 13);
    saddr = (sh & 0x7f00u) | CS;
  } else {
    const uint32_t sh = i == 0 ? (B << 7) : i == 1 ? B : i == 2 ? (B >> 7) : (B >> 14);
    saddr = (sh & 0x3f80u) | CS;
  }
  const uint4 m = *reinterpret_cast<const uint4*>(tm + maddr);
  const uint4 s = *reinterpret_cast<const uint4*>(sgn + saddr);
  const f16x2_t sc = __builtin_bit_cast(f16x2_t, SC);
  auto word = [&](uint32_t mw, uint32_t sw) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, mw ^ sw) * sc);
  };
  return make_uint4(word(m.x, s.x), word(m.y, s.y), word(m.z, s.z), word(m.w, s.w));
}

}  // namespace qmoe
