// VQ rows on the GPU (MOE_FMT_VQ12_L / VQ13_L): codeword indices and
// codewords.
//
// "YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 4.1: each 8
// consecutive weights of a row are one codeword of a per-layer codebook of
// E4M3 vectors, times one gain per row.  The kernels take a row in pieces of
// 8 indices = 64 inputs: 12 bytes of the index stream (three dwords, always
// 4-byte aligned) and, for 13-bit rows, one byte of the bit plane.  The
// codebook sits in LDS as E4M3 bytes (8 per codeword: 32 KB for 4096, 64 KB
// for 8192 codewords) and the hardware conversions turn a codeword into fp32
// (decode) or fp16 (prefill MFMA operands) exactly; the same section insists
// on the hardware conversion rather than a software decoder.
#pragma once

#include "common.hpp"

namespace qmoe {

typedef float vq_f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 vq_f16x2 __attribute__((ext_vector_type(2)));

// One piece of a row: the three stream dwords and (13 bits) the plane byte.
struct VqPiece {
  uint32_t w0, w1, w2, pl;
};

// Index q (0..7, a compile-time constant after unrolling) of a piece: stream
// bits 12q .. 12q + 11 of the 96 held in w0..w2, and bit q of the plane byte
// as bit 12 for 13-bit rows.
template <bool B13>
__device__ __forceinline__ uint32_t vq_index(const VqPiece& p, int q) {
  uint32_t v;
  switch (q) {
    case 0: v = p.w0; break;
    case 1: v = p.w0 >> 12; break;
    case 2: v = __builtin_amdgcn_alignbit(p.w1, p.w0, 24); break;
    case 3: v = p.w1 >> 4; break;
    case 4: v = p.w1 >> 16; break;
    case 5: v = __builtin_amdgcn_alignbit(p.w2, p.w1, 28); break;
    case 6: v = p.w2 >> 8; break;
    default: v = p.w2 >> 20; break;
  }
  v &= 0xfffu;
  if constexpr (B13) v |= ((p.pl >> q) & 1u) << 12;
  return v;
}

// Piece `piece` of row `row` of a VQ matrix in the device layout (stream
// plane at s, bit plane at b, K inputs per row).
template <bool B13>
__device__ __forceinline__ VqPiece vq_load_piece(const uint8_t* s, const uint8_t* b, int64_t row, int K, int piece) {
  VqPiece p;
  const uint3 v = *reinterpret_cast<const uint3*>(s + row * (3 * K / 16) + 12 * piece);
  p.w0 = v.x;
  p.w1 = v.y;
  p.w2 = v.z;
  p.pl = B13 ? (uint32_t)b[row * (K / 64) + piece] : 0u;
  return p;
}

// Codeword idx from the LDS codebook: 8 E4M3 bytes.
__device__ __forceinline__ uint2 vq_codeword(const uint8_t* cb, uint32_t idx) {
  return *reinterpret_cast<const uint2*>(cb + idx * 8u);
}

// fp32 values of the 8 E4M3 bytes of a codeword (exact).
__device__ __forceinline__ void vq_to_f32(uint2 c, float* v) {
  const vq_f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(c.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(c.x, true);
  const vq_f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(c.y, false), e = __builtin_amdgcn_cvt_pk_f32_fp8(c.y, true);
  v[0] = a[0];
  v[1] = a[1];
  v[2] = b[0];
  v[3] = b[1];
  v[4] = d[0];
  v[5] = d[1];
  v[6] = e[0];
  v[7] = e[1];
}

// The same as four packed fp16 pairs (an MFMA B fragment; exact: every E4M3
// value is an fp16).
__device__ __forceinline__ uint4 vq_to_f16(uint2 c) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.0f, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.0f, true)));
}

// Copy the first n_codes codewords of the codebook into LDS (every thread of
// the block takes a share of 16-byte pieces).
__device__ __forceinline__ void vq_stage_codebook(const uint8_t* __restrict__ cb, uint8_t* lds, int n_codes, int tid,
                                                  int nthreads) {
  const uint4* src = reinterpret_cast<const uint4*>(cb);
  uint4* dst = reinterpret_cast<uint4*>(lds);
  for (int i = tid; i < n_codes / 2; i += nthreads) dst[i] = src[i];
}

}  // namespace qmoe
