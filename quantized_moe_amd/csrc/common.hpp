// Internal definitions shared by the HIP kernels and the host API of libqmoe.
// (Not shared with the CPU oracle, which restates everything independently.)
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmoe {

enum : int { X_F32 = 0, X_BF16 = 1 };
enum : int { FMT_IQ2 = 1, FMT_Q2K = 2, FMT_Q8 = 3, FMT_Q4K = 4, FMT_MX4 = 5, FMT_VQ12 = 6, FMT_VQ13 = 7 };

// VQ rows: one 12- or 13-bit codeword index per 8 inputs and an fp16 gain per
// row (no blocks); codewords are 8 E4M3 bytes of a per-layer codebook.
__host__ __device__ constexpr bool is_vq(int fmt) { return fmt == FMT_VQ12 || fmt == FMT_VQ13; }
__host__ __device__ constexpr int vq_bits(int fmt) { return fmt == FMT_VQ13 ? 13 : 12; }
__host__ __device__ constexpr int vq_codes(int fmt) { return 1 << vq_bits(fmt); }

// Weights per block and bytes per block of each block format (canonical
// layout; not meaningful for the VQ formats, whose rows have no blocks: use
// row_bytes).
__host__ __device__ constexpr int block_weights(int fmt) { return fmt == FMT_Q8 || fmt == FMT_MX4 ? 32 : 256; }
__host__ __device__ constexpr int block_bytes(int fmt) {
  return fmt == FMT_IQ2 ? 66 : fmt == FMT_Q2K ? 84 : fmt == FMT_Q4K ? 144 : fmt == FMT_MX4 ? 17 : 34;
}
// Bytes of one row of K weights (both layouts hold the same bytes per row).
__host__ __device__ constexpr int64_t row_bytes(int fmt, int K) {
  return is_vq(fmt) ? 2 + 3 * (int64_t)K / 16 + (fmt == FMT_VQ13 ? K / 64 : 0)
                    : (int64_t)(K / block_weights(fmt)) * block_bytes(fmt);
}
// Bytes of n_experts matrices of `rows` rows by K inputs.
__host__ __device__ constexpr int64_t matrix_bytes(int fmt, int64_t n_experts, int rows, int K) {
  return n_experts * rows * row_bytes(fmt, K);
}
// Smallest K (inputs per row) a format allows; K must be a multiple of it.
__host__ __device__ constexpr int k_multiple(int fmt) { return is_vq(fmt) ? 64 : block_weights(fmt); }

// Scale bytes per superblock of the two K-quant formats (sub-block scales and mins).
__host__ __device__ constexpr int kq_scale_bytes(int fmt) { return fmt == FMT_Q4K ? 12 : 16; }
// Quant bytes per superblock of the two K-quant formats.
__host__ __device__ constexpr int kq_quant_bytes(int fmt) { return fmt == FMT_Q4K ? 128 : 64; }

// A weight tensor in the device layout: n_experts matrices of `rows` rows by
// K inputs.  Planes (see include/moe.h):
//   IQ2: p_scale = fp16 d[R][nb],            p_a = payload[R][nb][64]
//   Q2K: p_scale = {fp16 d, dmin}[R][nb],    p_a = scale bytes[R][nb][16],
//        p_b = quants[R][nb][64]
//   Q4K: p_scale = {fp16 d, dmin}[R][nb],    p_a = scale bytes[R][nb][12],
//        p_b = quants[R][nb][128]
//   Q8 : p_scale = fp16 d[R][nb],            p_a = int8 q[R][nb][32]
//   MX4: p_scale = E8M0 e[R][nb],            p_a = E2M1 codes[R][nb][16]
//   VQ : p_scale = fp16 gain[R],             p_a = 12-bit index streams[R][3K/16],
//        p_b = (13 bits) bit planes[R][K/64]
struct QMat {
  const uint8_t* p_scale;
  const uint8_t* p_a;
  const uint8_t* p_b;
  int fmt;
  int rows;  // rows per expert
  int K;     // inputs per row
  int nb;    // blocks per row
};

inline QMat make_qmat(const void* base, int fmt, int n_experts, int rows, int K) {
  QMat m;
  const uint8_t* b = static_cast<const uint8_t*>(base);
  int64_t nb = is_vq(fmt) ? K / 256 : K / block_weights(fmt);
  int64_t R = (int64_t)n_experts * rows;
  m.fmt = fmt;
  m.rows = rows;
  m.K = K;
  m.nb = (int)nb;
  m.p_scale = b;
  if (fmt == FMT_IQ2) {
    m.p_a = b + R * nb * 2;
    m.p_b = nullptr;
  } else if (fmt == FMT_Q2K) {
    m.p_a = b + R * nb * 4;
    m.p_b = b + R * nb * 20;
  } else if (fmt == FMT_Q4K) {
    m.p_a = b + R * nb * 4;
    m.p_b = b + R * nb * 16;
  } else if (fmt == FMT_MX4) {
    m.p_a = b + R * nb;
    m.p_b = nullptr;
  } else if (is_vq(fmt)) {
    m.nb = K / 256;
    m.p_a = b + R * 2;
    m.p_b = fmt == FMT_VQ13 ? m.p_a + R * (3 * (int64_t)K / 16) : nullptr;
  } else {
    m.p_a = b + R * nb * 2;
    m.p_b = nullptr;
  }
  return m;
}

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Load 16 bytes (as 4 dwords) with a plain vector load.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Non-temporal 16-byte load for weights that are streamed exactly once.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// SiLU g * sigmoid(g) with the hardware base-2 exponential and reciprocal
// (a few ulp from the correctly rounded value; the layer's bar is 1e-3
// relative L2).  Large negative g gives exp2 = inf, rcp = 0 and -0.
__device__ __forceinline__ float silu(float g) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace qmoe
