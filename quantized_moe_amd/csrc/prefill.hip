// Prefill path: grouped GEMMs over token buckets on fp16 MFMA.
//
// "YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 4.4 runs prefill
// experts on 16-bit matrix units and keeps every product exact by feeding
// codewords that convert to 16-bit floats without rounding.  The same idea on
// gfx950, with fp16 operands throughout:
//   * every B fragment handed to v_mfma is an exact small integer (IQ2:
//     (2s+1) * grid value <= 217; Q2K: sc * q <= 45), the fp16 superblock
//     scales are applied in an fp32 epilogue once per 256 inputs, and Q2K's
//     min term is a second, K=16 MFMA against per-sub-block sums of the A rows;
//     Q8 weights (the shared expert) enter as fp16(d*q*2^k), rounded once,
//     with 2^k a power of two per output row and superblock that keeps every
//     product a normal fp16 (undone in the fp32 epilogue);
//   * the activations x are converted once to fp16 with a per-token power of
//     two (exact) that puts max|x_t| in [2^13, 2^14), undone in the gate/up
//     epilogue; the SwiGLU output h is stored as fp16 times a power of two
//     per (row, 64 outputs) that puts max|h| over the work item's N tile
//     (a multiple of 64 outputs) in [2^14, 2^15) (one rounding, 2^-11 relative,
//     whatever the scale of x and of the weights); a short pass then brings
//     every row to its largest exponent (exact but for fp16 subnormals,
//     below 2^-24 of the row's maximum), and the down GEMM applies the row's
//     power of two to its fp32 outputs.
//
// One persistent kernel per GEMM (routed gate/up, routed down, shared gate/up,
// shared down).  A work item is (M tile of BM rows of one expert's bucket, or
// of the shared expert's rows, N tile of output rows); every wave owns 16
// output rows and all 16-row M sub-tiles, so each decoded B fragment feeds up
// to BM / 16 MFMAs per matrix.  The routed GEMMs run 32-row tiles in 16-wave
// blocks (128 VGPRs per wave), the shared GEMMs 64-row tiles in 8-wave blocks
// (256 VGPRs).  Each wave takes whole superblocks (KS = 1, N tile 16 per
// wave): a lane's weights of a superblock are one 16-byte load for the 2-bit
// formats.  Only the two-matrix Q8 gate/up in 16-wave blocks, which would
// spill, has the two waves of a pair split every superblock's inputs
// (KS = 2), their partial sums meeting in LDS once per item.
// The K loop runs over 256-input superblocks and is software-pipelined across
// work items: every wave keeps its weight loads PD superblocks ahead in
// registers, the A rows of the next superblock are loaded while the current
// one is computed and land in the other half of an LDS double buffer, and one
// barrier per superblock separates the two.  The address unit charges every
// vector load the same, whatever its width, so the loads are as wide as the
// layout allows.  Work items are mapped so that all N tiles of an M tile run
// on one XCD and share its L2.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_iq2.hpp"
#include "vq.hpp"

namespace qmoe {

// A rows in LDS (one superblock of fp16 inputs, 32 pieces of 16 bytes) in
// one of two layouts.  Swizzled, for the one-matrix down GEMMs: no padding,
// piece p of row r at slot p ^ (r % 8); an MFMA operand read (16 rows at one
// piece, four lane groups 8 pieces apart) meets no bank twice (measured 7.2
// LDS clocks per 1 KB wave read, against 9.0 with a 33-piece row stride and
// 7.5 for consecutive addresses), for one XOR per read step.  Padded, for
// the two-matrix gate/up GEMMs, which are bound by vector instructions and
// were slower with that XOR: 33-piece rows, every read an immediate offset.
__host__ __device__ constexpr int a_row_bytes(bool swizzled) { return swizzled ? 32 * 16 : 33 * 16; }

// Work-item shape: BM rows of A (one expert's bucket, or the shared
// expert's rows) by 16 output rows per wave of a W-wave block, the two waves
// of a pair sharing their output rows (KS = 2) or not (KS = 1).  The routed
// GEMMs run (32, 16): four waves per SIMD at 128 VGPRs hide the weight
// stream's latency, and their buckets hold few rows.  The shared GEMMs run
// (64, 8): every item has 64 rows, each decoded weight fragment feeds up to
// four MFMAs, and 256 VGPRs per wave hold them (measured at 1024 and 8 x
// 4096 tokens: (64, 8) was faster for the shared expert and slower for the
// routed experts, (64, 16) spilled).
template <int BM_, int W_>
struct GemmTile {
  static constexpr int BM = BM_, W = W_;
  static constexpr int THREADS = 64 * W, PAIRS = W / 2;
  static constexpr int NSUB = BM / 16;       // 16-row MFMA sub-tiles
  static constexpr int A_PIECES = BM * 32;   // 16-byte pieces of one A superblock chunk
  static constexpr int SGN = BM == 64 ? 8 : 16;  // IQ2 sign-table copies (the LDS of 64-row tiles)
  static constexpr int bn(int ks) { return 16 * W / ks; }  // output rows per work item
};
using RoutedTile = GemmTile<PREFILL_BM, 16>;
using SharedTile = GemmTile<PREFILL_SHARED_BM, 8>;

// ---------------------------------------------------------------------------
// x -> fp16 with a per-token power-of-two scale
// ---------------------------------------------------------------------------
// x16[t][i] = fp16(x[t][i] * 2^-e_t), xs[t] = 2^e_t, with e_t such that
// max_i |x[t][i]| * 2^-e_t lies in [2^13, 2^14) (e_t = 0 for a zero or
// non-finite row), and route_xs[pos[t][j]] = 2^e_t for the token's k routes.
// The scaling is exact; the fp16 rounding is the only error.
__global__ __launch_bounds__(256) void x16_kernel(const void* __restrict__ x, int x_dtype, int d,
                                                  uint16_t* __restrict__ x16, float* __restrict__ xs,
                                                  const int32_t* __restrict__ pos, int k,
                                                  float* __restrict__ route_xs) {
  const int n_routes = (int)gridDim.x * k;
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  auto load4 = [&](int i, float* v) {
    if (x_dtype == X_BF16) {
      const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + (int64_t)t * d + i);
      v[0] = __uint_as_float(b.x << 16);
      v[1] = __uint_as_float(b.x & 0xffff0000u);
      v[2] = __uint_as_float(b.y << 16);
      v[3] = __uint_as_float(b.y & 0xffff0000u);
    } else {
      const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + (int64_t)t * d + i);
      v[0] = f.x;
      v[1] = f.y;
      v[2] = f.z;
      v[3] = f.w;
    }
  };
  float m = 0.0f;
  for (int i = 4 * tid; i < d; i += 1024) {
    float v[4];
    load4(i, v);
#pragma unroll
    for (int u = 0; u < 4; u++) m = fmaxf(m, fabsf(v[u]));
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (m > 0.0f && m <= 3.4e38f) {
    int ex;
    frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
    e = ex - 14;
  }
  const float sc = ldexpf(1.0f, -e);
  for (int i = 4 * tid; i < d; i += 1024) {
    float v[4];
    load4(i, v);
    const uint2 h = make_uint2(to_h(v[0] * sc) | (to_h(v[1] * sc) << 16), to_h(v[2] * sc) | (to_h(v[3] * sc) << 16));
    *reinterpret_cast<uint2*>(x16 + (int64_t)t * d + i) = h;
  }
  if (tid == 0) xs[t] = ldexpf(1.0f, e);
  // the same scale at each of the token's routes in bucket order (a route
  // whose expert id is out of range has no place: pos holds n_routes)
  if (tid < k) {
    const int p = pos[(int64_t)t * k + tid];
    if ((unsigned)p < (unsigned)n_routes) route_xs[p] = ldexpf(1.0f, e);
  }
}

// ---------------------------------------------------------------------------
// arguments
// ---------------------------------------------------------------------------
struct GemmArgs {
  QMat B0, B1;                 // B0 = gate (or down), B1 = up (gate/up only)
  const uint8_t* grid;         // IQ2 grid [256][8]
  const uint8_t* vq_cb;        // VQ codebook: E4M3 codewords [n][8]
  const uint16_t* a16;         // fp16 A rows: x16 [T][K] (gate/up) or H [rows][K] (down)
  int a16_bytes;               // size of a16 (below 2^31)
  const float* rowxs;          // gate/up: scale of x16 for each row of the row space
  int K;                       // inputs (d for gate/up, f for down)
  int N;                       // output rows (f for gate/up, d for down)
  // grouping
  int routed;                  // 1: buckets of a routed expert, 0: shared (identity)
  int n_rows;                  // shared: number of rows (T)
  int E, k;
  const int32_t* offsets;      // routed: [E+1]
  const int32_t* tile_start;   // routed: [E+1]
  const int32_t* perm;         // routed: [T*k]
  // output
  void* out;                   // gate/up: fp16 H [rows][N]; down: fp32 [rows][N]
  // power-of-two exponents of H: H[row][c] = fp16(h * 2^-hexp[row][c / PREFILL_HCHUNK])
  int8_t* hexp_out;            // gate/up: written, [rows][N / PREFILL_HCHUNK]
  const float* row_scale;      // down: 2^e of each A row (H row = fp16(h 2^-e)), [rows]
};

// ---------------------------------------------------------------------------
// B operand: one lane's weight row, a superblock (KS = 1) or half a
// superblock (KS = 2) at a time.
//
// K order inside a superblock.  MFMA sums over K, so any permutation of the
// 256 inputs applied to A and B alike gives the same product.  At k32 step q
// lane group g4 = lane / 16 takes inputs 64*g4 + 8*q .. +7 (not the natural
// 32*q + 8*g4): each lane then needs one contiguous slice of the block and
// every field index below is a compile-time constant.  With KS = 1 a wave
// runs all eight steps and a lane loads inputs 64*g4 .. +63 (two IQ2
// sub-blocks, four Q2K ones).  With KS = 2 the two waves of a pair split the
// steps: half h runs q = 4h .. 4h+3, i.e. inputs 64*g4 + 32*h .. +31.  The A
// rows are laid out in LDS with the same permutation (16-byte piece 8*g4 + q).
// ---------------------------------------------------------------------------
template <int FMT, int KS>
struct BRegs;

// load(m, row0, lrow, sb, g4, h): row0 is wave-uniform (the item's first
// row), lrow the lane's row within it; the uniform part of every address is
// formed apart so it stays in scalar registers.
// KS = 2 (a wave takes half of each superblock's inputs): the lane's slice is
// inputs 64*g4 + 32*h .. +31, one 8-byte load.  KS = 1 (a wave takes whole
// superblocks): inputs 64*g4 .. +63, one 16-byte load -- half the load
// instructions per weight.  Words 2*hh, 2*hh + 1 hold half hh of the slice.
template <int KS>
struct BRegs<FMT_IQ2, KS> {
  uint32_t w[2 * (3 - KS)];  // (A, B) words of sub-block 2*g4 + h, or of 2*g4 and 2*g4 + 1
  __device__ __forceinline__ void load(const QMat& m, int64_t row0, int lrow, int sb, int g4, int h) {
    const uint8_t* base = m.p_a + (row0 * m.nb + sb) * 64;
    if constexpr (KS == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(base + (uint32_t)(lrow * m.nb * 64 + 16 * g4 + 8 * h));
      w[0] = v.x;
      w[1] = v.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(base + (uint32_t)(lrow * m.nb * 64 + 16 * g4));
      w[0] = v.x;
      w[1] = v.y;
      w[2] = v.z;
      w[3] = v.w;
    }
  }
};

template <int KS>
struct BRegs<FMT_Q2K, KS> {
  uint32_t q[2 * (3 - KS)];  // quant bytes 16*g4 + 8*h .. +7, or 16*g4 .. +15
  uint32_t sc;               // scale/min bytes of sub-blocks 4*g4 .. +3 ((d, dmin) come in an SGroup)
  __device__ __forceinline__ void load(const QMat& m, int64_t row0, int lrow, int sb, int g4, int h) {
    const int64_t blk0 = row0 * m.nb + sb;
    const uint32_t lb = (uint32_t)(lrow * m.nb);
    if constexpr (KS == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(m.p_b + blk0 * 64 + (lb * 64 + 16 * g4 + 8 * h));
      q[0] = v.x;
      q[1] = v.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(m.p_b + blk0 * 64 + (lb * 64 + 16 * g4));
      q[0] = v.x;
      q[1] = v.y;
      q[2] = v.z;
      q[3] = v.w;
    }
    sc = *reinterpret_cast<const uint32_t*>(m.p_a + blk0 * 16 + (lb * 16 + 4 * g4));
  }
};

// Q4K: quants of sub-block 2*g4 + h (16 bytes, KS = 2) or of sub-blocks
// 2*g4, 2*g4 + 1 (32 bytes); the superblock's 12 scale bytes come with one
// 12-byte load, of which the lane keeps its two low-bit bytes and its
// top-bit byte.
template <int KS>
struct BRegs<FMT_Q4K, KS> {
  uint4 q[3 - KS];
  uint32_t lo, hi;
  __device__ __forceinline__ void load(const QMat& m, int64_t row0, int lrow, int sb, int g4, int h) {
    const int64_t blk0 = row0 * m.nb + sb;
    const uint32_t lb = (uint32_t)(lrow * m.nb);
    const uint8_t* qp = m.p_b + blk0 * 128 + (lb * 128 + 32 * g4 + (KS == 2 ? 16 * h : 0));
#pragma unroll
    for (int i = 0; i < 3 - KS; i++) q[i] = *reinterpret_cast<const uint4*>(qp + 16 * i);
    const uint3 v = *reinterpret_cast<const uint3*>(m.p_a + blk0 * 12 + lb * 12);
    const uint32_t wlo = (g4 >> 1) ? v.y : v.x;
    lo = (g4 & 1) ? wlo >> 16 : wlo & 0xffffu;
    hi = (v.z >> (8 * g4)) & 255u;
  }
};

template <int KS>
struct BRegs<FMT_Q8, KS> {
  uint4 q[2 * (3 - KS)];  // quants of block 2*g4 + h (32 bytes), or of blocks 2*g4, 2*g4 + 1 (64 bytes)
  uint32_t d;             // fp16 scale of each block (KS = 1: both, one 4-byte load)
  __device__ __forceinline__ void load(const QMat& m, int64_t row0, int lrow, int sb, int g4, int h) {
    const int64_t blk0 = row0 * m.nb + sb * 8;
    const uint32_t lb = (uint32_t)(lrow * m.nb + 2 * g4 + (KS == 2 ? h : 0));
#pragma unroll
    for (int i = 0; i < 2 * (3 - KS); i++) q[i] = ld16_stream(m.p_a + blk0 * 32 + lb * 32 + 16 * i);
    if constexpr (KS == 2)
      d = reinterpret_cast<const uint16_t*>(m.p_scale)[blk0 + lb];
    else
      d = *reinterpret_cast<const uint32_t*>(m.p_scale + (blk0 + lb) * 2);
  }
};

// MXFP4: the codes of block 2*g4 + h (16 bytes, KS = 2) or of blocks 2*g4,
// 2*g4 + 1 (32 bytes), and their E8M0 scale bytes.
template <int KS>
struct BRegs<FMT_MX4, KS> {
  uint4 q[3 - KS];
  uint32_t e;
  __device__ __forceinline__ void load(const QMat& m, int64_t row0, int lrow, int sb, int g4, int h) {
    const int64_t blk0 = row0 * m.nb + sb * 8;
    const uint32_t lb = (uint32_t)(lrow * m.nb + 2 * g4 + (KS == 2 ? h : 0));
#pragma unroll
    for (int i = 0; i < 3 - KS; i++) q[i] = *reinterpret_cast<const uint4*>(m.p_a + (blk0 + lb) * 16 + 16 * i);
    if constexpr (KS == 2)
      e = m.p_scale[blk0 + lb];
    else
      e = *reinterpret_cast<const uint16_t*>(m.p_scale + blk0 + lb);
  }
};

// VQ rows: the 8 indices of inputs 64*g4 .. +63 of the superblock (12 stream
// bytes, one 12-byte load) and, for 13 bits, their plane byte.  Only whole
// superblocks per wave (KS = 1): half a lane's slice would start mid-dword.
template <int KS>
struct BRegs<FMT_VQ12, KS> {
  static_assert(KS == 1, "VQ rows are read in whole superblocks");
  VqPiece p;
  __device__ __forceinline__ void load(const QMat& m, int64_t row0, int lrow, int sb, int g4, int) {
    const int rs = 3 * m.K / 16;  // stream bytes per row
    const uint3 v = *reinterpret_cast<const uint3*>(m.p_a + row0 * rs + sb * 48 + (uint32_t)(lrow * rs + 12 * g4));
    p.w0 = v.x;
    p.w1 = v.y;
    p.w2 = v.z;
    p.pl = 0u;
  }
};
template <int KS>
struct BRegs<FMT_VQ13, KS> {
  static_assert(KS == 1, "VQ rows are read in whole superblocks");
  VqPiece p;
  __device__ __forceinline__ void load(const QMat& m, int64_t row0, int lrow, int sb, int g4, int) {
    const int rs = 3 * m.K / 16, bs = m.K / 64;  // stream and plane bytes per row
    const uint3 v = *reinterpret_cast<const uint3*>(m.p_a + row0 * rs + sb * 48 + (uint32_t)(lrow * rs + 12 * g4));
    p.w0 = v.x;
    p.w1 = v.y;
    p.w2 = v.z;
    p.pl = m.p_b[row0 * bs + sb * 4 + (uint32_t)(lrow * bs + g4)];
  }
};

// The superblock scales of PD consecutive superblocks sb0 .. sb0 + PD - 1 of
// the lane's row, fetched with one load (they are contiguous in the scale
// plane): IQ2 fp16 d, Q2K (fp16 d, fp16 dmin) pairs.  A vector-memory
// instruction costs the address unit the same whatever its width, so one
// load per PD superblocks instead of one per superblock.  (Q8 scales are per
// 32-input block and stay with the codes.)
template <int FMT, int PD>
struct SGroup {
  static constexpr bool KQ = FMT == FMT_Q2K || FMT == FMT_Q4K;  // (d, dmin) pairs
  static constexpr int NW = FMT == FMT_IQ2 ? (PD + 1) / 2 : KQ ? PD : 1;
  uint32_t w[NW];
  __device__ __forceinline__ void load(const QMat& m, int64_t row0, int lrow, int sb0) {
    if constexpr (FMT == FMT_IQ2) {
      const uint8_t* p = m.p_scale + ((row0 + lrow) * m.nb + sb0) * 2;
      if constexpr (PD == 1) w[0] = *reinterpret_cast<const uint16_t*>(p);
      if constexpr (PD == 2) w[0] = *reinterpret_cast<const uint32_t*>(p);
      if constexpr (PD == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x;
        w[1] = v.y;
      }
    } else if constexpr (KQ) {
      const uint8_t* p = m.p_scale + ((row0 + lrow) * m.nb + sb0) * 4;
      if constexpr (PD == 1) w[0] = *reinterpret_cast<const uint32_t*>(p);
      if constexpr (PD == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x;
        w[1] = v.y;
      }
      if constexpr (PD == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
      }
    }
  }
  // scale word of superblock sb0 + u (u a compile-time constant)
  __device__ __forceinline__ uint32_t word(int u) const {
    if constexpr (FMT == FMT_IQ2) return (w[u >> 1] >> (16 * (u & 1))) & 0xffffu;
    if constexpr (KQ) return w[u];
    return 0u;
  }
};

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;  // i is a compile-time constant
}

// Fragment of local step i (q = 4h + i): 8 exact integers, group i of the
// lane's sub-block.  SC = iq2_scale_h2 of the sub-block, CB = (lane % 16) << 4,
// CS = (lane % SGN) << 4.
template <int SGN, int KS>
__device__ __forceinline__ uint4 iq2_frag(const BRegs<FMT_IQ2, KS>& b, int hh, int i, uint32_t SC, uint32_t CB,
                                          uint32_t CS, const uint8_t* tm, const uint8_t* sgn) {
  return iq2_frag_words<SGN>(b.w[2 * hh], b.w[2 * hh + 1], i, SC, CB, CS, tm, sgn);
}

// Q2K fragment constants of a sub-block with scale sc: quants placed under
// the fp16 exponent byte 0x64 read 1024 + 4^p q for field p of their byte, and
// one packed fused multiply-add with (mul, add) per pair of fields leaves the
// exact integers sc * q (<= 45): fields 0, 1 take (sc, sc / 4) and
// (-1024 sc, -256 sc); fields 2, 3 take (sc / 16, sc / 64) and (-64 sc, -16 sc).
struct Q2kConst {
  f16x2_t mul01, add01, mul23, add23;
};
__device__ __forceinline__ Q2kConst q2k_const(uint32_t sc) {
  const _Float16 h = (_Float16)(float)sc;
  const f16x2_t hh = {h, h};
  Q2kConst k;
  k.mul01 = hh * f16x2_t{(_Float16)1.0f, (_Float16)0.25f};
  k.add01 = hh * f16x2_t{(_Float16)-1024.0f, (_Float16)-256.0f};
  k.mul23 = hh * f16x2_t{(_Float16)0.0625f, (_Float16)0.015625f};
  k.add23 = hh * f16x2_t{(_Float16)-64.0f, (_Float16)-16.0f};
  return k;
}

// Q2K fragment of local step i: quant bytes 2i, 2i+1 of the lane's 8 (four
// 2-bit quants each, weight 4j + p in field p of byte j) as the 8 exact
// integers sc * q, computed in registers: a table lookup per byte would put
// lanes with equal (sc, byte) bits on the same LDS banks.
template <int KS>
__device__ __forceinline__ uint4 q2k_frag(const BRegs<FMT_Q2K, KS>& b, int hh, int i, const Q2kConst& k) {
  const uint32_t w = (i >> 1) ? b.q[2 * hh + 1] : b.q[2 * hh];
  const uint32_t x0 = 2u * (uint32_t)(i & 1);  // quant bytes x0, x0 + 1 of word w
  auto words = [&](uint32_t x, uint32_t& w01, uint32_t& w23) {
    const uint32_t t = __builtin_amdgcn_perm(w, 0x64646464u, 0x00040004u + 0x00010001u * x);  // byte x in bytes 0, 2
    w01 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, t & 0xff0cff03u),
                                                                 k.mul01, k.add01));
    w23 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, t & 0xffc0ff30u),
                                                                 k.mul23, k.add23));
  };
  uint32_t a, bb, c, d;
  words(x0, a, bb);
  words(x0 + 1, c, d);
  return make_uint4(a, bb, c, d);
}

// Q2K min-term B fragment (K = the 16 sub-blocks): 16 m_j for j = 4*g4 .. +3,
// m_j being the high nibbles of this lane's scale word.
template <int KS>
__device__ __forceinline__ uint2 q2k_min_frag(const BRegs<FMT_Q2K, KS>& b) {
  const uint32_t w = b.sc;
  const uint32_t m0 = (w >> 4) & 15u, m1 = (w >> 12) & 15u, m2 = (w >> 20) & 15u, m3 = (w >> 28) & 15u;
  // 16 m: the sums of A are stored divided by 16
  return make_uint2(to_h((float)(16u * m0)) | (to_h((float)(16u * m1)) << 16),
                    to_h((float)(16u * m2)) | (to_h((float)(16u * m3)) << 16));
}

// Q4K: 6-bit scale and min of the lane's sub-block sbl (0 or 1 of its pair).
template <int KS>
__device__ __forceinline__ uint32_t q4k_sc(const BRegs<FMT_Q4K, KS>& b, int sbl) {
  return ((b.lo >> (8 * sbl)) & 15u) | (((b.hi >> (4 * sbl)) & 3u) << 4);
}
template <int KS>
__device__ __forceinline__ uint32_t q4k_min(const BRegs<FMT_Q4K, KS>& b, int sbl) {
  return ((b.lo >> (8 * sbl + 4)) & 15u) | (((b.hi >> (4 * sbl + 2)) & 3u) << 4);
}

// Q4K fragment of local step i: the 8 exact integers sc * q of quant word w
// (elements 2j, 2j+1 in the low and high nibble of byte j).  Byte j goes to
// bytes 0 and 2 under fp16 exponent bytes 0x64 (one v_perm); masking keeps
// the low nibble in the first half (1024 + q) and the high nibble, four bits
// up, in the second (1024 + 16 q); one packed fused multiply-add with
// (sc, sc / 16) and (-1024 sc, -64 sc) leaves sc * q <= 945, exact in fp16.
__device__ __forceinline__ uint4 q4k_frag(uint32_t w, f16x2_t mul, f16x2_t add) {
  auto pair = [&](uint32_t sel) {
    const uint32_t t = __builtin_amdgcn_perm(w, 0x64646464u, sel) & 0xfff0ff0fu;
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, t), mul, add));
  };
  return make_uint4(pair(0x00040004u), pair(0x00050005u), pair(0x00060006u), pair(0x00070007u));
}

// Q4K min-term B fragment (K = the 16 groups of 16 inputs): group j belongs
// to sub-block j / 2, so lane group g4 gives 16 m of sub-blocks 2*g4, 2*g4,
// 2*g4 + 1, 2*g4 + 1.
template <int KS>
__device__ __forceinline__ uint2 q4k_min_frag(const BRegs<FMT_Q4K, KS>& b) {
  const uint32_t m0 = to_h((float)(16u * q4k_min(b, 0))), m1 = to_h((float)(16u * q4k_min(b, 1)));  // (sums / 16)
  return make_uint2(m0 | (m0 << 16), m1 | (m1 << 16));
}

// Q8 block scales pre-multiplied by a power of two 2^k shared by the wave's
// four lane groups, i.e. by one output row's superblock (KS = 1: the lane's
// blocks 2*g4, 2*g4 + 1) or by the wave's half of it (KS = 2: block
// 2*g4 + h).  k puts the largest |d| among them in [2^7, 2^8), so every
// product d*q*2^k with 1 <= |q| <= 128 of that block is a normal fp16 below
// 2^15 whatever the magnitude of d; a block with a much smaller d loses
// only digits that are small against the largest block.  dw gets the scaled
// fp16 words (fp32 product, one rounding); returns 2^-k for the epilogue.
template <int KS>
__device__ __forceinline__ float q8_prescale(uint32_t d, uint32_t& dw) {
  uint32_t e = (d >> 10) & 31u;  // biased fp16 exponent of each |d|
  if constexpr (KS == 1) e = max(e, (d >> 26) & 31u);
  e = max(e, (uint32_t)__shfl_xor((int)e, 16, 64));
  e = max(e, (uint32_t)__shfl_xor((int)e, 32, 64));
  const int k = 22 - (int)max(e, 1u);  // |d| < 2^(e - 14)  ->  |d| 2^k < 2^8
  const float s = __builtin_amdgcn_ldexpf(1.0f, k);
  dw = to_h(from_h(d & 0xffffu) * s);
  if constexpr (KS == 1) dw |= to_h(from_h(d >> 16) * s) << 16;
  return __builtin_amdgcn_ldexpf(1.0f, -k);
}

// Q8 fragment of local step i: the 8 products d*q (d the prescaled scale of
// the block, from dw) as fp16, each rounded once.  A quant byte b becomes
// the exact fp16 integer q: (b ^ 0x80) placed under an fp16 exponent byte
// 0x64 reads 1024 + q + 128 (one v_perm per pair), minus 1152 (one packed
// add); one packed multiply by (d, d) then rounds q*d.
template <int KS>
__device__ __forceinline__ uint4 q8_frag(const BRegs<FMT_Q8, KS>& b, int hh, int i, uint32_t dw) {
  const uint32_t w0 = word_of(b.q[2 * hh + (i >> 1)], 2 * (i & 1)) ^ 0x80808080u;
  const uint32_t w1 = word_of(b.q[2 * hh + (i >> 1)], 2 * (i & 1) + 1) ^ 0x80808080u;
  const f16x2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const uint16_t dh = (uint16_t)(dw >> (16 * hh));
  const f16x2_t dd = {__builtin_bit_cast(_Float16, dh), __builtin_bit_cast(_Float16, dh)};
  auto pair = [&](uint32_t w, uint32_t sel) {
    const f16x2_t q = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(w, 0x64646464u, sel)) + bias;
    return __builtin_bit_cast(uint32_t, q * dd);
  };
  return make_uint4(pair(w0, 0x00050004u), pair(w0, 0x00070006u), pair(w1, 0x00050004u), pair(w1, 0x00070006u));
}

// MXFP4 block scales brought to the wave's superblock (KS = 1: the lane's
// blocks 2*g4, 2*g4 + 1; KS = 2: block 2*g4 + h; the four lane groups
// together hold the output row's 8 blocks, or their half): em = the largest
// E8M0 exponent among them; f0, f1 = 2^(e_b - em) for the lane's blocks, the
// factors the conversion applies (exact: an E2M1 value times a power of two
// <= 1 is an fp16, or below 2^-24 of the superblock's largest weights);
// returns 2^(em - 127), applied to the superblock's fp32 partial sums.
template <int KS>
__device__ __forceinline__ float mx4_prescale(uint32_t e, float& f0, float& f1) {
  const int e0 = (int)(e & 255u), e1 = KS == 1 ? (int)((e >> 8) & 255u) : e0;
  int em = max(e0, e1);
  em = max(em, __shfl_xor(em, 16, 64));
  em = max(em, __shfl_xor(em, 32, 64));
  f0 = __builtin_amdgcn_ldexpf(1.0f, e0 - em);
  f1 = __builtin_amdgcn_ldexpf(1.0f, e1 - em);
  return __builtin_amdgcn_ldexpf(1.0f, em - 127);
}

// MXFP4 fragment: the 8 codes of quant word w (element 2j, 2j + 1 in the low
// and high nibble of byte j) as fp16 values times f, by the hardware
// conversion (exact for a power-of-two f).
__device__ __forceinline__ uint4 mx4_frag(uint32_t w, float f) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, f, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, f, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, f, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, f, 3)));
}

// Maximum of v over each 16-lane row of the wave (the 16 output columns an
// MFMA result row spreads over), returned to every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0xb1>{}));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4e>{}));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
  return v;
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int FMT, bool GATEUP, int KS, class G>
struct GemmLds {
  static constexpr int BM = G::BM, NSUB = G::NSUB, GEMM_PAIRS = G::PAIRS;
  static constexpr bool SWZ = !GATEUP;          // A rows swizzled (one-matrix GEMMs) or padded
  static constexpr int A_ROW = a_row_bytes(SWZ);
  static constexpr int A_BUF = BM * A_ROW;      // LDS bytes per A buffer
  static constexpr int kMag = FMT == FMT_IQ2 ? IQ2_TM_BYTES : 0;
  static constexpr int kSgn = FMT == FMT_IQ2 ? iq2_sgn_bytes<G::SGN>() : 0;
  static constexpr int kCb = is_vq(FMT) ? vq_codes(FMT) * 8 : 0;      // VQ codebook (E4M3)
  // double-buffered A superblock chunk; the gate/up epilogue's h tile
  // (BM x (BN + 4) floats) overlays both buffers (KS = 1) or follows them
  // (KS = 2, whose epilogue holds partial sums in one of them)
  static constexpr int kHt = GATEUP ? BM * (G::bn(KS) + 4) * 4 : 0;
  static constexpr int kA = KS == 1 ? (2 * A_BUF > kHt ? 2 * A_BUF : kHt) : 2 * A_BUF + kHt;
  static constexpr int kS = FMT == FMT_Q2K || FMT == FMT_Q4K ? 2 * 2 * BM * 16 * 2 : 0;  // sums of 16 inputs: [buf][hi/lo][BM][16]
  static constexpr int kTok = 3 * BM * 8;                             // token (gate/up) and scale of each row, 3 items
  static constexpr int kRed = KS == 2 ? NSUB * 4 * GEMM_PAIRS * 64 * 4 : 0;  // one matrix's partial sums of the second halves
  static constexpr int kMax = GATEUP ? 2 * BM * 4 : 0;                // gate/up: [item parity][BM] row maxima of |h|
  static constexpr int oSgn = kMag, oCb = oSgn + kSgn, oA = oCb + kCb, oS = oA + kA, oTok = oS + kS,
                       oRed = oTok + kTok, oMax = oRed + kRed, oTiles = oMax + kMax;
  // then tile_start and offsets of the routed experts: [2][E + 1]
  static constexpr int bytes_for(int E) { return oTiles + 2 * (E + 1) * 4; }
};

// A work item's rows.
struct Item {
  int e;       // expert (0 for the shared expert)
  int nt;      // N tile
  int rows;    // valid rows (0: no item)
  int p0;      // first row of the item in the bucket-ordered row space
  int nm;      // active 16-row sub-tiles
};

template <int FMT, bool GATEUP, int PD, int KS, class G>
__global__ __launch_bounds__(G::THREADS) void gemm_kernel(GemmArgs a) {
  using L = GemmLds<FMT, GATEUP, KS, G>;
  constexpr int BM = G::BM, NSUB = G::NSUB, A_PIECES = G::A_PIECES;
  constexpr bool SWZ = L::SWZ;
  constexpr int A_ROW = L::A_ROW, A_BUF = L::A_BUF;
  constexpr int GEMM_THREADS = G::THREADS, GEMM_PAIRS = G::PAIRS;
  constexpr int BN = G::bn(KS);  // output rows per work item
  extern __shared__ __align__(16) uint8_t lds[];
  const uint8_t* tm = lds;
  const uint8_t* sgn = lds + L::oSgn;
  uint8_t* sA = lds + L::oA;
  uint16_t* sS = reinterpret_cast<uint16_t*>(lds + L::oS);
  int* sTok = reinterpret_cast<int*>(lds + L::oTok);              // [3][BM]
  float* sXs = reinterpret_cast<float*>(lds + L::oTok) + 3 * BM;  // [3][BM]
  float* sRed = reinterpret_cast<float*>(lds + L::oRed);
  uint32_t* sMax = reinterpret_cast<uint32_t*>(lds + L::oMax);  // gate/up: [j % 2][BM], fp32 bits of max|h|
  int* sTiles = reinterpret_cast<int*>(lds + L::oTiles);
  int* sOffsets = sTiles + (a.E + 1);  // (an expert's row count: the difference of two offsets)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = KS == 2 ? wave % GEMM_PAIRS : wave;  // output rows 16 wv .. of the N tile
  const int h = KS == 2 ? wave / GEMM_PAIRS : 0;      // K half: steps q = 4h .. 4h + 3 of every superblock
  const int g4 = lane >> 4, c16 = lane & 15;

  if constexpr (FMT == FMT_IQ2)
    build_iq2_tables<G::SGN>(a.grid, reinterpret_cast<uint4*>(lds), reinterpret_cast<uint4*>(lds + L::oSgn), tid,
                             GEMM_THREADS);
  if constexpr (is_vq(FMT)) vq_stage_codebook(a.vq_cb, lds + L::oCb, vq_codes(FMT), tid, GEMM_THREADS);
  if constexpr (GATEUP) {
    if (tid < 2 * BM) sMax[tid] = 0u;
  }
  if (a.routed) {
    for (int i = tid; i <= a.E; i += GEMM_THREADS) {
      sTiles[i] = a.tile_start[i];
      sOffsets[i] = a.offsets[i];
    }
  }
  __syncthreads();
  const int total_tiles = a.routed ? sTiles[a.E] : (a.n_rows + BM - 1) / BM;
  const int NT = a.N / BN;
  const int nsb = a.K / 256;

  // work-item mapping, XCD-aware (blocks are dealt to the 8 XCDs round-robin).
  // Routed experts (few rows, many distinct weights): an XCD owns M tiles and
  // runs all their N tiles, which share the M tile's A rows in its L2.  The
  // shared expert (every row, one weight matrix): an XCD owns N tiles and its
  // blocks sweep the M tiles across them, so each weight tile is read from
  // HBM once and then served from that XCD's L2.
  const int nblk = gridDim.x;
  const bool n_major = !a.routed;
  const bool xcd_map = (nblk % 8) == 0 && (n_major ? NT >= 8 : total_tiles >= 16);
  const int xcd = blockIdx.x % 8;
  const int n_items = !xcd_map ? total_tiles * NT
                      : n_major ? ((NT - xcd + 7) / 8) * total_tiles
                                : ((total_tiles - xcd + 7) / 8) * NT;
  const int first = xcd_map ? blockIdx.x / 8 : blockIdx.x;
  const int step = xcd_map ? nblk / 8 : nblk;
  const int cnt = first < n_items ? (n_items - first + step - 1) / step : 0;
  if (cnt == 0) return;  // uniform over the block

  // item j of this block
  auto item = [&](int j) {
    Item it;
    if (j >= cnt) {
      it.e = it.nt = it.rows = it.p0 = it.nm = 0;
      return it;
    }
    const int g = first + j * step;
    int tt;
    if (n_major) {
      const int nl = g / total_tiles;
      tt = g - nl * total_tiles;
      it.nt = xcd_map ? xcd + 8 * nl : nl;
    } else {
      const int mt = g / NT;
      it.nt = g - mt * NT;
      tt = xcd_map ? xcd + 8 * mt : mt;
    }
    if (a.routed) {
      int lo = 0, hi = a.E;  // largest e with tile_start[e] <= tt
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sTiles[mid] <= tt) lo = mid; else hi = mid;
      }
      int e = lo;
      while (e + 1 < a.E && sTiles[e + 1] <= tt) e++;  // skip experts with no tiles
      const int m0 = (tt - sTiles[e]) * BM;
      it.e = e;
      it.rows = min(BM, sOffsets[e + 1] - sOffsets[e] - m0);
      it.p0 = sOffsets[e] + m0;
    } else {
      const int m0 = tt * BM;
      it.e = 0;
      it.rows = min(BM, a.n_rows - m0);
      it.p0 = m0;
    }
    it.nm = (it.rows + 15) >> 4;
    // every lane computed the same item: say so, so it lives in SGPRs
    it.e = __builtin_amdgcn_readfirstlane(it.e);
    it.nt = __builtin_amdgcn_readfirstlane(it.nt);
    it.rows = __builtin_amdgcn_readfirstlane(it.rows);
    it.p0 = __builtin_amdgcn_readfirstlane(it.p0);
    it.nm = __builtin_amdgcn_readfirstlane(it.nm);
    return it;
  };
  // Per row of item j, into slot j % 3: gate/up, the token index and the x
  // scale; down, the A row's scale (its output factor).  In the steady state
  // the loads are issued one item ahead (tok_issue) and written to LDS an
  // item later (tok_commit), so no step waits for them.
  int tok_r = 0;
  float xs_r = 0.0f;
  auto tok_issue = [&](const Item& it) {
    const int i = tid % BM;  // every thread loads (uniform load count per step)
    const int p = it.p0 + (i < it.rows ? i : 0);
    if constexpr (GATEUP) {
      tok_r = a.routed ? a.perm[p] : p;
      xs_r = a.rowxs[p];
    } else {
      xs_r = a.row_scale[p];
    }
  };
  auto tok_commit = [&](int j) {
    if (tid < BM) {
      if constexpr (GATEUP) sTok[(j % 3) * BM + tid] = a.routed ? tok_r / a.k : tok_r;
      sXs[(j % 3) * BM + tid] = xs_r;
    }
  };

  // ---- A rows: issue (into registers) and store (into LDS) ----
  // Thread tid holds pieces tid + GEMM_THREADS * i (i < PPT): row
  // tid / 32 + (GEMM_THREADS / 32) i, piece tid % 32, stored at byte
  // row * A_ROW + 16 * (piece ^ row % 8) (swizzled) or + 16 * piece.
  // The swizzle or the padding spreads the 16 rows an MFMA operand read
  // touches over the banks.  A loads are raw buffer loads: a piece outside the
  // item's active rows is given an offset past the end of a16 and reads as
  // zero, so every step issues the same loads.
  constexpr int PPT = A_PIECES / GEMM_THREADS;  // A pieces per thread
  constexpr int RPP = GEMM_THREADS / 32;        // A rows per pass of the block
  static_assert(A_PIECES == PPT * GEMM_THREADS, "whole pieces per thread");
  // DA superblocks of A in flight in registers (set s % 2 holds superblock s)
  constexpr int DA = PD % 2 == 0 ? 2 : 1;
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.a16), (short)0, a.a16_bytes, 0x00020000);
  const int a_row = tid >> 5, a_piece = tid & 31;
  uint4 av0[PPT], av1[PPT];  // sets 0 and 1
  int ap0[PPT], ap1[PPT];    // their LDS byte offsets, -1 if inactive
#pragma unroll
  for (int i = 0; i < PPT; i++) ap0[i] = ap1[i] = -1;
  auto issue_piece = [&](int j, const Item& it, int sb, int row, uint4& v, int& pos) {
    const bool active = row < 16 * it.nm;
    int src;
    if constexpr (GATEUP) {
      src = sTok[(j % 3) * BM + row];
    } else {
      src = it.p0 + (row < it.rows ? row : 0);
    }
    const int off = active ? (src * a.K + sb * 256 + 8 * a_piece) * 2 : 0x7ffffff0;
    const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, off, 0, 0);
    v = make_uint4(w[0], w[1], w[2], w[3]);
    pos = active ? row * A_ROW + 16 * (SWZ ? a_piece ^ (row & 7) : a_piece) : -1;
  };
  // (a branch on set, not a reference chosen by it: the sets stay in registers)
  auto issueA = [&](int set, int j, const Item& it, int sb) {
#pragma unroll
    for (int i = 0; i < PPT; i++) {
      if (set) issue_piece(j, it, sb, a_row + RPP * i, av1[i], ap1[i]);
      else issue_piece(j, it, sb, a_row + RPP * i, av0[i], ap0[i]);
    }
  };
  auto store_piece = [&](int buf, const uint4& v, int pos, int row) {
    uint8_t* dst = sA + buf * A_BUF;
    if (pos >= 0) *reinterpret_cast<uint4*>(dst + pos) = v;
    if constexpr (FMT == FMT_Q2K || FMT == FMT_Q4K) {
      // sums of 16 inputs (pieces 2j, 2j+1, held by lanes t, t^1): Q2K's
      // sub-blocks, halves of Q4K's
      const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
      float sum = 0.0f;
      sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, v.x), one, sum, false);
      sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, v.y), one, sum, false);
      sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, v.z), one, sum, false);
      sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, v.w), one, sum, false);
      if (pos < 0) sum = 0.0f;
      const float o = __shfl_xor(sum, 1, 64);
      if (pos >= 0 && (a_piece & 1) == 0) {
        // stored / 16 (exact): scaled gate/up rows reach |a| < 2^14, and a
        // sum of 16 of them would pass the fp16 range; the min fragments
        // carry the factor 16 back (16 m <= 1008, exact)
        const float t = (sum + o) * 0.0625f;
        const uint32_t hs = to_h(t);
        uint16_t* ss = sS + buf * (2 * BM * 16);
        ss[row * 16 + (a_piece >> 1)] = (uint16_t)hs;
        ss[BM * 16 + row * 16 + (a_piece >> 1)] = (uint16_t)to_h(t - from_h(hs));
      }
    }
  };
  auto storeA = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < PPT; i++) {
      if (set) store_piece(buf, av1[i], ap1[i], a_row + RPP * i);
      else store_piece(buf, av0[i], ap0[i], a_row + RPP * i);
    }
  };

  // ---- B rows: PD superblocks in flight ----
  BRegs<FMT, KS> b0[PD], b1[PD];
  // B row of this lane: (first row of the item's N tile, uniform) + lrow
  const int lrow = wv * 16 + c16;
  // scale groups: *n holds the group of the steps in flight, *c (copied from
  // *n at the group's first step, after its compute) the current group's
  SGroup<FMT, PD> g0n, g1n, g0c, g1c;
  auto issueB = [&](int slot, const Item& it, int sb) {
#pragma unroll
    for (int s = 0; s < PD; s++) {
      if (s == slot) {  // (an item past the end has rows 0 and e = nt = 0: in bounds, unused)
        const int64_t row0 = (int64_t)it.e * a.B0.rows + it.nt * BN;
        if (s == 0) {  // the group's scales first: they return before its codes
          g0n.load(a.B0, row0, lrow, sb);
          if constexpr (GATEUP) g1n.load(a.B1, row0, lrow, sb);
        }
        b0[s].load(a.B0, row0, lrow, sb, g4, h);
        if constexpr (GATEUP) b1[s].load(a.B1, row0, lrow, sb, g4, h);
      }
    }
  };

  f32x4_t acc0[NSUB], acc1[NSUB];
#pragma unroll
  for (int m = 0; m < NSUB; m++) acc0[m] = acc1[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // K-quant gate/up GEMMs (two matrices of Q2K or Q4K) keep no per-superblock
  // partial sums, whose registers spilled: acc holds the item's sums in units
  // of the scale D of the last superblock with d != 0 (the lane's output row:
  // the sums are acc * D).  A superblock with d != 0 first multiplies acc by
  // D / d and sets D = d, and its exact-integer fragments then accumulate
  // straight into acc, its min term scaled by dmin / D; one with d = 0
  // zeroes its fragments' scales and leaves D.  |D / d| <= 2^40 for fp16
  // scales, so no sum leaves the fp32 range; each ratio is one rounding.
  // (Every other GEMM keeps D = 1.)
  float D0 = 1.0f, D1 = 1.0f;

  // VQ: the fp16 row gains of this lane's output column (gate and up, or
  // down) for the current item, requested as the item becomes current (a
  // whole item before its epilogue reads them)
  float vg0 = 1.0f, vg1 = 1.0f;
  auto load_gains = [&](const Item& it) {
    if constexpr (is_vq(FMT)) {
      const int64_t row = (int64_t)it.e * a.N + it.nt * BN + lrow;  // (an item past the end: e = nt = 0)
      vg0 = half_bits_to_float(reinterpret_cast<const uint16_t*>(a.B0.p_scale)[row]);
      if constexpr (GATEUP) vg1 = half_bits_to_float(reinterpret_cast<const uint16_t*>(a.B1.p_scale)[row]);
    }
  };

  // One superblock half-step with NM (a compile-time 1 or 2) active
  // sub-tiles: straight-line code, so the scheduler can overlap the table
  // reads, the fragment arithmetic and the MFMAs of consecutive k32 steps.
  auto compute = [&](auto nm_c, int slot, int buf, uint32_t sw0, uint32_t sw1) {
    constexpr int NM = decltype(nm_c)::value;
    const BRegs<FMT, KS>& B0 = b0[slot];
    const BRegs<FMT, KS>& B1 = b1[slot];
    // piece 8 g4 + j (j = 4 h + i) of row 16 m + c16: slot 8 g4 + j, or
    // 8 g4 + (j ^ c16 % 8) swizzled
    const int abase = SWZ ? (buf * A_BUF + c16 * A_ROW + g4 * 128) | (((c16 & 7) ^ (4 * h)) << 4)
                          : buf * A_BUF + c16 * A_ROW + g4 * 128 + h * 64;
    auto aread = [&](int m, int i) {
      const int off = SWZ ? abase ^ (i << 4) : abase + 16 * i;
      return *reinterpret_cast<const uint4*>(sA + off + m * 16 * A_ROW);
    };
    if constexpr (is_vq(FMT)) {
      // B fragment of step q = the codeword of the lane's index q, converted
      // to fp16 exactly; no per-superblock scale (the row gain is applied in
      // the item epilogue)
      const uint8_t* cb = lds + L::oCb;
      constexpr bool B13 = FMT == FMT_VQ13;
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const uint4 f0 = vq_to_f16(vq_codeword(cb, vq_index<B13>(B0.p, q)));
        uint4 f1;
        if constexpr (GATEUP) f1 = vq_to_f16(vq_codeword(cb, vq_index<B13>(B1.p, q)));
#pragma unroll
        for (int m = 0; m < NM; m++) {
          const uint4 av = aread(m, q);
          acc0[m] = mfma32(av, f0, acc0[m]);
          if constexpr (GATEUP) acc1[m] = mfma32(av, f1, acc1[m]);
        }
        if (q % 2 == 1) __builtin_amdgcn_sched_barrier(0);  // bound the live fragments
      }
    } else if constexpr (FMT == FMT_MX4) {
      float f00, f01, f10 = 0.f, f11 = 0.f;
      const float ps0 = mx4_prescale<KS>(B0.e, f00, f01);
      float ps1 = 0.0f;
      if constexpr (GATEUP) ps1 = mx4_prescale<KS>(B1.e, f10, f11);
      f32x4_t s0[NM], s1[NM];
#pragma unroll
      for (int m = 0; m < NM; m++) s0[m] = s1[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hh = 0; hh < 3 - KS; hh++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const uint4 f0 = mx4_frag(word_of(B0.q[hh], i), hh ? f01 : f00);
          uint4 f1;
          if constexpr (GATEUP) f1 = mx4_frag(word_of(B1.q[hh], i), hh ? f11 : f10);
#pragma unroll
          for (int m = 0; m < NM; m++) {
            const uint4 av = aread(m, 4 * hh + i);
            s0[m] = mfma32(av, f0, s0[m]);
            if constexpr (GATEUP) s1[m] = mfma32(av, f1, s1[m]);
          }
          if (i == 1 || i == 3) __builtin_amdgcn_sched_barrier(0);  // bound the live fragments
        }
      }
#pragma unroll
      for (int m = 0; m < NM; m++) {
        acc0[m] += ps0 * s0[m];
        if constexpr (GATEUP) acc1[m] += ps1 * s1[m];
      }
    } else if constexpr (FMT == FMT_Q8) {
      uint32_t dw0 = 0, dw1 = 0;
      const float ps0 = q8_prescale<KS>(B0.d, dw0);
      float ps1 = 0.0f;
      if constexpr (GATEUP) ps1 = q8_prescale<KS>(B1.d, dw1);
      f32x4_t s0[NM], s1[NM];
#pragma unroll
      for (int m = 0; m < NM; m++) s0[m] = s1[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hh = 0; hh < 3 - KS; hh++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const uint4 f0 = q8_frag(B0, hh, i, dw0);
          uint4 f1;
          if constexpr (GATEUP) f1 = q8_frag(B1, hh, i, dw1);
#pragma unroll
          for (int m = 0; m < NM; m++) {
            const uint4 av = aread(m, 4 * hh + i);
            s0[m] = mfma32(av, f0, s0[m]);
            if constexpr (GATEUP) s1[m] = mfma32(av, f1, s1[m]);
          }
          if (i == 1 || i == 3) __builtin_amdgcn_sched_barrier(0);  // bound the live fragments
        }
      }
#pragma unroll
      for (int m = 0; m < NM; m++) {
        acc0[m] += ps0 * s0[m];
        if constexpr (GATEUP) acc1[m] += ps1 * s1[m];
      }
    } else if constexpr ((FMT == FMT_Q2K || FMT == FMT_Q4K) && GATEUP) {
      // the running scale: acc in units of D (d, and for the min term dmin,
      // from the superblock's scale word)
      const uint32_t db0 = sw0 & 0xffffu, db1 = GATEUP ? sw1 & 0xffffu : 0u;
      const bool z0 = (db0 & 0x7fffu) == 0u, z1 = (db1 & 0x7fffu) == 0u;
      auto rescale = [&](f32x4_t* acc, float& D, uint32_t db, bool z) {
        if (!z) {
          const float dv = from_h(db);
          const float r = D * __builtin_amdgcn_rcpf(dv);
          D = dv;
#pragma unroll
          for (int m = 0; m < NM; m++) acc[m] *= r;
        }
      };
      rescale(acc0, D0, db0, z0);
      if constexpr (GATEUP) rescale(acc1, D1, db1, z1);
#pragma unroll
      for (int hh = 0; hh < 3 - KS; hh++) {
        uint32_t sc0 = 0, sc1 = 0;
        f16x2_t mul0 = {}, add0 = {}, mul1 = {}, add1 = {};
        Q2kConst kq0 = {}, kq1 = {};
        if constexpr (FMT == FMT_Q4K) {
          const int sbl = KS == 2 ? h : hh;
          auto consts = [&](uint32_t sc, f16x2_t& mul, f16x2_t& add) {
            const float f = (float)sc;
            mul = f16x2_t{(_Float16)f, (_Float16)(f * 0.0625f)};
            add = f16x2_t{(_Float16)(-1024.0f * f), (_Float16)(-64.0f * f)};
          };
          consts(z0 ? 0u : q4k_sc(B0, sbl), mul0, add0);
          if constexpr (GATEUP) consts(z1 ? 0u : q4k_sc(B1, sbl), mul1, add1);
        } else {
          const int hs = KS == 2 ? h : hh;
          sc0 = z0 ? 0u : B0.sc >> (16 * hs);
          if constexpr (GATEUP) sc1 = z1 ? 0u : B1.sc >> (16 * hs);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
          uint4 f0, f1;
          if constexpr (FMT == FMT_Q4K) {
            f0 = q4k_frag(word_of(B0.q[KS == 2 ? 0 : hh], i), mul0, add0);
            if constexpr (GATEUP) f1 = q4k_frag(word_of(B1.q[KS == 2 ? 0 : hh], i), mul1, add1);
          } else {
            if (i % 2 == 0) {
              kq0 = q2k_const((sc0 >> (8 * (i >> 1))) & 15u);
              if constexpr (GATEUP) kq1 = q2k_const((sc1 >> (8 * (i >> 1))) & 15u);
            }
            f0 = q2k_frag(B0, hh, i, kq0);
            if constexpr (GATEUP) f1 = q2k_frag(B1, hh, i, kq1);
          }
#pragma unroll
          for (int m = 0; m < NM; m++) {
            const uint4 av = aread(m, 4 * hh + i);
            acc0[m] = mfma32(av, f0, acc0[m]);
            if constexpr (GATEUP) acc1[m] = mfma32(av, f1, acc1[m]);
          }
          if (i == 1 || i == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (h == 0) {
        const float dm0 = from_h(sw0 >> 16) * __builtin_amdgcn_rcpf(D0);
        float dm1 = 0.0f;
        if constexpr (GATEUP) dm1 = from_h(sw1 >> 16) * __builtin_amdgcn_rcpf(D1);
        uint2 mf0, mf1;
        if constexpr (FMT == FMT_Q4K) {
          mf0 = q4k_min_frag(B0);
          if constexpr (GATEUP) mf1 = q4k_min_frag(B1);
        } else {
          mf0 = q2k_min_frag(B0);
          if constexpr (GATEUP) mf1 = q2k_min_frag(B1);
        }
        const uint16_t* ss = sS + buf * (2 * BM * 16);
#pragma unroll
        for (int m = 0; m < NM; m++) {
          const uint2 shi = *reinterpret_cast<const uint2*>(ss + (m * 16 + c16) * 16 + 4 * g4);
          const uint2 slo = *reinterpret_cast<const uint2*>(ss + BM * 16 + (m * 16 + c16) * 16 + 4 * g4);
          f32x4_t mm = mfma16(shi, mf0, f32x4_t{0.f, 0.f, 0.f, 0.f});
          mm = mfma16(slo, mf0, mm);
          acc0[m] -= dm0 * mm;
          if constexpr (GATEUP) {
            f32x4_t m1 = mfma16(shi, mf1, f32x4_t{0.f, 0.f, 0.f, 0.f});
            m1 = mfma16(slo, mf1, m1);
            acc1[m] -= dm1 * m1;
          }
        }
      }
    } else {
      f32x4_t s0[NM], s1[NM];
#pragma unroll
      for (int m = 0; m < NM; m++) s0[m] = s1[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint32_t CB = (uint32_t)c16 << 4, CS = (uint32_t)(lane & (G::SGN - 1)) << 4;
#pragma unroll
      for (int hh = 0; hh < 3 - KS; hh++) {  // halves of the lane's slice (one for KS = 2)
        uint32_t S0 = 0, S1 = 0, sc0 = 0, sc1 = 0;
        f16x2_t mul0 = {}, add0 = {}, mul1 = {}, add1 = {};
        Q2kConst kq0 = {}, kq1 = {};
        if constexpr (FMT == FMT_IQ2) {
          S0 = iq2_scale_h2(B0.w[2 * hh + 1]);
          if constexpr (GATEUP) S1 = iq2_scale_h2(B1.w[2 * hh + 1]);
        } else if constexpr (FMT == FMT_Q4K) {
          const int sbl = KS == 2 ? h : hh;  // the lane's sub-block 2*g4 + sbl
          auto consts = [&](uint32_t sc, f16x2_t& mul, f16x2_t& add) {
            const float f = (float)sc;
            mul = f16x2_t{(_Float16)f, (_Float16)(f * 0.0625f)};
            add = f16x2_t{(_Float16)(-1024.0f * f), (_Float16)(-64.0f * f)};
          };
          consts(q4k_sc(B0, sbl), mul0, add0);
          if constexpr (GATEUP) consts(q4k_sc(B1, sbl), mul1, add1);
        } else {
          const int hs = KS == 2 ? h : hh;  // scale bytes of sub-blocks 4*g4 + 2hs, + 1
          sc0 = B0.sc >> (16 * hs);
          if constexpr (GATEUP) sc1 = B1.sc >> (16 * hs);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
          uint4 f0, f1;
          if constexpr (FMT == FMT_IQ2) {
            f0 = iq2_frag<G::SGN>(B0, hh, i, S0, CB, CS, tm, sgn);
            if constexpr (GATEUP) f1 = iq2_frag<G::SGN>(B1, hh, i, S1, CB, CS, tm, sgn);
          } else if constexpr (FMT == FMT_Q4K) {
            f0 = q4k_frag(word_of(B0.q[KS == 2 ? 0 : hh], i), mul0, add0);
            if constexpr (GATEUP) f1 = q4k_frag(word_of(B1.q[KS == 2 ? 0 : hh], i), mul1, add1);
          } else {
            // low nibble of scale byte i/2
            if (i % 2 == 0) {
              kq0 = q2k_const((sc0 >> (8 * (i >> 1))) & 15u);
              if constexpr (GATEUP) kq1 = q2k_const((sc1 >> (8 * (i >> 1))) & 15u);
            }
            f0 = q2k_frag(B0, hh, i, kq0);
            if constexpr (GATEUP) f1 = q2k_frag(B1, hh, i, kq1);
          }
#pragma unroll
          for (int m = 0; m < NM; m++) {
            const uint4 av = aread(m, 4 * hh + i);
            s0[m] = mfma32(av, f0, s0[m]);
            if constexpr (GATEUP) s1[m] = mfma32(av, f1, s1[m]);
          }
          // keep the scheduler from hoisting every step's table reads (and
          // their registers) to the top: at most two steps overlap
          if (i == 1 || i == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
      // superblock epilogue: fp32 scales (and, in the first half, Q2K's min term)
      if constexpr (FMT == FMT_IQ2) {
        const float d0 = from_h(sw0), d1 = GATEUP ? from_h(sw1) : 0.0f;
#pragma unroll
        for (int m = 0; m < NM; m++) {
          acc0[m] += d0 * s0[m];
          if constexpr (GATEUP) acc1[m] += d1 * s1[m];
        }
      } else {
        const float dd0 = from_h(sw0 & 0xffffu), dmin0 = from_h(sw0 >> 16);
        float dd1 = 0.0f, dmin1 = 0.0f;
        if constexpr (GATEUP) {
          dd1 = from_h(sw1 & 0xffffu);
          dmin1 = from_h(sw1 >> 16);
        }
#pragma unroll
        for (int m = 0; m < NM; m++) {
          acc0[m] += dd0 * s0[m];
          if constexpr (GATEUP) acc1[m] += dd1 * s1[m];
        }
        if (h == 0) {
          uint2 mf0, mf1;
          if constexpr (FMT == FMT_Q4K) {
            mf0 = q4k_min_frag(B0);
            if constexpr (GATEUP) mf1 = q4k_min_frag(B1);
          } else {
            mf0 = q2k_min_frag(B0);
            if constexpr (GATEUP) mf1 = q2k_min_frag(B1);
          }
          const uint16_t* ss = sS + buf * (2 * BM * 16);
#pragma unroll
          for (int m = 0; m < NM; m++) {
            const uint2 shi = *reinterpret_cast<const uint2*>(ss + (m * 16 + c16) * 16 + 4 * g4);
            const uint2 slo = *reinterpret_cast<const uint2*>(ss + BM * 16 + (m * 16 + c16) * 16 + 4 * g4);
            f32x4_t mm = mfma16(shi, mf0, f32x4_t{0.f, 0.f, 0.f, 0.f});
            mm = mfma16(slo, mf0, mm);
            acc0[m] -= dmin0 * mm;
            if constexpr (GATEUP) {
              f32x4_t m1 = mfma16(shi, mf1, f32x4_t{0.f, 0.f, 0.f, 0.f});
              m1 = mfma16(slo, mf1, m1);
              acc1[m] -= dmin1 * m1;
            }
          }
        }
      }
    }
  };

  // End of an item (after a barrier: every wave is past the item's last
  // compute, so A buffer `freebuf` is free): the second-half waves hand their
  // partial sums to the first-half waves, which write the outputs.
  auto epilogue = [&](int j, const Item& it, int freebuf) {
    // lane-derived values re-read through an opaque copy: nothing here is
    // computed ahead of the loop and held (spilled) across it
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int wv = KS == 2 ? (int)(threadIdx.x >> 6) % GEMM_PAIRS : (int)(threadIdx.x >> 6);
    const int g4 = ln >> 4, c16 = ln & 15, lane = ln;
    float* red1 = reinterpret_cast<float*>(sA + freebuf * A_BUF);  // second matrix (gate/up)
    static_assert(NSUB * 4 * GEMM_PAIRS * 64 * 4 <= A_BUF, "partials fit an A buffer");
    if (KS == 2 && h == 1) {
#pragma unroll
      for (int m = 0; m < NSUB; m++) {
        if (m < it.nm) {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int o = ((m * 4 + r) * GEMM_PAIRS + wv) * 64 + lane;
            sRed[o] = acc0[m][r];
            if constexpr (GATEUP) red1[o] = acc1[m][r];
          }
        }
      }
    }
    if constexpr (KS == 2) __syncthreads();
    const int n = it.nt * BN + wv * 16 + c16;  // this lane's output row (B column)
    const int cl = wv * 16 + c16;              // ... inside the N tile
    if constexpr (GATEUP) {
      // Two phases around a barrier.  First h goes to LDS (both A buffers
      // are free: the next superblock's A is stored after the epilogue) and
      // each row's max|h| over the wave's 16 columns (DPP) into the row's
      // maximum for the item (an LDS atomic maximum on the fp32 bits, which
      // order like unsigned integers for non-negative values; buffer j % 2,
      // cleared during item j - 1).  Then e follows from the row maximum and
      // h is stored as fp16(h 2^-e).  (h goes through LDS rather than
      // registers so that nothing is held across the barrier.)
      constexpr int HROW = BN + 4;  // floats per row of the h tile (padded: the 4 row groups meet other banks)
      static_assert(BM * HROW * 4 == L::kHt, "the h tile's LDS");
      float* hbuf = reinterpret_cast<float*>(sA + (KS == 1 ? 0 : 2 * A_BUF));
      uint32_t* rmax = sMax + (j & 1) * BM;
      if (h == 0) {
#pragma unroll
        for (int m = 0; m < NSUB; m++) {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int o = ((m * 4 + r) * GEMM_PAIRS + wv) * 64 + lane;
            const int i = m * 16 + 4 * g4 + r;
            float hv = 0.0f;
            if (m < it.nm && i < it.rows) {
              const float v0 = (KS == 2 ? acc0[m][r] + sRed[o] : acc0[m][r]) * D0;
              const float v1 = (KS == 2 ? acc1[m][r] + red1[o] : acc1[m][r]) * D1;
              const float xs = sXs[(j % 3) * BM + i];
              hv = is_vq(FMT) ? silu(v0 * xs * vg0) * (v1 * xs * vg1) : silu(v0 * xs) * (v1 * xs);
            }
            hbuf[i * HROW + cl] = hv;
            const float mx = row16_max(fabsf(hv));
            if (c16 == 0) atomicMax(rmax + i, __float_as_uint(mx));
          }
        }
      }
      __syncthreads();
      if (tid < BM) sMax[((j + 1) & 1) * BM + tid] = 0u;  // the next item's maxima (last read by item j - 1)
      if (h == 0) {
        // wave-uniform bases (scalar registers), 32-bit lane offsets
        _Float16* hout = static_cast<_Float16*>(a.out) + (int64_t)it.p0 * a.N + it.nt * BN;
        constexpr int HC = PREFILL_HCHUNK;
        static_assert(BN % HC == 0, "whole exponent chunks per N tile");
        int8_t* eout = a.hexp_out + (int64_t)it.p0 * (a.N / HC) + it.nt * (BN / HC) + wv;
#pragma unroll
        for (int m = 0; m < NSUB; m++) {
          if (m < it.nm) {
            const uint4 rm = *reinterpret_cast<const uint4*>(rmax + m * 16 + 4 * g4);
            const uint32_t rmw[4] = {rm.x, rm.y, rm.z, rm.w};
#pragma unroll
            for (int r = 0; r < 4; r++) {
              const int i = m * 16 + 4 * g4 + r;
              if (i < it.rows) {
                const float mx = __uint_as_float(rmw[r]);
                int e = 0;
                if (mx > 0.0f && mx <= 3.4e38f) {
                  int ex;
                  frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
                  e = min(max(ex - 15, -100), 100);
                }
                const float hv = hbuf[i * HROW + cl];
                hout[i * a.N + cl] = (_Float16)(hv * __builtin_amdgcn_ldexpf(1.0f, -e));
                if (wv < BN / HC && c16 == 0) eout[i * (a.N / HC)] = (int8_t)e;  // one lane per row and chunk
              }
            }
          }
        }
      }
      __syncthreads();  // the h tile is read before the next A store overwrites it
    } else if (h == 0) {
#pragma unroll
      for (int m = 0; m < NSUB; m++) {
        if (m < it.nm) {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int o = ((m * 4 + r) * GEMM_PAIRS + wv) * 64 + lane;
            const int i = m * 16 + 4 * g4 + r;
            const float v0 = (KS == 2 ? acc0[m][r] + sRed[o] : acc0[m][r]) * D0;
            const float v = is_vq(FMT) ? v0 * sXs[(j % 3) * BM + i] * vg0 : v0 * sXs[(j % 3) * BM + i];
            if (i < it.rows) static_cast<float*>(a.out)[(int64_t)it.p0 * a.N + (i * a.N + n)] = v;
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NSUB; m++) acc0[m] = acc1[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    D0 = D1 = 1.0f;
  };

  // ---- prologue ----
  // Loads return in issue order, so A of superblock s + 1 is requested
  // before the weight loads issued in the step before it is needed: waiting
  // for it never waits for weights that are not yet due.
  Item cur = item(0), nxt = item(1);
  load_gains(cur);
  tok_issue(cur);
  tok_commit(0);
  tok_issue(nxt);
  tok_commit(1);
  tok_issue(item(2));
  __syncthreads();
  const int total = cnt * nsb;
  issueA(0, 0, cur, 0);
  if (DA == 2) {
    if (nsb > 1) issueA(1, 0, cur, 1);
    else issueA(1, 1, nxt, 0);
  }
#pragma unroll
  for (int s = 0; s < PD; s++) issueB(s, cur, s);  // PD divides nsb: all in item 0
  storeA(0, 0);
  __syncthreads();

  // ---- steady state: step s = item j, superblock sb; items end only at the
  // last step of a group of PD (PD divides nsb) ----
  int j = 0, sbase = 0;
  for (int s0 = 0; s0 < total; s0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; u++) {
      const int s = s0 + u;
      const int sb = sbase + u;
      const bool last = u == PD - 1 && sbase + PD == nsb;
      {  // A of step s + DA (item j or j + 1; past the end: no active rows)
        const int sa = sb + DA;
        if (sa >= nsb) issueA((u + DA) & 1, j + 1, nxt, sa - nsb);
        else issueA((u + DA) & 1, j, cur, sa);
      }
      {
        const uint32_t sw0 = u == 0 ? g0n.word(0) : g0c.word(u);
        const uint32_t sw1 = u == 0 ? g1n.word(0) : g1c.word(u);
        static_assert(NSUB == 2 || NSUB == 4, "sub-tile dispatch");
        if (NSUB == 4 && cur.nm == 4) compute(std::integral_constant<int, NSUB == 4 ? 4 : 2>{}, u, s & 1, sw0, sw1);
        else if (NSUB == 4 && cur.nm == 3) compute(std::integral_constant<int, NSUB == 4 ? 3 : 2>{}, u, s & 1, sw0, sw1);
        else if (cur.nm == 2) compute(std::integral_constant<int, 2>{}, u, s & 1, sw0, sw1);
        else compute(std::integral_constant<int, 1>{}, u, s & 1, sw0, sw1);
        if (u == 0) {  // the group's scales are back (its first codes were waited for)
          g0c = g0n;
          g1c = g1n;
        }
      }
      {  // weights of step s + PD (past the end: in bounds, unused)
        const int sbB = sb + PD;
        if (sbB >= nsb) issueB(u, nxt, sbB - nsb);
        else issueB(u, cur, sbB);
      }
      if (last) {
        __syncthreads();
        epilogue(j, cur, s & 1);
        cur = nxt;
        load_gains(cur);
        nxt = item(j + 2);
        tok_commit(j + 2);  // slot (j + 2) % 3 was last read for item j - 1
        tok_issue(item(j + 3));
        j++;
      }
      if (s + 1 < total) storeA((u + 1) & 1, (s + 1) & 1);
      __syncthreads();
    }
    sbase += PD;
    if (sbase == nsb) sbase = 0;
  }
}

// ---------------------------------------------------------------------------
// row normalisation of H between the two GEMMs
// ---------------------------------------------------------------------------
// The gate/up epilogue stores each PREFILL_HCHUNK-output chunk c of a row as
// fp16(h 2^-e_c).  One wave per row: e = max_c e_c; every chunk with e_c < e
// is multiplied by 2^(e_c - e) in place (exact but for fp16 subnormals,
// which lie below 2^-24 of the row's largest |h|), so the row is fp16(h 2^-e)
// throughout and the down GEMM can scale its fp32 outputs by 2^e.  Rows
// [0, n0) are H0's (routed, exponents e0), [n0, n0 + n1) H1's (shared).
__global__ __launch_bounds__(256) void hnorm_kernel(uint16_t* __restrict__ H0, const int8_t* __restrict__ e0,
                                                    float* __restrict__ sc0, int n0, uint16_t* __restrict__ H1,
                                                    const int8_t* __restrict__ e1, float* __restrict__ sc1, int n1,
                                                    int f) {
  constexpr int HC = PREFILL_HCHUNK;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n0 + n1) return;  // uniform per wave
  const bool first = row < n0;
  const int r = first ? row : row - n0;
  uint16_t* h = (first ? H0 : H1) + (int64_t)r * f;
  const int nch = f / HC;  // chunks per row (<= 128: lane l holds chunks l and l + 64)
  const int8_t* er = (first ? e0 : e1) + (int64_t)r * nch;
  const int ea = lane < nch ? er[lane] : -128, eb = lane + 64 < nch ? er[lane + 64] : -128;
  int e = max(ea, eb);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) e = max(e, __shfl_xor(e, o, 64));
  // 16-byte pieces: piece q of the row covers values 8q .. 8q + 7 (chunk q / (HC / 8))
  for (int q = lane; q < f / 8; q += 64) {
    const int c = q / (HC / 8);
    const int ca = __shfl(ea, c & 63, 64), cb = __shfl(eb, c & 63, 64);
    const int d = (c < 64 ? ca : cb) - e;
    if (d != 0) {
      const _Float16 fac = (_Float16)__builtin_amdgcn_ldexpf(1.0f, d);
      const f16x2_t ff = {fac, fac};
      uint4 v = *reinterpret_cast<const uint4*>(h + 8 * q);
      v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.x) * ff);
      v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.y) * ff);
      v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.z) * ff);
      v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, v.w) * ff);
      *reinterpret_cast<uint4*>(h + 8 * q) = v;
    }
  }
  if (lane == 0) (first ? sc0 : sc1)[r] = __builtin_amdgcn_ldexpf(1.0f, e);
}

// ---------------------------------------------------------------------------
// combine: y[t] = sum_j wt[t][j] * (g_e * Ye[pos[t*k+j]]) + ysh[t]   (fixed j order; g_e the route's
// per-channel down gains, one when none are given; ysh[t][c] times ysh_row[t] ysh_col[c] when those
// are given: the dense shared expert's powers of two)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ye, const float* __restrict__ ysh,
                                                      const float* __restrict__ ysh_row, const float* __restrict__ ysh_col,
                                                      const int32_t* __restrict__ pos, const float* __restrict__ wt,
                                                      const int32_t* __restrict__ idx, const float* __restrict__ gain,
                                                      int E, int k, int d, int n_routes, float* __restrict__ y) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; j++) {
      const int p = pos[(int64_t)t * k + j];
      if ((unsigned)p >= (unsigned)n_routes) continue;  // a route with an out-of-range expert id
      const float w = wt[(int64_t)t * k + j];
      float4 v = *reinterpret_cast<const float4*>(ye + (int64_t)p * d + 4 * c);
      if (gain) {  // per-channel down gains of the route's expert
        const int e = idx[(int64_t)t * k + j];
        if ((unsigned)e >= (unsigned)E) continue;
        const float4 g = *reinterpret_cast<const float4*>(gain + (int64_t)e * d + 4 * c);
        v = make_float4(g.x * v.x, g.y * v.y, g.z * v.z, g.w * v.w);
      }
      acc.x = __builtin_fmaf(w, v.x, acc.x);
      acc.y = __builtin_fmaf(w, v.y, acc.y);
      acc.z = __builtin_fmaf(w, v.z, acc.z);
      acc.w = __builtin_fmaf(w, v.w, acc.w);
    }
    if (ysh) {
      float4 s = *reinterpret_cast<const float4*>(ysh + (int64_t)t * d + 4 * c);
      if (ysh_col) {
        const float r = ysh_row[t];
        const float4 cs = *reinterpret_cast<const float4*>(ysh_col + 4 * c);
        s = make_float4(s.x * r * cs.x, s.y * r * cs.y, s.z * r * cs.z, s.w * r * cs.w);
      }
      acc.x += s.x;
      acc.y += s.y;
      acc.z += s.z;
      acc.w += s.w;
    }
    *reinterpret_cast<float4*>(y + (int64_t)t * d + 4 * c) = acc;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int FMT, bool GATEUP, int PD, int KS, class G>
static hipError_t run_gemm_pd(const GemmArgs& a, int m_tiles, hipStream_t s) {
  const int max_items = m_tiles * (a.N / G::bn(KS));
  const char* name = GATEUP ? (a.routed ? "prefill_gateup" : "prefill_shared_gateup")
                            : (a.routed ? "prefill_down" : "prefill_shared_down");
  using L = GemmLds<FMT, GATEUP, KS, G>;
  static_assert(L::bytes_for(MAX_EXPERTS) <= 160 * 1024, "LDS of one block");
  auto kern = gemm_kernel<FMT, GATEUP, PD, KS, G>;
  const int bytes = L::bytes_for(a.routed ? a.E : 0);
  int per_cu = 1, n_cus = 256;  // resident blocks per CU at that LDS size, CUs of the device
  hipError_t e = launch_shape((const void*)kern, G::THREADS, bytes, L::bytes_for(MAX_EXPERTS), &per_cu, &n_cus);
  if (e != hipSuccess) return e;
  int grid = per_cu * n_cus;
  grid = (grid / 8) * 8;
  if (max_items < grid) grid = ((max_items + 7) / 8) * 8;
  if (grid < 8) grid = 8;
  const int pid = prof_begin(name, s);
  QMOE_LAUNCH(kern, dim3(grid), dim3(G::THREADS), bytes, s, a);
  prof_end(pid, s);
  return hipGetLastError();
}

template <int FMT, bool GATEUP, class G>
static hipError_t run_gemm(const GemmArgs& a, int m_tiles, hipStream_t s) {
  const int nsb = a.K / 256;
  if constexpr (is_vq(FMT)) {  // whole superblocks per wave: 12 (13) bytes of indices per lane and matrix
    if (nsb % 2 == 0) return run_gemm_pd<FMT, GATEUP, 2, 1, G>(a, m_tiles, s);
    return run_gemm_pd<FMT, GATEUP, 1, 1, G>(a, m_tiles, s);
  } else if constexpr (FMT == FMT_MX4) {  // whole superblocks per wave: 32 bytes of codes per lane and matrix
    if constexpr (GATEUP) {
      return run_gemm_pd<FMT, GATEUP, 1, 1, G>(a, m_tiles, s);
    } else {
      if (nsb % 2 == 0) return run_gemm_pd<FMT, GATEUP, 2, 1, G>(a, m_tiles, s);
      return run_gemm_pd<FMT, GATEUP, 1, 1, G>(a, m_tiles, s);
    }
  } else {
    // 2-bit formats: a wave takes whole superblocks (KS = 1, 16-byte weight
    // loads).  Superblocks kept in flight (PD) per wave, at 128 VGPRs per wave
    // (16 waves per CU).
    if constexpr (FMT != FMT_Q8) {
      if constexpr (!GATEUP && FMT != FMT_Q4K) {
        if (nsb % 4 == 0) return run_gemm_pd<FMT, GATEUP, 4, 1, G>(a, m_tiles, s);
      }
      // (two Q2K or Q4K matrices hold more registers per superblock than two
      // IQ2 ones; one Q4K superblock holds twice the quant registers)
      if constexpr (FMT == FMT_Q4K) {
        if constexpr (GATEUP) {  // whole superblocks of both matrices (spill-free with the running scale)
          return run_gemm_pd<FMT, GATEUP, 1, 1, G>(a, m_tiles, s);
        } else {
          if (nsb % 2 == 0) return run_gemm_pd<FMT, GATEUP, 2, 1, G>(a, m_tiles, s);
          return run_gemm_pd<FMT, GATEUP, 1, 1, G>(a, m_tiles, s);
        }
      } else {
        // (gate/up: two superblocks in flight spill once the IQ2 fragments
        // carry their scale multiply; measured 1.62 ms against 1.90 ms with
        // two at 8 x 4096 Zipf tokens)
        if constexpr (!GATEUP) {
          if (nsb % 2 == 0) return run_gemm_pd<FMT, GATEUP, 2, 1, G>(a, m_tiles, s);
        }
        return run_gemm_pd<FMT, GATEUP, 1, 1, G>(a, m_tiles, s);
      }
    } else {
      // Q8: whole superblocks for the one-matrix down GEMM; the two-matrix
      // gate/up keeps the pair split (whole superblocks of two matrices spill)
      if constexpr (!GATEUP) {
        if (nsb % 2 == 0) return run_gemm_pd<FMT, GATEUP, 2, 1, G>(a, m_tiles, s);
        return run_gemm_pd<FMT, GATEUP, 1, 1, G>(a, m_tiles, s);
      }
      // (two superblocks in flight spill: measured 220 us against 152 us with
      // one).  With 8-wave blocks (256 VGPRs per wave) whole superblocks of
      // both matrices fit: 404 against 510 us at 8 x 4096 tokens.
      if constexpr (G::W == 8) return run_gemm_pd<FMT, GATEUP, 1, 1, G>(a, m_tiles, s);
      return run_gemm_pd<FMT, GATEUP, 1, 2, G>(a, m_tiles, s);
    }
  }
}

// (the shared expert takes IQ2XXS_L, Q2K_L or Q8_0_L only)
#define PF_SHARED_FMT_SWITCH(fmt, F, ...)                              \
  switch (fmt) {                                                       \
    case FMT_IQ2: { constexpr int F = FMT_IQ2; __VA_ARGS__; } break;   \
    case FMT_Q2K: { constexpr int F = FMT_Q2K; __VA_ARGS__; } break;   \
    default: { constexpr int F = FMT_Q8; __VA_ARGS__; } break;         \
  }

#define PF_FMT_SWITCH(fmt, F, ...)                                     \
  switch (fmt) {                                                       \
    case FMT_IQ2: { constexpr int F = FMT_IQ2; __VA_ARGS__; } break;   \
    case FMT_Q2K: { constexpr int F = FMT_Q2K; __VA_ARGS__; } break;   \
    case FMT_Q4K: { constexpr int F = FMT_Q4K; __VA_ARGS__; } break;   \
    case FMT_MX4: { constexpr int F = FMT_MX4; __VA_ARGS__; } break;   \
    case FMT_VQ12: { constexpr int F = FMT_VQ12; __VA_ARGS__; } break; \
    case FMT_VQ13: { constexpr int F = FMT_VQ13; __VA_ARGS__; } break; \
    default: { constexpr int F = FMT_Q8; __VA_ARGS__; } break;         \
  }

hipError_t launch_prefill_gemms(const PrefillLaunch& P, hipStream_t s) {
  hipError_t err = hipSuccess;
  const int n = P.T * P.k;  // (the host checked prefill_fits: A offsets stay below 2^31)
  {
    const int pid = prof_begin("prefill_x16", s);
    QMOE_LAUNCH(x16_kernel, dim3(P.T), dim3(256), 0, s, P.x, P.x_dtype, P.d, P.x16, P.xs, P.pos, P.k, P.route_xs);
    prof_end(pid, s);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // routed gate/up -> H (fp16, bucket order)
  {
    GemmArgs a{};
    a.B0 = make_qmat(P.w_gate, P.fmt_gate_up, P.E, P.f, P.d);
    a.B1 = make_qmat(P.w_up, P.fmt_gate_up, P.E, P.f, P.d);
    a.grid = P.grid;
    a.vq_cb = P.vq_cb;
    a.a16 = P.x16;
    a.a16_bytes = P.T * P.d * 2;
    a.rowxs = P.route_xs;
    a.K = P.d;
    a.N = P.f;
    a.routed = 1;
    a.E = P.E;
    a.k = P.k;
    a.offsets = P.offsets;
    a.tile_start = P.tile_start;
    a.perm = P.perm;
    a.out = P.H;
    a.hexp_out = P.Hexp;
    const int m_tiles = n / RoutedTile::BM + P.E;
    PF_FMT_SWITCH(P.fmt_gate_up, F, err = (run_gemm<F, true, RoutedTile>(a, m_tiles, s)))
    if (err != hipSuccess) return err;
  }
  // the shared expert as dense fp16 GEMMs when the workspace has their
  // buffers (a Q8 shared expert and a caller's workspace)
  const bool dense = P.has_shared && P.Wgu && shared_dense_ready(P.T, P.d, P.f, s);
  SharedDense S{};
  if (dense) {
    S.T = P.T;
    S.d = P.d;
    S.f = P.f;
    S.gate = make_qmat(P.s_gate, P.fmt_shared, 1, P.f, P.d);
    S.up = make_qmat(P.s_up, P.fmt_shared, 1, P.f, P.d);
    S.down = make_qmat(P.s_down, P.fmt_shared, 1, P.d, P.f);
    S.x16 = P.x16;
    S.xs = P.xs;
    S.w_gu = P.Wgu;
    S.w_dn = P.Wdn;
    S.colsc = P.colsc;
    S.dgu = P.Dgu;
    S.hs = static_cast<uint16_t*>(P.Hs);
    S.hsexp = P.Hsexp;
    S.ysh = P.Ysh;
    if ((err = launch_shared_dense_gateup(S, s)) != hipSuccess) return err;
  } else if (P.has_shared) {
    GemmArgs a{};
    a.B0 = make_qmat(P.s_gate, P.fmt_shared, 1, P.f, P.d);
    a.B1 = make_qmat(P.s_up, P.fmt_shared, 1, P.f, P.d);
    a.grid = P.grid;
    a.vq_cb = P.vq_cb;
    a.a16 = P.x16;
    a.a16_bytes = P.T * P.d * 2;
    a.rowxs = P.xs;
    a.K = P.d;
    a.N = P.f;
    a.routed = 0;
    a.n_rows = P.T;
    a.E = 1;
    a.k = 1;
    a.out = P.Hs;
    a.hexp_out = P.Hsexp;
    const int m_tiles = (P.T + SharedTile::BM - 1) / SharedTile::BM;
    PF_SHARED_FMT_SWITCH(P.fmt_shared, F, err = (run_gemm<F, true, SharedTile>(a, m_tiles, s)))
    if (err != hipSuccess) return err;
  }
  // every row of H and Hs to one exponent (the down GEMMs scale their outputs by it)
  {
    const int rows = n + (P.has_shared ? P.T : 0);
    const int pid = prof_begin("prefill_hnorm", s);
    QMOE_LAUNCH(hnorm_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, static_cast<uint16_t*>(P.H), (const int8_t*)P.Hexp,
                P.Hsc, n, static_cast<uint16_t*>(P.Hs), (const int8_t*)P.Hsexp, P.Hssc, P.has_shared ? P.T : 0, P.f);
    prof_end(pid, s);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // routed down -> Ye (fp32, bucket order); same M tiles as the gate/up GEMM
  {
    GemmArgs a{};
    a.B0 = make_qmat(P.w_down, P.fmt_down, P.E, P.d, P.f);
    a.grid = P.grid;
    a.vq_cb = P.vq_cb;
    a.a16 = static_cast<const uint16_t*>(P.H);
    a.a16_bytes = n * P.f * 2;
    a.K = P.f;
    a.N = P.d;
    a.routed = 1;
    a.E = P.E;
    a.k = P.k;
    a.offsets = P.offsets;
    a.tile_start = P.tile_start;
    a.perm = P.perm;
    a.out = P.Ye;
    a.row_scale = P.Hsc;
    const int m_tiles = n / RoutedTile::BM + P.E;
    PF_FMT_SWITCH(P.fmt_down, F, err = (run_gemm<F, false, RoutedTile>(a, m_tiles, s)))
    if (err != hipSuccess) return err;
  }
  if (dense) {
    if ((err = launch_shared_dense_down(S, s)) != hipSuccess) return err;
  } else if (P.has_shared) {
    GemmArgs b{};
    b.B0 = make_qmat(P.s_down, P.fmt_shared, 1, P.d, P.f);
    b.grid = P.grid;
    b.vq_cb = P.vq_cb;
    b.a16 = static_cast<const uint16_t*>(P.Hs);
    b.a16_bytes = P.T * P.f * 2;
    b.K = P.f;
    b.N = P.d;
    b.routed = 0;
    b.n_rows = P.T;
    b.E = 1;
    b.k = 1;
    b.out = P.Ysh;
    b.row_scale = P.Hssc;
    const int m_tiles2 = (P.T + SharedTile::BM - 1) / SharedTile::BM;
    PF_SHARED_FMT_SWITCH(P.fmt_shared, F, err = (run_gemm<F, false, SharedTile>(b, m_tiles2, s)))
    if (err != hipSuccess) return err;
  }
  const int pid = prof_begin("prefill_combine", s);
  QMOE_LAUNCH(combine_kernel, dim3(P.T), dim3(256), 0, s, (const float*)P.Ye, (const float*)(P.has_shared ? P.Ysh : nullptr),
              (const float*)(dense ? P.Hssc : nullptr), (const float*)(dense ? P.colsc + 2 * P.f : nullptr),
              (const int32_t*)P.pos, (const float*)P.wt, P.idx, P.down_gain, P.E, P.k, P.d, P.T * P.k, P.y);
  prof_end(pid, s);
  return hipGetLastError();
}

}  // namespace qmoe
