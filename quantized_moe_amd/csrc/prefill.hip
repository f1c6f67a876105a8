// Prefill path: grouped GEMMs over token buckets on bf16/fp16 MFMA.
//
// "YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 4.4 runs prefill
// experts on 16-bit matrix units and keeps every product exact by feeding
// codewords that convert to bf16 without rounding.  The same idea on gfx950:
// every B fragment handed to v_mfma is an exact small integer (IQ2: (2s+1) *
// grid value <= 217; Q2K: sc * q <= 45), the fp16 superblock scales are applied
// in an fp32 epilogue once per 256 inputs, and Q2K's min term is a second,
// K=16 MFMA against per-sub-block sums of the A rows.  Q8 weights (the shared
// expert) enter as an exact two-term split d*q = hi + lo.  A operands: bf16
// activations as given; fp32 activations as bf16 hi + lo (two MFMAs); the
// SwiGLU output h as fp16 (one rounding, relative 2^-11).
//
// One persistent kernel serves all four GEMMs (routed gate/up, routed down,
// shared gate/up, shared down).  A work item is (M tile of one expert's
// bucket, N tile of 128 output rows); 8 waves own 16 output rows each and all
// M sub-tiles, so each decoded B fragment feeds up to BM/16 MFMAs.  Tiles are
// read from device memory (no host round trip).  Work items are mapped so
// that all N tiles of an M tile run on one XCD and share its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace qmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum : int { AT_BF16 = 0, AT_F16 = 1 };

constexpr int GEMM_WAVES = 8;
constexpr int GEMM_THREADS = 64 * GEMM_WAVES;
constexpr int GEMM_BN = 16 * GEMM_WAVES;  // output rows per work item
constexpr int A_STRIDE = 256 + 8;         // LDS row stride of the A tile (elements)

template <int AT>
__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  if constexpr (AT == AT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

template <int AT>
__device__ __forceinline__ f32x4_t mfma16(uint2 a, uint2 b, f32x4_t c) {
  if constexpr (AT == AT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                     c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0,
                                                 0, 0);
}

// fp32 -> 16-bit value of the A/B type (round to nearest even).
template <int AT>
__device__ __forceinline__ uint32_t to16(float v) {
  if constexpr (AT == AT_BF16)
    return __builtin_bit_cast(uint16_t, (__bf16)v);
  else
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <int AT>
__device__ __forceinline__ float from16(uint32_t b) {
  if constexpr (AT == AT_BF16)
    return __uint_as_float(b << 16);
  else
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// ---------------------------------------------------------------------------
// arguments
// ---------------------------------------------------------------------------
struct GemmArgs {
  QMat B0, B1;                 // B0 = gate (or down), B1 = up (gate/up only)
  const uint8_t* grid;         // IQ2 grid [256][8]
  // A operand source
  const void* a_src;           // x (gate/up) or H (down)
  int a_dtype;                 // X_BF16 / X_F32 for x; H is always fp16
  int K;                       // inputs (d for gate/up, f for down)
  int N;                       // output rows (f for gate/up, d for down)
  // grouping
  int routed;                  // 1: buckets of a routed expert, 0: shared (identity)
  int n_rows;                  // shared: number of rows (T)
  int E, k;
  const int32_t* counts;       // routed: [E]
  const int32_t* offsets;      // routed: [E+1]
  const int32_t* tile_start;   // routed: [E+1]
  const int32_t* perm;         // routed: [T*k]
  // output
  void* out;                   // gate/up: fp16 H [rows][N]; down: fp32 [rows][N]
};

// ---------------------------------------------------------------------------
// LDS tables (built once per persistent block)
// ---------------------------------------------------------------------------
// IQ2: t1[s][row] = 8 x 16-bit (2s+1)*grid[row][p]; sgn[b7] = XOR masks for
// the 7 stored signs plus the parity sign.
template <int AT>
__device__ void build_iq2_tables(const uint8_t* grid, uint4* t1, uint4* sgn) {
  for (int e = threadIdx.x; e < 16 * 256; e += blockDim.x) {
    const int s = e >> 8, row = e & 255;
    const uint2 g = *reinterpret_cast<const uint2*>(grid + 8 * row);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t word = i < 2 ? g.x : g.y;
      const float v0 = (float)((2 * s + 1) * ((word >> (16 * (i & 1))) & 255u));
      const float v1 = (float)((2 * s + 1) * ((word >> (16 * (i & 1) + 8)) & 255u));
      w[i] = to16<AT>(v0) | (to16<AT>(v1) << 16);
    }
    t1[e] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  for (int b = threadIdx.x; b < 128; b += blockDim.x) {
    const uint32_t s8 = b | ((__popc(b) & 1u) << 7);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) w[i] = (((s8 >> (2 * i)) & 1u) << 15) | (((s8 >> (2 * i + 1)) & 1u) << 31);
    sgn[b] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Q2K: tqs[sc][byte] = 4 x 16-bit sc * q_i for the four 2-bit quants of byte.
template <int AT>
__device__ void build_q2k_table(uint2* tqs) {
  for (int e = threadIdx.x; e < 16 * 256; e += blockDim.x) {
    const int sc = e >> 8, b = e & 255;
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = to16<AT>((float)(sc * ((b >> (2 * i)) & 3)));
    tqs[e] = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
  }
}

// ---------------------------------------------------------------------------
// B operand: one lane's weight row, one superblock (256 inputs) at a time.
//
// K order inside a superblock.  MFMA sums over K, so any permutation of the
// 256 inputs applied to A and B alike gives the same product.  At k32 step q
// lane group g4 = lane / 16 takes inputs 64*g4 + 8*q .. +7 (not the natural
// 32*q + 8*g4): each lane then needs one contiguous slice of the block --
// 16 bytes of IQ2 payload or Q2K quants, 64 bytes of Q8 quants -- and every
// field index below is a compile-time constant.
// ---------------------------------------------------------------------------
template <int FMT>
struct BRegs;

template <>
struct BRegs<FMT_IQ2> {
  uint4 p;  // (A, B) words of sub-blocks 2*g4 and 2*g4 + 1
  float d;
  __device__ __forceinline__ void load(const QMat& m, int64_t row, int sb, int g4) {
    p = ld16_stream(m.p_a + (row * m.nb + sb) * 64 + 16 * g4);
    d = half_bits_to_float(reinterpret_cast<const uint16_t*>(m.p_scale)[row * m.nb + sb]);
  }
};

template <>
struct BRegs<FMT_Q2K> {
  uint4 q;      // quant bytes 16*g4 .. +15 (inputs 64*g4 .. +63)
  uint32_t sc;  // scale/min bytes of sub-blocks 4*g4 .. +3
  float d, dmin;
  __device__ __forceinline__ void load(const QMat& m, int64_t row, int sb, int g4) {
    const int64_t blk = row * m.nb + sb;
    q = ld16_stream(m.p_b + blk * 64 + 16 * g4);
    sc = *reinterpret_cast<const uint32_t*>(m.p_a + blk * 16 + 4 * g4);
    const uint32_t dm = *reinterpret_cast<const uint32_t*>(m.p_scale + blk * 4);
    d = half_bits_to_float(dm & 0xffffu);
    dmin = half_bits_to_float(dm >> 16);
  }
};

template <>
struct BRegs<FMT_Q8> {
  uint4 q[4];  // quants of blocks 2*g4 and 2*g4 + 1 of the superblock (64 bytes)
  float d[2];
  __device__ __forceinline__ void load(const QMat& m, int64_t row, int sb, int g4) {
    const int64_t blk = row * m.nb + sb * 8 + 2 * g4;
#pragma unroll
    for (int i = 0; i < 4; i++) q[i] = ld16_stream(m.p_a + blk * 32 + 16 * i);
    const uint32_t dd = *reinterpret_cast<const uint32_t*>(m.p_scale + blk * 2);
    d[0] = half_bits_to_float(dd & 0xffffu);
    d[1] = half_bits_to_float(dd >> 16);
  }
};

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;  // i is a compile-time constant
}

// Fragment of k32 step q: 8 exact integers for inputs 64*g4 + 8q .. +7.
template <int AT>
__device__ __forceinline__ uint4 iq2_frag(const BRegs<FMT_IQ2>& b, int q, const uint4* t1, const uint4* sgn) {
  const uint32_t A = q < 4 ? b.p.x : b.p.z;
  const uint32_t B = q < 4 ? b.p.y : b.p.w;
  const int i = q & 3;  // group inside the sub-block
  const uint32_t row = (A >> (8 * i)) & 255u;
  const uint32_t sg = (B >> (7 * i)) & 127u;
  const uint4 mag = t1[((B >> 28) << 8) | row];
  const uint4 sm = sgn[sg];
  return make_uint4(mag.x ^ sm.x, mag.y ^ sm.y, mag.z ^ sm.z, mag.w ^ sm.w);
}

template <int AT>
__device__ __forceinline__ uint4 q2k_frag(const BRegs<FMT_Q2K>& b, int q, const uint2* tqs) {
  const uint32_t hw = (word_of(b.q, q >> 1) >> (16 * (q & 1))) & 0xffffu;  // quant bytes 2q, 2q+1
  const uint32_t sc = (b.sc >> (8 * (q >> 1))) & 15u;                       // sub-block 4*g4 + q/2
  const uint2 lo = tqs[(sc << 8) | (hw & 255u)];
  const uint2 hi = tqs[(sc << 8) | (hw >> 8)];
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Q2K min-term B fragment (K = the 16 sub-blocks): m_j for j = 4*g4 .. +3,
// which are exactly the high nibbles of this lane's scale word.
template <int AT>
__device__ __forceinline__ uint2 q2k_min_frag(const BRegs<FMT_Q2K>& b) {
  const uint32_t w = b.sc;
  const uint32_t m0 = (w >> 4) & 15u, m1 = (w >> 12) & 15u, m2 = (w >> 20) & 15u, m3 = (w >> 28) & 15u;
  return make_uint2(to16<AT>((float)m0) | (to16<AT>((float)m1) << 16),
                    to16<AT>((float)m2) | (to16<AT>((float)m3) << 16));
}

// Q8: d*q split into two 16-bit terms hi + lo (16 significant bits for bf16,
// 22 for fp16; the exact product of an 8-bit quant and an 11-bit scale has 19).
template <int AT>
__device__ __forceinline__ void q8_frag(const BRegs<FMT_Q8>& b, int q, uint4& hi, uint4& lo) {
  const int blk = q >> 2;            // block 2*g4 + blk
  const int w0 = 2 * (q & 3);        // its dwords w0, w0 + 1
  const uint32_t w2[2] = {word_of(b.q[2 * blk + (w0 >> 2)], w0 & 3), word_of(b.q[2 * blk + ((w0 + 1) >> 2)], (w0 + 1) & 3)};
  const float d = b.d[blk];
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t word = w2[i >> 1];
    const float v0 = d * (float)(int8_t)((word >> (16 * (i & 1))) & 255u);
    const float v1 = d * (float)(int8_t)((word >> (16 * (i & 1) + 8)) & 255u);
    const uint32_t h0 = to16<AT>(v0), h1 = to16<AT>(v1);
    h[i] = h0 | (h1 << 16);
    l[i] = to16<AT>(v0 - from16<AT>(h0)) | (to16<AT>(v1 - from16<AT>(h1)) << 16);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int FMT, int AT, bool XSPLIT, bool GATEUP, int BM>
struct GemmLds {
  static constexpr int kT1 = FMT == FMT_IQ2 ? 16 * 256 * 16 + 128 * 16 : 0;
  static constexpr int kTQS = FMT == FMT_Q2K ? 16 * 256 * 8 : 0;
  static constexpr int kA = BM * A_STRIDE * 2 * (XSPLIT ? 2 : 1);
  static constexpr int kS = FMT == FMT_Q2K ? BM * 16 * 2 * 2 : 0;  // hi, lo
  static constexpr int kTok = BM * 4;
  static constexpr int kTiles = (MAX_EXPERTS + 1) * 4;
  static constexpr int bytes = kT1 + kTQS + kA + kS + kTok + kTiles;
};

template <int FMT, int AT, bool XSPLIT, bool GATEUP, int BM>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(GemmArgs a) {
  using L = GemmLds<FMT, AT, XSPLIT, GATEUP, BM>;
  extern __shared__ __align__(16) uint8_t lds[];
  uint4* t1 = reinterpret_cast<uint4*>(lds);
  uint4* sgn = t1 + 16 * 256;
  uint2* tqs = reinterpret_cast<uint2*>(lds + L::kT1);
  uint16_t* sA = reinterpret_cast<uint16_t*>(lds + L::kT1 + L::kTQS);
  uint16_t* sAlo = sA + BM * A_STRIDE;
  uint16_t* sS = reinterpret_cast<uint16_t*>(lds + L::kT1 + L::kTQS + L::kA);  // [BM][16] hi, then lo
  int* sTok = reinterpret_cast<int*>(lds + L::kT1 + L::kTQS + L::kA + L::kS);
  int* sTiles = sTok + BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;

  if constexpr (FMT == FMT_IQ2) build_iq2_tables<AT>(a.grid, t1, sgn);
  if constexpr (FMT == FMT_Q2K) build_q2k_table<AT>(tqs);
  int total_tiles;
  if (a.routed) {
    for (int i = tid; i <= a.E; i += GEMM_THREADS) sTiles[i] = a.tile_start[i];
    __syncthreads();
    total_tiles = sTiles[a.E];
  } else {
    __syncthreads();
    total_tiles = (a.n_rows + BM - 1) / BM;
  }
  const int NT = a.N / GEMM_BN;
  const int nsb = a.K / 256;

  // work-item mapping: XCD-aware when there are enough M tiles
  const int nblk = gridDim.x;
  const bool xcd_map = total_tiles >= 16 && (nblk % 8) == 0;
  const int xcd = blockIdx.x % 8, lb = blockIdx.x / 8, nbx = nblk / 8;
  const int n_items = xcd_map ? ((total_tiles - xcd + 7) / 8) * NT : total_tiles * NT;
  const int first = xcd_map ? lb : blockIdx.x;
  const int step = xcd_map ? nbx : nblk;

  for (int it = first; it < n_items; it += step) {
    const int mt = it / NT, nt = it % NT;
    const int tt = xcd_map ? xcd + 8 * mt : mt;
    // which expert / rows
    int e = 0, m0, rows, p0;
    if (a.routed) {
      int lo = 0, hi = a.E;  // largest e with tile_start[e] <= tt
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sTiles[mid] <= tt) lo = mid; else hi = mid;
      }
      // skip experts with zero tiles that share the same start
      e = lo;
      while (e + 1 < a.E && sTiles[e + 1] <= tt) e++;
      m0 = (tt - sTiles[e]) * BM;
      rows = min(BM, a.counts[e] - m0);
      p0 = a.offsets[e] + m0;
    } else {
      m0 = tt * BM;
      rows = min(BM, a.n_rows - m0);
      p0 = m0;
    }
    const int nm = (rows + 15) >> 4;  // active 16-row sub-tiles
    if (GATEUP) {
      for (int i = tid; i < rows; i += GEMM_THREADS) sTok[i] = a.routed ? a.perm[p0 + i] / a.k : p0 + i;
    }
    __syncthreads();

    const int n = nt * GEMM_BN + wave * 16 + c16;  // this lane's output row (B column)
    const int64_t brow = (int64_t)e * a.B0.rows + n;

    f32x4_t acc0[BM / 16], acc1[BM / 16], sb0[BM / 16], sb1[BM / 16];
#pragma unroll
    for (int m = 0; m < BM / 16; m++) acc0[m] = acc1[m] = sb0[m] = sb1[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int sb = 0; sb < nsb; sb++) {
      // ---- stage the A tile (rows x 256 inputs) into LDS ----
      if constexpr (GATEUP) {
        if constexpr (XSPLIT) {
          const float* x = static_cast<const float*>(a.a_src);
          for (int s = tid; s < rows * 64; s += GEMM_THREADS) {
            const int i = s >> 6, c = s & 63;
            const float4 v = *reinterpret_cast<const float4*>(x + (int64_t)sTok[i] * a.K + sb * 256 + 4 * c);
            const float f[4] = {v.x, v.y, v.z, v.w};
            uint32_t h[4], l[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
              h[u] = to16<AT>(f[u]);
              l[u] = to16<AT>(f[u] - from16<AT>(h[u]));
            }
            *reinterpret_cast<uint2*>(sA + i * A_STRIDE + 4 * c) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            *reinterpret_cast<uint2*>(sAlo + i * A_STRIDE + 4 * c) =
                make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
          }
        } else {
          const uint16_t* x = static_cast<const uint16_t*>(a.a_src);
          for (int s = tid; s < rows * 32; s += GEMM_THREADS) {
            const int i = s >> 5, c = s & 31;
            *reinterpret_cast<uint4*>(sA + i * A_STRIDE + 8 * c) =
                *reinterpret_cast<const uint4*>(x + (int64_t)sTok[i] * a.K + sb * 256 + 8 * c);
          }
        }
      } else {
        const uint16_t* h = static_cast<const uint16_t*>(a.a_src);
        for (int s = tid; s < rows * 32; s += GEMM_THREADS) {
          const int i = s >> 5, c = s & 31;
          *reinterpret_cast<uint4*>(sA + i * A_STRIDE + 8 * c) =
              *reinterpret_cast<const uint4*>(h + (int64_t)(p0 + i) * a.K + sb * 256 + 8 * c);
        }
      }
      // ---- B registers of this superblock ----
      BRegs<FMT> b0, b1;
      b0.load(a.B0, brow, sb, g4);
      if constexpr (GATEUP) b1.load(a.B1, brow, sb, g4);
      __syncthreads();
      // ---- Q2K min term: per-sub-block sums of the A rows (hi + lo) ----
      if constexpr (FMT == FMT_Q2K) {
        for (int s = tid; s < rows * 16; s += GEMM_THREADS) {
          const int i = s >> 4, j = s & 15;
          float sum = 0.0f;
#pragma unroll
          for (int u = 0; u < 16; u++) {
            sum += from16<AT>(sA[i * A_STRIDE + 16 * j + u]);
            if constexpr (XSPLIT) sum += from16<AT>(sAlo[i * A_STRIDE + 16 * j + u]);
          }
          const uint32_t sh = to16<AT>(sum);
          sS[i * 16 + j] = (uint16_t)sh;
          sS[BM * 16 + i * 16 + j] = (uint16_t)to16<AT>(sum - from16<AT>(sh));
        }
        __syncthreads();
      }
      // ---- 8 k32 steps ----
#pragma unroll
      for (int q = 0; q < 8; q++) {
        uint4 f0, f1, f0l, f1l;
        if constexpr (FMT == FMT_IQ2) {
          f0 = iq2_frag<AT>(b0, q, t1, sgn);
          if constexpr (GATEUP) f1 = iq2_frag<AT>(b1, q, t1, sgn);
        } else if constexpr (FMT == FMT_Q2K) {
          f0 = q2k_frag<AT>(b0, q, tqs);
          if constexpr (GATEUP) f1 = q2k_frag<AT>(b1, q, tqs);
        } else {
          q8_frag<AT>(b0, q, f0, f0l);
          if constexpr (GATEUP) q8_frag<AT>(b1, q, f1, f1l);
        }
#pragma unroll
        for (int m = 0; m < BM / 16; m++) {
          if (m < nm) {
            // inputs 64*g4 + 8q .. +7 (the K order of the B fragments)
            const uint4 av = *reinterpret_cast<const uint4*>(sA + (m * 16 + c16) * A_STRIDE + 64 * g4 + 8 * q);
            uint4 avl;
            if constexpr (XSPLIT) avl = *reinterpret_cast<const uint4*>(sAlo + (m * 16 + c16) * A_STRIDE + 64 * g4 + 8 * q);
            if constexpr (FMT == FMT_Q8) {
              acc0[m] = mfma32<AT>(av, f0, acc0[m]);
              acc0[m] = mfma32<AT>(av, f0l, acc0[m]);
              if constexpr (XSPLIT) acc0[m] = mfma32<AT>(avl, f0, acc0[m]);
              if constexpr (GATEUP) {
                acc1[m] = mfma32<AT>(av, f1, acc1[m]);
                acc1[m] = mfma32<AT>(av, f1l, acc1[m]);
                if constexpr (XSPLIT) acc1[m] = mfma32<AT>(avl, f1, acc1[m]);
              }
            } else {
              sb0[m] = mfma32<AT>(av, f0, sb0[m]);
              if constexpr (XSPLIT) sb0[m] = mfma32<AT>(avl, f0, sb0[m]);
              if constexpr (GATEUP) {
                sb1[m] = mfma32<AT>(av, f1, sb1[m]);
                if constexpr (XSPLIT) sb1[m] = mfma32<AT>(avl, f1, sb1[m]);
              }
            }
          }
        }
      }
      // ---- superblock epilogue: fp32 scales ----
      if constexpr (FMT == FMT_IQ2) {
#pragma unroll
        for (int m = 0; m < BM / 16; m++) {
          if (m < nm) {
            acc0[m] += b0.d * sb0[m];
            sb0[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (GATEUP) {
              acc1[m] += b1.d * sb1[m];
              sb1[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
      } else if constexpr (FMT == FMT_Q2K) {
        const uint2 mf0 = q2k_min_frag<AT>(b0);
        uint2 mf1;
        if constexpr (GATEUP) mf1 = q2k_min_frag<AT>(b1);
#pragma unroll
        for (int m = 0; m < BM / 16; m++) {
          if (m < nm) {
            const uint2 shi = *reinterpret_cast<const uint2*>(sS + (m * 16 + c16) * 16 + 4 * g4);
            const uint2 slo = *reinterpret_cast<const uint2*>(sS + BM * 16 + (m * 16 + c16) * 16 + 4 * g4);
            f32x4_t mm = mfma16<AT>(shi, mf0, f32x4_t{0.f, 0.f, 0.f, 0.f});
            mm = mfma16<AT>(slo, mf0, mm);
            acc0[m] += b0.d * sb0[m] - b0.dmin * mm;
            sb0[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (GATEUP) {
              f32x4_t m1 = mfma16<AT>(shi, mf1, f32x4_t{0.f, 0.f, 0.f, 0.f});
              m1 = mfma16<AT>(slo, mf1, m1);
              acc1[m] += b1.d * sb1[m] - b1.dmin * m1;
              sb1[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
      }
      __syncthreads();  // A tile is overwritten by the next superblock
    }

    // ---- output ----
#pragma unroll
    for (int m = 0; m < BM / 16; m++) {
      if (m < nm) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int i = m * 16 + 4 * g4 + r;
          if (i < rows) {
            if constexpr (GATEUP) {
              const float h = silu(acc0[m][r]) * acc1[m][r];
              static_cast<_Float16*>(a.out)[(int64_t)(p0 + i) * a.N + n] = (_Float16)h;
            } else {
              static_cast<float*>(a.out)[(int64_t)(p0 + i) * a.N + n] = acc0[m][r];
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine: y[t] = sum_j wt[t][j] * Ye[pos[t*k+j]] + ysh[t]   (fixed j order)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ ye, const float* __restrict__ ysh,
                                                      const int32_t* __restrict__ pos, const float* __restrict__ wt,
                                                      int k, int d, int n_routes, float* __restrict__ y) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; j++) {
      const int p = pos[(int64_t)t * k + j];
      if ((unsigned)p >= (unsigned)n_routes) continue;  // a route with an out-of-range expert id
      const float w = wt[(int64_t)t * k + j];
      const float4 v = *reinterpret_cast<const float4*>(ye + (int64_t)p * d + 4 * c);
      acc.x = __builtin_fmaf(w, v.x, acc.x);
      acc.y = __builtin_fmaf(w, v.y, acc.y);
      acc.z = __builtin_fmaf(w, v.z, acc.z);
      acc.w = __builtin_fmaf(w, v.w, acc.w);
    }
    if (ysh) {
      const float4 s = *reinterpret_cast<const float4*>(ysh + (int64_t)t * d + 4 * c);
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
static int g_num_cus = 0;

static int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

template <int FMT, int AT, bool XSPLIT, bool GATEUP, int BM>
static hipError_t run_gemm(const GemmArgs& a, int max_items, hipStream_t s) {
  const char* name = GATEUP ? (a.routed ? "prefill_gateup" : "prefill_shared_gateup")
                            : (a.routed ? "prefill_down" : "prefill_shared_down");
  using L = GemmLds<FMT, AT, XSPLIT, GATEUP, BM>;
  auto kern = gemm_kernel<FMT, AT, XSPLIT, GATEUP, BM>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int grid = num_cus();
  grid = (grid / 8) * 8;
  if (grid < 8) grid = 8;
  if (max_items < grid) grid = ((max_items + 7) / 8) * 8;
  if (grid < 8) grid = 8;
  const int pid = prof_begin(name, s);
  kern<<<dim3(grid), dim3(GEMM_THREADS), L::bytes, s>>>(a);
  prof_end(pid, s);
  return hipGetLastError();
}

#define PF_FMT_SWITCH(fmt, F, ...)                                     \
  switch (fmt) {                                                       \
    case FMT_IQ2: { constexpr int F = FMT_IQ2; __VA_ARGS__; } break;   \
    case FMT_Q2K: { constexpr int F = FMT_Q2K; __VA_ARGS__; } break;   \
    default: { constexpr int F = FMT_Q8; __VA_ARGS__; } break;         \
  }

hipError_t launch_prefill_gemms(const PrefillLaunch& P, hipStream_t s) {
  hipError_t err = hipSuccess;
  const int n = P.T * P.k;
  // routed gate/up -> H (fp16, bucket order)
  {
    GemmArgs a{};
    a.B0 = make_qmat(P.w_gate, P.fmt_gate_up, P.E, P.f, P.d);
    a.B1 = make_qmat(P.w_up, P.fmt_gate_up, P.E, P.f, P.d);
    a.grid = P.grid;
    a.a_src = P.x;
    a.a_dtype = P.x_dtype;
    a.K = P.d;
    a.N = P.f;
    a.routed = 1;
    a.E = P.E;
    a.k = P.k;
    a.counts = P.counts;
    a.offsets = P.offsets;
    a.tile_start = P.tile_start;
    a.perm = P.perm;
    a.out = P.H;
    if (P.x_dtype == X_BF16) {
      const int max_items = (n / PREFILL_BM + P.E) * (P.f / GEMM_BN);
      PF_FMT_SWITCH(P.fmt_gate_up, F, err = (run_gemm<F, AT_BF16, false, true, PREFILL_BM>(a, max_items, s)))
    } else {
      const int max_items = (n / PREFILL_BM_SPLIT + P.E) * (P.f / GEMM_BN);
      PF_FMT_SWITCH(P.fmt_gate_up, F, err = (run_gemm<F, AT_BF16, true, true, PREFILL_BM_SPLIT>(a, max_items, s)))
    }
    if (err != hipSuccess) return err;
  }
  // routed down -> Ye (fp32, bucket order)
  {
    GemmArgs a{};
    a.B0 = make_qmat(P.w_down, P.fmt_down, P.E, P.d, P.f);
    a.grid = P.grid;
    a.a_src = P.H;
    a.a_dtype = X_F32;
    a.K = P.f;
    a.N = P.d;
    a.routed = 1;
    a.E = P.E;
    a.k = P.k;
    a.counts = P.counts;
    a.offsets = P.offsets;
    a.tile_start = P.tile_start;
    a.perm = P.perm;
    a.out = P.Ye;
    // same M tiles as the gate/up GEMM (the bucket tile schedule is shared)
    if (P.x_dtype == X_BF16) {
      const int max_items = (n / PREFILL_BM + P.E) * (P.d / GEMM_BN);
      PF_FMT_SWITCH(P.fmt_down, F, err = (run_gemm<F, AT_F16, false, false, PREFILL_BM>(a, max_items, s)))
    } else {
      const int max_items = (n / PREFILL_BM_SPLIT + P.E) * (P.d / GEMM_BN);
      PF_FMT_SWITCH(P.fmt_down, F, err = (run_gemm<F, AT_F16, false, false, PREFILL_BM_SPLIT>(a, max_items, s)))
    }
    if (err != hipSuccess) return err;
  }
  if (P.has_shared) {
    GemmArgs a{};
    a.B0 = make_qmat(P.s_gate, P.fmt_shared, 1, P.f, P.d);
    a.B1 = make_qmat(P.s_up, P.fmt_shared, 1, P.f, P.d);
    a.grid = P.grid;
    a.a_src = P.x;
    a.a_dtype = P.x_dtype;
    a.K = P.d;
    a.N = P.f;
    a.routed = 0;
    a.n_rows = P.T;
    a.E = 1;
    a.k = 1;
    a.out = P.Hs;
    if (P.x_dtype == X_BF16) {
      const int max_items = ((P.T + PREFILL_BM - 1) / PREFILL_BM) * (P.f / GEMM_BN);
      PF_FMT_SWITCH(P.fmt_shared, F, err = (run_gemm<F, AT_BF16, false, true, PREFILL_BM>(a, max_items, s)))
    } else {
      const int max_items = ((P.T + PREFILL_BM_SPLIT - 1) / PREFILL_BM_SPLIT) * (P.f / GEMM_BN);
      PF_FMT_SWITCH(P.fmt_shared, F, err = (run_gemm<F, AT_BF16, true, true, PREFILL_BM_SPLIT>(a, max_items, s)))
    }
    if (err != hipSuccess) return err;
    GemmArgs b{};
    b.B0 = make_qmat(P.s_down, P.fmt_shared, 1, P.d, P.f);
    b.grid = P.grid;
    b.a_src = P.Hs;
    b.a_dtype = X_F32;
    b.K = P.f;
    b.N = P.d;
    b.routed = 0;
    b.n_rows = P.T;
    b.E = 1;
    b.k = 1;
    b.out = P.Ysh;
    const int max_items2 = ((P.T + PREFILL_BM - 1) / PREFILL_BM) * (P.d / GEMM_BN);
    PF_FMT_SWITCH(P.fmt_shared, F, err = (run_gemm<F, AT_F16, false, false, PREFILL_BM>(b, max_items2, s)))
    if (err != hipSuccess) return err;
  }
  const int pid = prof_begin("prefill_combine", s);
  combine_kernel<<<dim3(P.T), 256, 0, s>>>(P.Ye, P.has_shared ? P.Ysh : nullptr, P.pos, P.wt, P.k, P.d, P.T * P.k,
                                           P.y);
  prof_end(pid, s);
  return hipGetLastError();
}

}  // namespace qmoe
