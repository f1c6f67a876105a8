// Decode path: streaming GEMVs over the selected experts' packed weights.
//
// Decode reads every selected weight once per token and is bound by HBM
// bytes ("YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 4.4:
// decoding is memory-bound; the engine's expert kernel streams whole cache
// lines and decodes codes in registers).  Here every lane owns 64
// consecutive inputs of a row (one 16-byte chunk of 2-bit codes, or 64 bytes
// of int8 codes), keeps the matching 64 activations in registers for the
// whole wave, and decodes its chunk in registers; LPR = K/64 lanes share a
// row and reduce with a fixed butterfly.
//
// Three launches per layer:
//   K1  router logits (all experts) and the shared expert's gate/up+SwiGLU
//       (both depend only on x);
//   K2  routed gate/up + SwiGLU; with routing fused, each block first runs
//       the exact top-k of its token from the logits K1 wrote;
//   K3  down projections of the routed experts and the shared expert, and
//       the fixed-order combine y = sum_j wt_j ye_j + ysh (the per-layer sum
//       of the YoungAi page, section 4.2).
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace qmoe {

// ---------------------------------------------------------------------------
// chunk decoders: partial dot of one lane's 64 weights with its 64 inputs
// ---------------------------------------------------------------------------
// IQ2: 16-byte chunk c of a row = sub-blocks 2(c%4), 2(c%4)+1 of superblock
// c/4, i.e. words A0 B0 A1 B1.  w = d (2s+1) grid[row][p] sign.
__device__ __forceinline__ float iq2_chunk_dot(const QMat& m, int64_t row, int c, const float* xs,
                                               const uint32_t* __restrict__ grid2) {
  const uint4 v = ld16_stream(m.p_a + (row * m.nb) * 64 + (int64_t)c * 16);
  const float d = half_bits_to_float(reinterpret_cast<const uint16_t*>(m.p_scale)[row * m.nb + c / 4]);
  float acc = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const uint32_t A = h ? v.z : v.x;
    const uint32_t B = h ? v.w : v.y;
    float sb = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t gr = (A >> (8 * i)) & 255u;
      const uint32_t sg = (B >> (7 * i)) & 127u;
      const uint32_t s8 = sg | ((__popc(sg) & 1u) << 7);
      const uint32_t lo = grid2[2 * gr], hi = grid2[2 * gr + 1];
#pragma unroll
      for (int p = 0; p < 8; p++) {
        const uint32_t word = p < 4 ? lo : hi;
        float mag = (float)((word >> (8 * (p & 3))) & 255u);
        mag = __uint_as_float(__float_as_uint(mag) ^ (((s8 >> p) & 1u) << 31));
        sb = __builtin_fmaf(mag, xs[32 * h + 8 * i + p], sb);
      }
    }
    acc = __builtin_fmaf((float)(2 * (B >> 28) + 1), sb, acc);
  }
  return d * acc;
}

// Q2K: chunk c = 64 quants (sub-blocks 4(c%4) .. +3 of superblock c/4).
// sum w x = d sum_u sc_u (sum q x) - dmin sum_u m_u (sum x).
__device__ __forceinline__ float q2k_chunk_dot(const QMat& m, int64_t row, int c, const float* xs) {
  const uint4 q = ld16_stream(m.p_b + (row * m.nb) * 64 + (int64_t)c * 16);
  const uint32_t sc4 = *reinterpret_cast<const uint32_t*>(m.p_a + (row * m.nb) * 16 + (int64_t)c * 4);
  const uint32_t dm = *reinterpret_cast<const uint32_t*>(m.p_scale + (row * m.nb + c / 4) * 4);
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  float accd = 0.0f, accm = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    float qs = 0.0f, xsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const float qi = (float)((qw[u] >> (2 * i)) & 3u);
      qs = __builtin_fmaf(qi, xs[16 * u + i], qs);
      xsum += xs[16 * u + i];
    }
    const uint32_t b = (sc4 >> (8 * u)) & 255u;
    accd = __builtin_fmaf((float)(b & 15u), qs, accd);
    accm = __builtin_fmaf((float)(b >> 4), xsum, accm);
  }
  return half_bits_to_float(dm & 0xffffu) * accd - half_bits_to_float(dm >> 16) * accm;
}

// Q8: chunk c = 64 int8 quants = blocks 2c, 2c+1 (two fp16 scales).
__device__ __forceinline__ float q8_chunk_dot(const QMat& m, int64_t row, int c, const float* xs) {
  const uint8_t* q = m.p_a + row * (int64_t)m.K + (int64_t)c * 64;
  const uint32_t dd = *reinterpret_cast<const uint32_t*>(m.p_scale + (row * m.nb + 2 * c) * 2);
  float acc[2] = {0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint4 v = ld16_stream(q + 16 * j);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int b = 0; b < 16; b++) {
      const float qi = (float)(int8_t)((w[b >> 2] >> (8 * (b & 3))) & 255u);
      acc[j >> 1] = __builtin_fmaf(qi, xs[16 * j + b], acc[j >> 1]);
    }
  }
  return half_bits_to_float(dd & 0xffffu) * acc[0] + half_bits_to_float(dd >> 16) * acc[1];
}

template <int FMT>
__device__ __forceinline__ float chunk_dot(const QMat& m, int64_t row, int c, const float* xs,
                                           const uint32_t* grid2) {
  if (FMT == FMT_IQ2) return iq2_chunk_dot(m, row, c, xs, grid2);
  if (FMT == FMT_Q2K) return q2k_chunk_dot(m, row, c, xs);
  return q8_chunk_dot(m, row, c, xs);
}

// Load the lane's 64 * CPL inputs (chunks c, c + 64, ...) of an fp32 or bf16
// vector.
template <int CPL>
__device__ __forceinline__ void load_slice(const void* v, int v_dtype, int64_t off, int c, int LPR, float* xs) {
#pragma unroll
  for (int k = 0; k < CPL; k++) {
    const int cc = c + LPR * k;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      float4 f;
      if (v_dtype == X_BF16) {
        const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(v) + off + 64 * cc + 4 * j);
        f = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u), __uint_as_float(b.y << 16),
                        __uint_as_float(b.y & 0xffff0000u));
      } else {
        f = *reinterpret_cast<const float4*>(static_cast<const float*>(v) + off + 64 * cc + 4 * j);
      }
      xs[64 * k + 4 * j + 0] = f.x;
      xs[64 * k + 4 * j + 1] = f.y;
      xs[64 * k + 4 * j + 2] = f.z;
      xs[64 * k + 4 * j + 3] = f.w;
    }
  }
}

// Sum over the LPR lanes that share a row (butterfly; fixed order).
__device__ __forceinline__ float row_reduce(float v, int LPR) {
  for (int off = LPR >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void load_grid_lds(const uint8_t* grid, uint32_t* grid2) {
  if (grid)
    for (int i = threadIdx.x; i < 512; i += blockDim.x) grid2[i] = reinterpret_cast<const uint32_t*>(grid)[i];
  __syncthreads();
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU rows [r_begin, r_end) of one expert for one token, by one
// wave.  h[n] = silu(G_n . x) * (U_n . x).
// ---------------------------------------------------------------------------
template <int FMT, int CPL>
__device__ __forceinline__ void gateup_wave(const QMat& G, const QMat& U, int expert, const void* x, int x_dtype,
                                            int64_t x_off, int r_begin, int r_end, float* __restrict__ h,
                                            const uint32_t* grid2) {
  const int lane = threadIdx.x & 63;
  const int LPR = (G.K / 64) / CPL;  // lanes per row
  const int RPS = 64 / LPR;          // rows per step
  const int sub = lane / LPR, c = lane % LPR;
  float xs[64 * CPL];
  load_slice<CPL>(x, x_dtype, x_off, c, LPR, xs);
  const int64_t rbase = (int64_t)expert * G.rows;
  for (int r0 = r_begin; r0 < r_end; r0 += RPS) {
    const int n = r0 + sub;
    float g = 0.0f, u = 0.0f;
    if (n < r_end) {
#pragma unroll
      for (int k = 0; k < CPL; k++) {
        g += chunk_dot<FMT>(G, rbase + n, c + LPR * k, xs + 64 * k, grid2);
        u += chunk_dot<FMT>(U, rbase + n, c + LPR * k, xs + 64 * k, grid2);
      }
    }
    g = row_reduce(g, LPR);
    u = row_reduce(u, LPR);
    if (c == 0 && n < r_end) h[n] = silu(g) * u;
  }
}

// ---------------------------------------------------------------------------
// K1: router logits (blocks [0, n_router_blocks)) and shared gate/up
// (remaining blocks: one per (row tile, token)).
// ---------------------------------------------------------------------------
struct DecodeArgs {
  QMat gate, up, down;           // routed experts
  QMat s_gate, s_up, s_down;     // shared expert
  const uint8_t* grid;
  const float* w_router;
  int E, d, f, k, T;
  int has_shared;
  const void* x;
  int x_dtype;
  float* z;                      // [T][E] logits (fused routing)
  int32_t* idx;                  // [T][k] routes (workspace copy)
  float* wt;                     // [T][k]
  int32_t* idx_out;              // nullable user copies
  float* wt_out;
  float* h;                      // [T*k + T][f]
  float* y;                      // [T][d]
  int fused_topk;
};

constexpr int GU_ROWS_PER_WAVE = 8;
constexpr int GU_ROWS_PER_BLOCK = 4 * GU_ROWS_PER_WAVE;
constexpr int DN_ROWS_PER_BLOCK = 16;
constexpr int DN_WAVES = 8;

template <int FMT, int CPL>
__global__ __launch_bounds__(256) void decode_k1_kernel(DecodeArgs a, int n_router_blocks) {
  __shared__ uint32_t grid2[512];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((int)blockIdx.x < n_router_blocks) {
    // router: wave per expert, tokens in a loop (fixed fp32 order, route.hip)
    const int e = blockIdx.x * 4 + wave;
    if (e >= a.E) return;
    const int chunks = a.d / 256;
    for (int t = 0; t < a.T; t++) {
      float p = 0.0f;
      for (int m = 0; m < chunks; m++) {
        const int cc = lane + 64 * m;
        const float4 w = *reinterpret_cast<const float4*>(a.w_router + (int64_t)e * a.d + 4 * cc);
        float4 xv;
        if (a.x_dtype == X_BF16) {
          const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.x) + (int64_t)t * a.d + 4 * cc);
          xv = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u), __uint_as_float(b.y << 16),
                           __uint_as_float(b.y & 0xffff0000u));
        } else {
          xv = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + (int64_t)t * a.d + 4 * cc);
        }
        p = __builtin_fmaf(xv.x, w.x, p);
        p = __builtin_fmaf(xv.y, w.y, p);
        p = __builtin_fmaf(xv.z, w.z, p);
        p = __builtin_fmaf(xv.w, w.w, p);
      }
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) p = p + __shfl_down(p, s, 64);
      if (lane == 0) a.z[(int64_t)t * a.E + e] = p;
    }
    return;
  }
  load_grid_lds(a.grid, grid2);
  const int b = blockIdx.x - n_router_blocks;
  const int tiles = a.f / GU_ROWS_PER_BLOCK;
  const int tile = b % tiles, t = b / tiles;
  const int r0 = tile * GU_ROWS_PER_BLOCK + wave * GU_ROWS_PER_WAVE;
  gateup_wave<FMT, CPL>(a.s_gate, a.s_up, 0, a.x, a.x_dtype, (int64_t)t * a.d, r0, r0 + GU_ROWS_PER_WAVE,
                        a.h + (int64_t)(a.T * a.k + t) * a.f, grid2);
}

// K2: routed gate/up.  grid = (f / GU_ROWS_PER_BLOCK, T * k).
template <int FMT, int CPL>
__global__ __launch_bounds__(256) void decode_k2_kernel(DecodeArgs a) {
  __shared__ uint32_t grid2[512];
  __shared__ int s_expert;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int route = blockIdx.y, t = route / a.k, j = route % a.k;
  if (a.fused_topk) {
    if (wave == 0) {
      int sel[TOPK_MAX_K];
      float zs[TOPK_MAX_K];
      wave_topk(a.z + (int64_t)t * a.E, a.E, a.k, sel, zs);
      int ej = sel[0];
#pragma unroll
      for (int q = 1; q < TOPK_MAX_K; q++)
        if (q == j) ej = sel[q];
      if (lane == 0) {
        s_expert = ej;
        if (blockIdx.x == 0 && j == 0) {
          float w[TOPK_MAX_K];
          topk_weights(zs, a.k, w);
#pragma unroll
          for (int q = 0; q < TOPK_MAX_K; q++) {
            if (q >= a.k) continue;
            a.idx[(int64_t)t * a.k + q] = sel[q];
            a.wt[(int64_t)t * a.k + q] = w[q];
            if (a.idx_out) a.idx_out[(int64_t)t * a.k + q] = sel[q];
            if (a.wt_out) a.wt_out[(int64_t)t * a.k + q] = w[q];
          }
        }
      }
    }
  } else if (threadIdx.x == 0) {
    s_expert = a.idx[route];
  }
  load_grid_lds(a.grid, grid2);  // includes the barrier that publishes s_expert
  const int e = s_expert;
  const int r0 = blockIdx.x * GU_ROWS_PER_BLOCK + wave * GU_ROWS_PER_WAVE;
  if ((unsigned)e >= (unsigned)a.E) {  // caller route with an out-of-range expert id: contributes zero
    if (lane < GU_ROWS_PER_WAVE) a.h[(int64_t)route * a.f + r0 + lane] = 0.0f;
    return;
  }
  gateup_wave<FMT, CPL>(a.gate, a.up, e, a.x, a.x_dtype, (int64_t)t * a.d, r0, r0 + GU_ROWS_PER_WAVE,
                        a.h + (int64_t)route * a.f, grid2);
}

// K3: down + combine.  grid = (d / DN_ROWS_PER_BLOCK, T); 8 waves.  Tasks:
// routed route j (all rows of the tile), then the shared expert in two row
// halves.  Each task's row dots go to LDS; then y = sum_j wt_j ye_j + ysh in
// that fixed order.
template <int FMT_R, int FMT_S, int CPL>
__global__ __launch_bounds__(512) void decode_k3_kernel(DecodeArgs a) {
  __shared__ uint32_t grid2[512];
  __shared__ float ye[(TOPK_MAX_K + 1) * DN_ROWS_PER_BLOCK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.y;
  const int row0 = blockIdx.x * DN_ROWS_PER_BLOCK;
  load_grid_lds(a.grid, grid2);
  const int n_tasks = a.k + (a.has_shared ? 2 : 0);
  for (int task = wave; task < n_tasks; task += DN_WAVES) {
    const bool shared = task >= a.k;
    const int src = shared ? a.T * a.k + t : t * a.k + task;
    int e = shared ? 0 : a.idx[src];
    if ((unsigned)e >= (unsigned)a.E) e = -1;  // out-of-range caller route: contributes zero
    const QMat& D = shared ? a.s_down : a.down;
    const int LPR = (D.K / 64) / CPL;
    const int RPS = 64 / LPR;
    const int sub = lane / LPR, c = lane % LPR;
    int rb = 0, re = DN_ROWS_PER_BLOCK;
    if (shared) {
      rb = (task - a.k) * (DN_ROWS_PER_BLOCK / 2);
      re = rb + DN_ROWS_PER_BLOCK / 2;
    }
    float xs[64 * CPL];
    load_slice<CPL>(a.h, X_F32, (int64_t)src * a.f, c, LPR, xs);
    const int64_t rbase = (int64_t)e * D.rows + row0;
    for (int r = rb; r < re; r += RPS) {
      const int n = r + sub;
      float v = 0.0f;
      if (n < re && e >= 0) {
#pragma unroll
        for (int k = 0; k < CPL; k++) {
          if (shared)
            v += chunk_dot<FMT_S>(D, rbase + n, c + LPR * k, xs + 64 * k, grid2);
          else
            v += chunk_dot<FMT_R>(D, rbase + n, c + LPR * k, xs + 64 * k, grid2);
        }
      }
      v = row_reduce(v, LPR);
      if (c == 0 && n < re) ye[(shared ? a.k : task) * DN_ROWS_PER_BLOCK + n] = v;
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
template <int FMT, int CPL>
static void k1(const DecodeArgs& a, int nrb, int nsb, hipStream_t s) {
  const int pid = prof_begin("decode_router_shared_gateup", s);
  decode_k1_kernel<FMT, CPL><<<dim3(nrb + nsb), 256, 0, s>>>(a, nrb);
  prof_end(pid, s);
}
template <int FMT, int CPL>
static void k2(const DecodeArgs& a, hipStream_t s) {
  const int pid = prof_begin("decode_gateup", s);
  decode_k2_kernel<FMT, CPL><<<dim3(a.f / GU_ROWS_PER_BLOCK, a.T * a.k), 256, 0, s>>>(a);
  prof_end(pid, s);
}
template <int FR, int FS, int CPL>
static void k3(const DecodeArgs& a, hipStream_t s) {
  const int pid = prof_begin("decode_down_combine", s);
  decode_k3_kernel<FR, FS, CPL><<<dim3(a.d / DN_ROWS_PER_BLOCK, a.T), 512, 0, s>>>(a);
  prof_end(pid, s);
}

#define FMT_SWITCH(fmt, F, ...)                   \
  switch (fmt) {                                  \
    case FMT_IQ2: { constexpr int F = FMT_IQ2; __VA_ARGS__; } break; \
    case FMT_Q2K: { constexpr int F = FMT_Q2K; __VA_ARGS__; } break; \
    default: { constexpr int F = FMT_Q8; __VA_ARGS__; } break;       \
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
  a.h = L.h; a.y = L.y;
  a.fused_topk = L.fused_topk;
  if (L.T == 0) return hipSuccess;
  const int cpl_d = L.d > 4096 ? 2 : 1;  // chunks per lane of the d-wide rows (gate/up)
  const int cpl_f = L.f > 4096 ? 2 : 1;  // of the f-wide rows (down)
  const int nrb = L.fused_topk ? (L.E + 3) / 4 : 0;
  const int nsb = L.has_shared ? (L.f / GU_ROWS_PER_BLOCK) * L.T : 0;
  if (nrb + nsb > 0) {
    const int fs = L.has_shared ? L.fmt_shared : L.fmt_gate_up;
    if (cpl_d == 1) { FMT_SWITCH(fs, F, k1<F, 1>(a, nrb, nsb, s)) } else { FMT_SWITCH(fs, F, k1<F, 2>(a, nrb, nsb, s)) }
  }
  if (cpl_d == 1) { FMT_SWITCH(L.fmt_gate_up, F, k2<F, 1>(a, s)) } else { FMT_SWITCH(L.fmt_gate_up, F, k2<F, 2>(a, s)) }
  const int fsd = L.has_shared ? L.fmt_shared : L.fmt_down;
  if (cpl_f == 1) {
    FMT_SWITCH(L.fmt_down, FR, FMT_SWITCH(fsd, FS, k3<FR, FS, 1>(a, s)))
  } else {
    FMT_SWITCH(L.fmt_down, FR, FMT_SWITCH(fsd, FS, k3<FR, FS, 2>(a, s)))
  }
  return hipGetLastError();
}

}  // namespace qmoe
