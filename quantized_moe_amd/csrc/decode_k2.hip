// Second decode launch: exact top-k, routed gate/up + SwiGLU and the
// quantization of the routed SwiGLU outputs for the down projections; for a
// single token also the shared expert's gate/up + SwiGLU.
//
// The routed h rows of all tokens (T * k * d_ff, route-major) are cut into
// groups of 16, the unit of h's quantization scale; a block takes GCNT
// consecutive groups of one token (8 waves, 2 GCNT rows each), so every block
// streams the same bytes and finishes whole groups.  Block prologue, in
// parallel: wave 0 selects the token's experts from the router logits (every
// block of the token does the same exact top-k; the token's first block
// publishes idx / wt at its end); waves 1..7 build the IQ2 tables and run
// the block's share of a single token's shared gate/up, whose weights stream
// while the routes are not yet known.  Then every wave requests its rows'
// scale bytes and first weights and the rows run software-pipelined (x comes
// quantized from the first launch).
//
// VQ routed formats: waves 1..7 also copy the codebook into LDS during the
// prologue; the rows take x in fp32 straight from the caller's tensor and
// write h in fp32 (no quantization: the down rows read it as it is).
#include "decode_rows.hpp"
#include "topk.hpp"

namespace qmoe {
namespace dec {

template <int FMT, int FS, int D, int GCNT>
__global__ __launch_bounds__(THREADS) void k2_kernel(DecodeArgs a, int down_layout) {
  __shared__ Iq2Tab itab;
  __shared__ __attribute__((aligned(16))) float hbuf[16 * GCNT];
  __shared__ int s_sel[TOPK_MAX_K];
  __shared__ float s_zs[TOPK_MAX_K];
  extern __shared__ __align__(16) uint8_t k2_cb[];  // VQ: the codebook (dynamic LDS)
  constexpr int RPW = 2 * GCNT;  // h rows per wave
  // One step of codes in flight ahead of the compute: the rows are bound by
  // the decode arithmetic once streaming, and a deeper start (every wave of
  // the GPU requesting several steps at the barrier) delays every wave's
  // first step behind the whole flood (measured: depth 3 -> 1, -0.8 us).
  constexpr int PD = 1;
  constexpr int SH_RPW = 2;            // shared gate/up rows per wave call
  constexpr int SH_NS = (SH_RPW + Geo<FS, D>::RPS - 1) / Geo<FS, D>::RPS;
  constexpr int SCL_R = gateup_scale_bytes<FMT, D, RPW>(), SCL_S = gateup_scale_bytes<FS, D, SH_RPW>();
  constexpr int SCL_BYTES = SCL_R > SCL_S ? SCL_R : SCL_S;
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[WAVES * SCL_BYTES];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g0 = blockIdx.x * GCNT;  // first group of 16 rows
  const int R0 = 16 * g0;            // first routed h row (route-major over all tokens)
  const int t = R0 / (a.k * a.f);

  // A single token's shared gate/up (shared_k2): pairs of rows spread over
  // the blocks, taken by waves 1..7 of each block; h to hsh in fp32.
  auto shared_rows = [&]() {
    const int npair = a.f / SH_RPW;
    const int ppb = (npair + (int)gridDim.x - 1) / (int)gridDim.x;
    const int p0 = (int)blockIdx.x * ppb, p1 = min(npair, p0 + ppb);
    for (int pp = p0 + wave - 1; pp < p1; pp += WAVES - 1)
      gateup_rows<FS, D, SH_RPW, SH_NS>(a.s_gate, a.s_up, 1, a.f, 1, SH_RPW * pp, 0, nullptr, 0, a.xq_s, a.xs_s,
                                        &itab, s_scl + wave * SCL_BYTES, a.hsh + SH_RPW * pp);
  };

  // ---- prologue: wave 0 selects the routes while the others build the IQ2
  // tables and run the shared gate/up (its weights do not depend on the routes)
  if (wave == 0) {
    if (a.fused_topk) {
      if (a.router_bias)  // keys computed with the logits in the first launch
        wave_topk(a.zkey + (int64_t)t * a.E, a.E, a.k, s_sel, s_zs, nullptr, a.z + (int64_t)t * a.E);
      else
        wave_topk(a.z + (int64_t)t * a.E, a.E, a.k, s_sel, s_zs, nullptr);
    } else if (lane < a.k) {
      s_sel[lane] = a.idx[(int64_t)t * a.k + lane];
    }
  } else {
    if constexpr (is_vq(FMT)) vq_stage_codebook(a.vq_cb, k2_cb, vq_codes(FMT), threadIdx.x - 64, THREADS - 64);
    if constexpr (FMT == FMT_IQ2 || FS == FMT_IQ2) iq2_build(a.grid, threadIdx.x - 64, &itab);  // 384 items
    if constexpr (FS != FMT_IQ2) {
      if (a.shared_k2) shared_rows();
    }
  }
  __syncthreads();
  if constexpr (FS == FMT_IQ2) {  // the tables are published only now
    if (a.shared_k2 && wave > 0) shared_rows();
  }

  // ---- this wave's rows, software-pipelined ----
  if constexpr (is_vq(FMT)) {
    VqAct<D> act;
    act.load(static_cast<const uint8_t*>(a.x) + (int64_t)t * D * (a.x_dtype == X_BF16 ? 2 : 4), a.x_dtype,
             (threadIdx.x & 63) % VqGeo<D>::LPR);
    vq_gateup_rows<FMT, D, RPW, 2>(a.gate, a.up, a.E, a.f, a.k, R0 + wave * RPW, t, s_sel, act, k2_cb,
                                   a.hf + R0 + wave * RPW);
  } else {
    gateup_rows<FMT, D, RPW, PD>(a.gate, a.up, a.E, a.f, a.k, R0 + wave * RPW, t, s_sel, -1,
                                 a.xq + (int64_t)t * (D / 64) * CHUNK_BYTES, a.xs + (int64_t)t * (D / 64), &itab,
                                 s_scl + wave * SCL_BYTES, hbuf + wave * RPW);
    __syncthreads();
    if (wave == 0) quant_g32(hbuf, GCNT, 0, down_layout, a.hq + (int64_t)g0 * G16_BYTES, a.hs + g0);
  }
  // The token's first block publishes its routes and mixing weights (needed
  // only by the next launch, so off the prologue's critical path).
  if (wave == 1 && a.fused_topk && R0 % (a.k * a.f) == 0) {
    const float w = topk_weight_lane(s_zs, a.k);
    if (lane < a.k) {
      const int64_t o = (int64_t)t * a.k + lane;
      a.idx[o] = s_sel[lane];
      a.wt[o] = w;
      if (a.idx_out) a.idx_out[o] = s_sel[lane];
      if (a.wt_out) a.wt_out[o] = w;
    }
  }
}

template <int FMT, int FS, int D, int GCNT>
static hipError_t run_k2(const DecodeArgs& a, int blocks, int down_layout, hipStream_t s) {
  constexpr int dyn = is_vq(FMT) ? vq_codes(FMT) * 8 : 0;  // the codebook in LDS
  if constexpr (dyn > 0) {  // (raises the kernel's dynamic-LDS limit on first use)
    int per_cu = 0, n_cus = 0;
    if (hipError_t e = launch_shape((const void*)k2_kernel<FMT, FS, D, GCNT>, THREADS, dyn, dyn, &per_cu, &n_cus);
        e != hipSuccess)
      return e;
  }
  QMOE_LAUNCH((k2_kernel<FMT, FS, D, GCNT>), dim3(blocks), dim3(THREADS), dyn, s, a, down_layout);
  return hipGetLastError();
}

template <int FMT, int FS, int D>
static hipError_t run_k2_g(const DecodeArgs& a, int gcnt, int blocks, int dl, hipStream_t s) {
  if constexpr (!is_vq(FMT)) {  // (several tokens of the block formats only)
    if (gcnt == 6) return run_k2<FMT, FS, D, 6>(a, blocks, dl, s);
  }
  switch (gcnt) {
    case 3: return run_k2<FMT, FS, D, 3>(a, blocks, dl, s);
    case 2: return run_k2<FMT, FS, D, 2>(a, blocks, dl, s);
    default: return run_k2<FMT, FS, D, 1>(a, blocks, dl, s);
  }
}

template <int FMT, int D>
static hipError_t run_k2_s(const DecodeArgs& a, int fs, int gcnt, int blocks, int dl, hipStream_t s) {
  switch (fs) {
    case FMT_IQ2: return run_k2_g<FMT, FMT_IQ2, D>(a, gcnt, blocks, dl, s);
    case FMT_Q2K: return run_k2_g<FMT, FMT_Q2K, D>(a, gcnt, blocks, dl, s);
    default: return run_k2_g<FMT, FMT_Q8, D>(a, gcnt, blocks, dl, s);
  }
}

hipError_t launch_k2(const DecodeArgs& a, int fmt, int fs, int gcnt, int blocks, int down_layout, hipStream_t s) {
#define K2_FMT(D)                                                                  \
  switch (fmt) {                                                                   \
    case FMT_IQ2: return run_k2_s<FMT_IQ2, D>(a, fs, gcnt, blocks, down_layout, s); \
    case FMT_Q2K: return run_k2_s<FMT_Q2K, D>(a, fs, gcnt, blocks, down_layout, s); \
    case FMT_Q4K: return run_k2_s<FMT_Q4K, D>(a, fs, gcnt, blocks, down_layout, s); \
    case FMT_MX4: return run_k2_s<FMT_MX4, D>(a, fs, gcnt, blocks, down_layout, s); \
    case FMT_VQ12: return run_k2_s<FMT_VQ12, D>(a, fs, gcnt, blocks, down_layout, s); \
    case FMT_VQ13: return run_k2_s<FMT_VQ13, D>(a, fs, gcnt, blocks, down_layout, s); \
    default: return run_k2_s<FMT_Q8, D>(a, fs, gcnt, blocks, down_layout, s);       \
  }
  switch (a.d) {
    case 256: K2_FMT(256)
    case 512: K2_FMT(512)
    case 1024: K2_FMT(1024)
    case 2048: K2_FMT(2048)
    case 4096: K2_FMT(4096)
    default: K2_FMT(8192)
  }
#undef K2_FMT
}

}  // namespace dec
}  // namespace qmoe
