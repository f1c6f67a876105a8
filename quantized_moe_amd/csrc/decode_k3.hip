// Third decode launch: down projections of the routed experts and of the
// shared expert, and the combine y = sum_j wt_j (g_j ye_j) + ysh in that
// fixed order (the per-layer MoE sum of "YoungAi -- DeepSeek V4.1 Flash on
// one DGX Spark", section 4.2; g_j the routed expert's per-channel down
// gains, one when none are given; ye is taken before the routing weight).
//
// Block = 16 output rows of one token.  Tasks: the k routed experts (16 rows
// each, or two tasks of 8 rows) and the shared expert (in two or four
// tasks); a wave runs one task at a time with that task's h slice in
// registers (the shared expert's fp32 h is quantized by the task itself).
// Row results meet in LDS.  VQ routed down rows read the fp32 h of the
// previous launch and the codebook, which the block first copies into LDS.
#include "decode_rows.hpp"

namespace qmoe {
namespace dec {

// ROWS rows of expert e's down matrix against one h vector (quantized in
// groups of 16 at hq / hs, or fp32 at hf and quantized here when hq is
// null); row results to out[0 .. ROWS).  The h slice is requested before the
// codes, so both loads are in flight together.
template <int FMT, int K, int ROWS>
__device__ __forceinline__ void down_rows(const QMat& m, int e, int E, int r0, const uint8_t* hq, const float* hs,
                                          const float* hf, const float* gain, const Iq2Tab* tab, uint8_t* my_scales,
                                          float* out) {
  constexpr int NS = DownRows<FMT, K, ROWS, 1>::NS;
  // three steps of loads kept in flight ahead of the compute; Q4K's pieces
  // are twice as large and MXFP4's carry twice the activation registers
  // (two steps, one for rows of more than 64 pieces)
  constexpr int CPL = Geo<FMT, K>::CPL;
  constexpr int PDMAX = FMT == FMT_Q4K || FMT == FMT_MX4 ? (CPL > 1 ? 1 : 2) : 3;
  DownRows<FMT, K, ROWS, (NS < PDMAX ? NS : PDMAX)> dr;
  if constexpr (FMT == FMT_MX4) {  // routed experts only: h always comes quantized
    dr.load_act(hq, hs);
    dr.issue(m, e, E, r0, my_scales, gain);
  } else if (hq) {
    dr.load_act(hq, hs);
    dr.issue(m, e, E, r0, my_scales, gain);
  } else {
    dr.fetch_act_f32(hf);
    dr.issue(m, e, E, r0, my_scales, gain);
    dr.quant_act_f32();
  }
  dr.run(tab, my_scales, out);
}

template <int FR, int FS, int F>
__global__ __launch_bounds__(64 * k3_waves(FR, FS, F)) void k3_kernel(DecodeArgs a) {
  constexpr int K3_WAVES = k3_waves(FR, FS, F);
  constexpr int RT_PARTS = K3_WAVES / 8;
  constexpr int SH_PARTS = K3_WAVES / 4;  // the shared expert's 16 rows as tasks of 4 (16 waves) or 8
  __shared__ Iq2Tab itab;
  __shared__ float ye[(TOPK_MAX_K + 1) * DN_ROWS];
  constexpr int SH_ROWS = DN_ROWS / SH_PARTS;
  constexpr int SCL_R = RowScales<FR, F>::STAGE ? (DN_ROWS / RT_PARTS) * RowScales<FR, F>::BYTES : 16;
  constexpr int SCL_S = RowScales<FS, F>::STAGE ? SH_ROWS * RowScales<FS, F>::BYTES : 16;
  constexpr int SCL_BYTES = SCL_R > SCL_S ? SCL_R : SCL_S;
  __shared__ __attribute__((aligned(16))) uint8_t s_scl[K3_WAVES * SCL_BYTES];
  extern __shared__ __align__(16) uint8_t k3_cb[];  // VQ: the codebook (dynamic LDS)
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.y;
  const int row0 = blockIdx.x * DN_ROWS;
  if constexpr (is_vq(FR)) vq_stage_codebook(a.vq_cb, k3_cb, vq_codes(FR), threadIdx.x, 64 * K3_WAVES);
  if constexpr (FR == FMT_IQ2 || FS == FMT_IQ2) iq2_build(a.grid, threadIdx.x, &itab);
  if constexpr (is_vq(FR) || FR == FMT_IQ2 || FS == FMT_IQ2) __syncthreads();
  constexpr int NG = F / 16;  // groups of 16 per h vector
  constexpr int RT_ROWS = DN_ROWS / RT_PARTS;
  const int n_rt = a.k * RT_PARTS;
  const int n_tasks = n_rt + (a.has_shared ? SH_PARTS : 0);
  for (int task = wave; task < n_tasks; task += K3_WAVES) {
    if (task < n_rt) {
      const int q = task / RT_PARTS, part = task % RT_PARTS;
      const int64_t r = (int64_t)t * a.k + q;
      const int e = a.idx[r];
      // the expert's output gains scale its row results (ye holds g * y_e)
      const float* gain = a.down_gain && (unsigned)e < (unsigned)a.E ? a.down_gain + (int64_t)e * a.d : nullptr;
      if constexpr (is_vq(FR)) {
        vq_down_rows<FR, F, RT_ROWS>(a.down, e, a.E, row0 + part * RT_ROWS, a.hf + r * F, gain, k3_cb,
                                     ye + q * DN_ROWS + part * RT_ROWS);
      } else {
        down_rows<FR, F, RT_ROWS>(a.down, e, a.E, row0 + part * RT_ROWS, a.hq + r * NG * G16_BYTES, a.hs + r * NG,
                                  nullptr, gain, &itab, s_scl + wave * SCL_BYTES, ye + q * DN_ROWS + part * RT_ROWS);
      }
    } else {
      const int part = task - n_rt;
      down_rows<FS, F, SH_ROWS>(a.s_down, 0, 1, row0 + part * SH_ROWS, nullptr, nullptr, a.hsh + (int64_t)t * F,
                                nullptr, &itab, s_scl + wave * SCL_BYTES, ye + a.k * DN_ROWS + part * SH_ROWS);
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < DN_ROWS) {
    const int n = threadIdx.x;
    float acc = 0.0f;
    for (int q = 0; q < a.k; q++) acc = __builtin_fmaf(a.wt[(int64_t)t * a.k + q], ye[q * DN_ROWS + n], acc);
    if (a.has_shared) acc += ye[a.k * DN_ROWS + n];
    a.y[(int64_t)t * a.d + row0 + n] = acc;
  }
}

template <int FR, int FS, int F>
static hipError_t run_k3(const DecodeArgs& a, hipStream_t s) {
  constexpr int dyn = is_vq(FR) ? vq_codes(FR) * 8 : 0;  // the codebook in LDS
  constexpr int threads = 64 * k3_waves(FR, FS, F);
  if constexpr (dyn > 0) {  // (raises the kernel's dynamic-LDS limit on first use)
    int per_cu = 0, n_cus = 0;
    if (hipError_t e = launch_shape((const void*)k3_kernel<FR, FS, F>, threads, dyn, dyn, &per_cu, &n_cus);
        e != hipSuccess)
      return e;
  }
  QMOE_LAUNCH((k3_kernel<FR, FS, F>), dim3(a.d / DN_ROWS, a.T), dim3(threads), dyn, s, a);
  return hipGetLastError();
}

template <int F>
static hipError_t run_k3_f(const DecodeArgs& a, int fr, int fs, hipStream_t s) {
#define K3_FS(FR)                                             \
  switch (fs) {                                               \
    case FMT_IQ2: return run_k3<FR, FMT_IQ2, F>(a, s);        \
    case FMT_Q2K: return run_k3<FR, FMT_Q2K, F>(a, s);        \
    default: return run_k3<FR, FMT_Q8, F>(a, s);              \
  }
  switch (fr) {
    case FMT_IQ2: K3_FS(FMT_IQ2)
    case FMT_Q2K: K3_FS(FMT_Q2K)
    case FMT_Q4K: K3_FS(FMT_Q4K)
    case FMT_MX4: K3_FS(FMT_MX4)
    case FMT_VQ12: K3_FS(FMT_VQ12)
    case FMT_VQ13: K3_FS(FMT_VQ13)
    default: K3_FS(FMT_Q8)
  }
#undef K3_FS
}

hipError_t launch_k3(const DecodeArgs& a, int fmt_down, int fmt_shared, hipStream_t s) {
  switch (a.f) {
    case 256: return run_k3_f<256>(a, fmt_down, fmt_shared, s);
    case 512: return run_k3_f<512>(a, fmt_down, fmt_shared, s);
    case 1024: return run_k3_f<1024>(a, fmt_down, fmt_shared, s);
    case 2048: return run_k3_f<2048>(a, fmt_down, fmt_shared, s);
    case 4096: return run_k3_f<4096>(a, fmt_down, fmt_shared, s);
    default: return run_k3_f<8192>(a, fmt_down, fmt_shared, s);
  }
}

}  // namespace dec
}  // namespace qmoe
