// The shared expert on the prefill path as plain dense GEMMs: every token of
// a chunk goes through it, so its Q8 weights are converted to fp16 once per
// call (one pass over the three matrices) and multiplied by a library GEMM
// (hipBLASLt, fp16 operands, fp32 accumulation and output) instead of being
// decoded again for every M tile.  The pages
// run prefill experts on 16-bit matrix units ("YoungAi -- DeepSeek V4.1
// Flash on one DGX Spark", section 4.4, prefill), and list a Q8-to-F16
// weight conversion among the optional CUDA settings ("Running DeepSeek V4
// Flash on an RTX 5080 with 16GB VRAM Under Linux/WSL2 via DS4", table of
// launcher variables).
//
//   1. dequant: row n of a Q8 matrix -> fp16(d q 2^k_n), one rounding, with
//      2^k_n a power of two per row that puts the row's largest |d| * 128 in
//      [2^14, 2^15): no product overflows, and every nonzero one is a
//      normal fp16 when its block scale is at least 2^-21 of the row's
//      largest; colsc[n] = 2^-k_n;
//   2. G|U = x16 W_gu^T (T x 2f, fp32) by hipBLASLt, on dense_rows(T) rows;
//   3. swiglu: h = silu(g xs_t colsc) * (u xs_t colsc), stored as the grouped
//      GEMMs' gate/up epilogue stores it (fp16 times a power of two per row
//      and 64 outputs, with its exponent), so the row normalisation and the
//      down GEMM that follow are unchanged;
//   4. Ysh' = Hs W_d^T (T x d, fp32) by hipBLASLt; the combine multiplies it
//      by the row's and the column's powers of two.
#include <hipblaslt/hipblaslt.h>

#include <mutex>
#include <utility>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"

namespace qmoe {

namespace {

// One launch for the three matrices: row r < f of gate, f + r of up and
// 2f + r of down (the order of w_gu, w_dn and colsc), one wave per row.
// Lane l takes the row's 16-byte code pieces l, l + 64, ... (half a block
// each), so a wave reads 1 KB of codes and writes 2 KB of fp16 contiguously.
__global__ __launch_bounds__(256) void dequant_q8_kernel(QMat gate, QMat up, QMat down, int f, int d,
                                                         uint16_t* __restrict__ w_gu, uint16_t* __restrict__ w_dn,
                                                         float* __restrict__ colsc) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= 2 * f + d) return;  // uniform per wave
  const QMat& m = r < f ? gate : (r < 2 * f ? up : down);
  const int n = r < f ? r : (r < 2 * f ? r - f : r - 2 * f);
  uint16_t* o = r < 2 * f ? w_gu + (int64_t)r * d : w_dn + (int64_t)(r - 2 * f) * f;
  const int nb = m.nb;
  const uint16_t* ds = reinterpret_cast<const uint16_t*>(m.p_scale) + (int64_t)n * nb;
  float dmax = 0.0f;
  for (int b = lane; b < nb; b += 64) dmax = fmaxf(dmax, fabsf(half_bits_to_float(ds[b])));
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) dmax = fmaxf(dmax, __shfl_xor(dmax, s, 64));
  int k = 0;
  const float mx = dmax * 128.0f;
  if (mx > 0.0f && mx <= 3.4e38f) {
    int ex;
    frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
    k = min(max(15 - ex, -100), 100);
  }
  if (lane == 0) colsc[r] = __builtin_amdgcn_ldexpf(1.0f, -k);
  const uint8_t* q = m.p_a + (int64_t)n * nb * 32;
  for (int p = lane; p < 2 * nb; p += 64) {
    const float sc = __builtin_amdgcn_ldexpf(half_bits_to_float(ds[p >> 1]), k);
    const uint4 w = *reinterpret_cast<const uint4*>(q + 16 * p);
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float v0 = sc * (float)(int8_t)(wv[i] & 255u), v1 = sc * (float)(int8_t)((wv[i] >> 8) & 255u);
      const float v2 = sc * (float)(int8_t)((wv[i] >> 16) & 255u), v3 = sc * (float)(int8_t)(wv[i] >> 24);
      h[2 * i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1) << 16);
      h[2 * i + 1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v2) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v3) << 16);
    }
    *reinterpret_cast<uint4*>(o + 16 * p) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4*>(o + 16 * p + 8) = make_uint4(h[4], h[5], h[6], h[7]);
  }
}

// One wave per (token, 256 outputs): lane l takes outputs 4l .. 4l + 3 of
// the wave's run, and each group of 16 lanes one 64-output exponent chunk.
// D = [T][2f] (gate columns, then up).
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ D, const float* __restrict__ xs,
                                                     const float* __restrict__ colsc, int T, int f,
                                                     uint16_t* __restrict__ H, int8_t* __restrict__ Hexp) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int runs = f / 256;
  if (w >= T * runs) return;  // uniform per wave
  const int t = w / runs;
  const int n = 256 * (w - t * runs) + 4 * lane;
  const float x = xs[t];
  const float4 g = *reinterpret_cast<const float4*>(D + (int64_t)t * 2 * f + n);
  const float4 u = *reinterpret_cast<const float4*>(D + (int64_t)t * 2 * f + f + n);
  const float4 cg = *reinterpret_cast<const float4*>(colsc + n);
  const float4 cu = *reinterpret_cast<const float4*>(colsc + f + n);
  float hv[4] = {silu(g.x * x * cg.x) * (u.x * x * cu.x), silu(g.y * x * cg.y) * (u.y * x * cu.y),
                 silu(g.z * x * cg.z) * (u.z * x * cu.z), silu(g.w * x * cg.w) * (u.w * x * cu.w)};
  float mx = fmaxf(fmaxf(fabsf(hv[0]), fabsf(hv[1])), fmaxf(fabsf(hv[2]), fabsf(hv[3])));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));  // over the 16 lanes of the chunk
  int e = 0;
  if (mx > 0.0f && mx <= 3.4e38f) {
    int ex;
    frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
    e = min(max(ex - 15, -100), 100);
  }
  const float sc = __builtin_amdgcn_ldexpf(1.0f, -e);
  uint32_t h01 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(hv[0] * sc)) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(hv[1] * sc)) << 16);
  uint32_t h23 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(hv[2] * sc)) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(hv[3] * sc)) << 16);
  *reinterpret_cast<uint2*>(H + (int64_t)t * f + n) = make_uint2(h01, h23);
  if ((lane & 15) == 0) Hexp[(int64_t)t * (f / 64) + n / 64] = (int8_t)e;
}

// hipBLASLt: one handle per device, one plan (descriptors and the
// heuristic's first algorithm) per device and shape, made on first use under
// a lock and kept until the process ends; a shape the library has no
// algorithm for is remembered as such (ok = false) and not asked again.
// Only algorithms that need no workspace are taken: nothing is cleared
// between calls, the same bits come back every call, and a captured graph
// holds nothing but kernel launches.
struct GemmPlan {
  int dev, T, N, K;
  bool ok;
  hipblasLtMatmulDesc_t md;
  hipblasLtMatrixLayout_t la, lb, ld;
  hipblasLtMatmulAlgo_t algo;
};
std::mutex g_blt_mu;
std::vector<std::pair<int, hipblasLtHandle_t>> g_handles;
std::vector<GemmPlan> g_plans;

hipError_t blt_err(hipblasStatus_t st) { return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorUnknown; }

const GemmPlan* find_plan(int dev, int T, int N, int K) {  // (under the lock)
  for (const auto& p : g_plans)
    if (p.dev == dev && p.T == T && p.N == N && p.K == K) return &p;
  return nullptr;
}

// The descriptors and algorithm of D^T (N x T, column-major) = op(W) A^T,
// with W given as K x N (transposed) and A^T as K x T: column-major views of
// the row-major [N][K], [T][K] and [T][N] arrays.  p.ok = false when any
// step fails (whatever was created is destroyed).
void make_plan(hipblasLtHandle_t h, GemmPlan& p) {
  p.ok = false;
  p.md = nullptr;
  p.la = p.lb = p.ld = nullptr;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  bool good = hipblasLtMatmulDescCreate(&p.md, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16F, p.K, p.N, p.K) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16F, p.K, p.T, p.K) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.ld, HIP_R_32F, p.N, p.T, p.N) == HIPBLAS_STATUS_SUCCESS;
  if (good) {
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t no_ws = 0;
    hipblasLtMatmulHeuristicResult_t res[8];
    int nres = 0;
    good = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
           hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &no_ws,
                                                 sizeof(no_ws)) == HIPBLAS_STATUS_SUCCESS &&
           hipblasLtMatmulAlgoGetHeuristic(h, p.md, p.la, p.lb, p.ld, p.ld, pref, 8, res, &nres) ==
               HIPBLAS_STATUS_SUCCESS;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    for (int i = 0; good && i < nres && !p.ok; i++)
      if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize == 0) {
        p.algo = res[i].algo;
        p.ok = true;
      }
  }
  if (!p.ok) {
    if (p.ld) hipblasLtMatrixLayoutDestroy(p.ld);
    if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
    if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
    if (p.md) hipblasLtMatmulDescDestroy(p.md);
    p.md = nullptr;
    p.la = p.lb = p.ld = nullptr;
  }
}

hipError_t get_plan(int T, int N, int K, hipblasLtHandle_t* h_out, GemmPlan* p_out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_blt_mu);
  hipblasLtHandle_t h = nullptr;
  for (auto& x : g_handles)
    if (x.first == dev) h = x.second;
  if (!h) {
    if (hipblasStatus_t st = hipblasLtCreate(&h); st != HIPBLAS_STATUS_SUCCESS) return blt_err(st);
    g_handles.emplace_back(dev, h);
  }
  *h_out = h;
  const GemmPlan* q = find_plan(dev, T, N, K);
  if (!q) {
    GemmPlan p{};
    p.dev = dev;
    p.T = T;
    p.N = N;
    p.K = K;
    make_plan(h, p);
    g_plans.push_back(p);
    q = &g_plans.back();
  }
  if (!q->ok) return hipErrorNotSupported;
  *p_out = *q;
  return hipSuccess;
}

// D [T][N] fp32 (row-major) = A [T][K] fp16 times W [N][K]^T fp16
hipError_t gemm_tn(int T, int N, int K, const uint16_t* A, const uint16_t* W, float* D, hipStream_t s) {
  hipblasLtHandle_t h;
  GemmPlan p;
  if (hipError_t e = get_plan(T, N, K, &h, &p); e != hipSuccess) return e;
  const float alpha = 1.0f, beta = 0.0f;
  return blt_err(hipblasLtMatmul(h, p.md, &alpha, W, p.la, A, p.lb, &beta, D, p.ld, D, p.ld, &p.algo, nullptr, 0, s));
}

}  // namespace

bool shared_dense_ready(int T, int d, int f, hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return false;
  if (cs == hipStreamCaptureStatusNone) {  // make both plans now; none (no handle, no algorithm): grouped kernels
    hipblasLtHandle_t h;
    GemmPlan p;
    return get_plan(dense_rows(T), 2 * f, d, &h, &p) == hipSuccess && get_plan(dense_rows(T), d, f, &h, &p) == hipSuccess;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lk(g_blt_mu);
  const GemmPlan* gu = find_plan(dev, dense_rows(T), 2 * f, d);
  const GemmPlan* dn = find_plan(dev, dense_rows(T), d, f);
  return gu && gu->ok && dn && dn->ok;
}

hipError_t launch_shared_dense_gateup(const SharedDense& S, hipStream_t s) {
  int pid = prof_begin("prefill_shared_dequant", s);
  QMOE_LAUNCH(dequant_q8_kernel, dim3((2 * S.f + S.d + 3) / 4), dim3(256), 0, s, S.gate, S.up, S.down, S.f, S.d,
              S.w_gu, S.w_dn, S.colsc);
  prof_end(pid, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  pid = prof_begin("prefill_shared_gateup", s);
  prof_library_call(s);
  e = gemm_tn(dense_rows(S.T), 2 * S.f, S.d, S.x16, S.w_gu, S.dgu, s);
  prof_end(pid, s);
  if (e != hipSuccess) return e;
  pid = prof_begin("prefill_shared_swiglu", s);
  const int waves = S.T * (S.f / 256);
  QMOE_LAUNCH(swiglu_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, (const float*)S.dgu, S.xs, (const float*)S.colsc,
              S.T, S.f, S.hs, S.hsexp);
  prof_end(pid, s);
  return hipGetLastError();
}

hipError_t launch_shared_dense_down(const SharedDense& S, hipStream_t s) {
  const int pid = prof_begin("prefill_shared_down", s);
  prof_library_call(s);
  const hipError_t e = gemm_tn(dense_rows(S.T), S.d, S.f, S.hs, S.w_dn, S.ysh, s);
  prof_end(pid, s);
  return e;
}

}  // namespace qmoe
