// Launchers of the HIP kernels (host side), used by the C-ABI layer api.cpp.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "moe.h"

namespace qmoe {

// Limits (mirrored by the validation in api.cpp and documented in moe.h).
constexpr int MAX_EXPERTS = 1024;
constexpr int TOPK_MAX_K = 16;
constexpr int TOPK_MAX_PER_LANE = MAX_EXPERTS / 64;
constexpr int ROUTER_ROWS_MAX_T = 8;  // above this the tiled router runs (router + top-k measured 29 / 32 us at 8 tokens, 51 / 33 us at 16)
constexpr int DECODE_MAX_T = MOE_DECODE_MAX_T;            // the decode path's limit
constexpr int AUTO_DECODE_MAX_T = MOE_AUTO_DECODE_MAX_T;  // MOE_PATH_AUTO's switch to prefill

// Per-kernel timing hooks (api.hip).  When profiling is enabled, prof_begin
// creates a start/stop event pair for the one launch that follows and hands it
// to that launch through QMOE_LAUNCH, which gives them to
// hipExtLaunchKernelGGL: the events are then stamped at the kernel's own
// start and end (no dispatch gap).  No-ops otherwise.
int prof_begin(const char* name, hipStream_t s);
void prof_end(int id, hipStream_t s);
void prof_take_events(hipEvent_t* start, hipEvent_t* stop);  // the pending pair, or nulls
// A region around a library call instead of one QMOE_LAUNCH: the start event
// is recorded on the stream now, the stop by prof_end (stream order, so the
// time includes the gaps between the library's launches).
void prof_library_call(hipStream_t s);

#define QMOE_LAUNCH(kern, grid, block, shmem, stream, ...)                                   \
  do {                                                                                         \
    hipEvent_t qmoe_ev_a_, qmoe_ev_b_;                                                          \
    ::qmoe::prof_take_events(&qmoe_ev_a_, &qmoe_ev_b_);                                         \
    hipExtLaunchKernelGGL(kern, grid, block, shmem, stream, qmoe_ev_a_, qmoe_ev_b_, 0, __VA_ARGS__); \
  } while (0)

// Launch shape of a kernel on the current device (api.hip): the number of its
// blocks of `threads` threads and `lds_bytes` of dynamic LDS that fit one CU
// at once, and the device's CU count.  The first query for a kernel on a
// device raises its dynamic-LDS limit to lds_max.  Results are cached per
// (device, kernel, lds_bytes) under a lock, so concurrent host threads and
// several devices are safe.  kernel = nullptr queries only the CU count.
hipError_t launch_shape(const void* kernel, int threads, int lds_bytes, int lds_max, int* blocks_per_cu,
                        int* n_cus);

// route.hip
hipError_t launch_router(const float* W, int E, int d, const void* x, int x_dtype, int T, float* z, hipStream_t s);
hipError_t launch_topk(const float* z, int T, int E, int k, const float* bias, int32_t* idx, float* wt, int32_t* idx2,
                       float* wt2, hipStream_t s);

// bucket.hip.  tile_start (nullable): [E+1] exclusive prefix of
// ceil(counts[e] / tile_m) -- the M-tile schedule of the grouped GEMMs.
// scratch (nullable): bucket_scratch_ints(T k, E) counts, which saves a
// launch (without it the chunk histograms are kept in pos).  Each launch is
// timed under its own profiler name (bucket_count, _scan, _place, _inverse).
hipError_t launch_bucket(const int32_t* idx, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* pos, int32_t* tile_start, int tile_m, int32_t* scratch, hipStream_t s);
size_t bucket_scratch_ints(int n, int E);

// decode.hip (+ decode_k1/k2/k3.hip): the three decode launches of one layer
// (or of given routes).
struct DecodeLaunch {
  int E, d, f, k, T;
  int fmt_gate_up, fmt_down, fmt_shared, has_shared;
  const void *w_gate, *w_up, *w_down, *s_gate, *s_up, *s_down;
  const uint8_t* grid;
  const uint8_t* vq_cb;    // E4M3 codewords [n][8] (VQ routed formats)
  const float* w_router;   // used when fused_topk
  const void* x;
  int x_dtype;
  float* z;                // [T][E] workspace (fused_topk)
  int32_t* idx;            // [T][k] routes: written (fused_topk) or read
  float* wt;               // [T][k]
  int32_t* idx_out;        // nullable copies for the caller (fused_topk)
  float* wt_out;
  void* quant;             // decode_quant_bytes() of workspace: shared h, quantized h
  float* y;                // [T][d]
  int fused_topk;          // 1: router logits in the first launch, top-k in the second
  const float* router_bias;  // nullable [E]: select on sigmoid32(z) + bias (fused_topk)
  float* zkey;               // [T][E] workspace for the keys (fused_topk with a bias)
  const float* down_gain;    // nullable [E][d]: per-channel gains of each routed expert's output
};
hipError_t launch_decode(const DecodeLaunch& L, hipStream_t s);
size_t decode_quant_bytes(int T, int k, int d, int f);

// prefill.hip: grouped GEMMs + combine (bucketing already done).
constexpr int PREFILL_BM = 32;         // M tile of the routed grouped GEMMs (rows of one expert's bucket)
constexpr int PREFILL_SHARED_BM = 64;  // M tile of the shared expert's GEMMs
constexpr int PREFILL_HCHUNK = 64;  // outputs per power-of-two exponent of the gate/up GEMMs' fp16 H rows
struct PrefillLaunch {
  int E, d, f, k, T;
  int fmt_gate_up, fmt_down, fmt_shared, has_shared;
  const void *w_gate, *w_up, *w_down, *s_gate, *s_up, *s_down;
  const uint8_t* grid;
  const uint8_t* vq_cb;  // E4M3 codewords [n][8] (VQ routed formats)
  const void* x;
  int x_dtype;
  const int32_t *counts, *offsets, *tile_start, *perm, *pos;
  const int32_t* idx;      // [T][k] routes (for the down gains)
  const float* wt;
  const float* down_gain;  // nullable [E][d]
  uint16_t* x16;  // fp16 [T][d]: x times a per-token power of two
  float* xs;      // [T]: that power of two
  float* route_xs;  // [T*k]: the same at each route, in bucket order
  void* H;      // fp16 [T*k][f]: h * 2^-Hexp of its 128-column chunk
  void* Hs;     // fp16 [T][f]
  int8_t* Hexp;   // [T*k][f/PREFILL_HCHUNK]
  int8_t* Hsexp;  // [T][f/PREFILL_HCHUNK]
  float* Hsc;     // [T*k]: 2^e of each H row once its chunks share one exponent
  float* Hssc;    // [T]
  float* Ye;    // [T*k][d]
  float* Ysh;   // [T][d]
  float* y;     // [T][d]
  // a Q8 shared expert as dense fp16 GEMMs (dense.hip): the buffers, all
  // null when the workspace has none (then the grouped kernels run it)
  uint16_t *Wgu, *Wdn;  // fp16 [2f][d] (gate rows, then up), [d][f]
  float* colsc;         // [2f + d]: each dequantized row's power of two
  float* Dgu;           // fp32 [T][2f]
};
hipError_t launch_prefill_gemms(const PrefillLaunch& P, hipStream_t s);

// dense.hip: the shared expert of a prefill chunk as dense GEMMs on fp16
// copies of its Q8 weights (made by each call).  The GEMMs run on
// dense_rows(T) rows (a multiple of 64, so that one GEMM plan serves 64 chunk
// sizes); x16, Hs and Ysh are carved with that many rows, and the rows past
// T hold whatever the buffers held (their results are never read).
inline int dense_rows(int T) { return (T + 63) & ~63; }
struct SharedDense {
  int T, d, f;
  QMat gate, up, down;
  const uint16_t* x16;  // [T][d], x16 * xs = x
  const float* xs;      // [T]
  uint16_t *w_gu, *w_dn;
  float* colsc;  // [2f + d]
  float* dgu;    // [T][2f]
  uint16_t* hs;  // [T][f]: fp16 h times a power of two per 64 outputs ...
  int8_t* hsexp;  // [T][f/64]: ... and its exponent
  float* ysh;     // [T][d]: before the row and column powers of two
};
// Whether the dense path can run this chunk: outside stream capture it makes
// the chunk size's two GEMM plans (false if the library offers no algorithm
// or no handle); under capture it only looks them up (making them may
// allocate).  false: the grouped kernels run the shared expert.
bool shared_dense_ready(int T, int d, int f, hipStream_t s);
hipError_t launch_shared_dense_gateup(const SharedDense& S, hipStream_t s);
hipError_t launch_shared_dense_down(const SharedDense& S, hipStream_t s);
// The grouped GEMMs address their A operands (x16, H, Hs) with 32-bit byte
// offsets: false when T, k, d, f would pass 2^31.
inline bool prefill_fits(int T, int k, int d, int f) {
  return (int64_t)T * d * 2 < (int64_t(1) << 31) && (int64_t)T * k * f * 2 < (int64_t(1) << 31);
}

// repack.hip: n_rows rows of K inputs
hipError_t launch_repack(int fmt, int64_t n_rows, int K, const void* src, void* dst, int to_device, hipStream_t s);

}  // namespace qmoe
