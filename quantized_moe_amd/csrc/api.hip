// C ABI of libqmoe (declarations and contracts: include/moe.h).
//
// Host side only: argument validation (before anything is enqueued),
// workspace carving, path selection and launches.  The narrow C interface
// that hides tensor internals from its callers follows the ds4 engine's
// design of a small public header over a fixed in-engine layout ("ds4
// timeline", files.btbytes.com: ds4.h as the narrow public API), and the
// refusal of unknown formats and versions follows the fail-loudly format
// whitelist on "YoungAi -- DeepSeek V4.1 Flash on one DGX Spark", section 4.1.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace qmoe;

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local std::string g_err;

static int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

static int ok() {
  g_err.clear();
  return MOE_OK;
}

static int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_CHECK(expr, what)                  \
  do {                                         \
    hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// ---------------------------------------------------------------------------
// profiling (events on the launch stream; eager use only)
// ---------------------------------------------------------------------------
namespace qmoe {
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
static std::mutex g_prof_mu;
static std::vector<ProfRec> g_prof;
static bool g_prof_on = false;

static thread_local hipEvent_t t_pend_a = nullptr, t_pend_b = nullptr;

int prof_begin(const char* name, hipStream_t s) {
  (void)s;
  if (!g_prof_on) return -1;
  ProfRec r;
  r.name = name;
  if (hipEventCreate(&r.a) != hipSuccess) return -1;
  if (hipEventCreate(&r.b) != hipSuccess) {
    (void)hipEventDestroy(r.a);
    return -1;
  }
  t_pend_a = r.a;
  t_pend_b = r.b;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back(r);
  return (int)g_prof.size() - 1;
}

void prof_take_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = t_pend_a;
  *stop = t_pend_b;
  t_pend_a = t_pend_b = nullptr;
}

static thread_local hipEvent_t t_lib_b = nullptr;

void prof_library_call(hipStream_t s) {
  if (t_pend_a == nullptr) return;
  (void)hipEventRecord(t_pend_a, s);
  t_lib_b = t_pend_b;
  t_pend_a = t_pend_b = nullptr;
}

void prof_end(int id, hipStream_t s) {
  if (id < 0) return;
  if (t_lib_b != nullptr) {  // a library call's region: its end in stream order
    (void)hipEventRecord(t_lib_b, s);
    t_lib_b = nullptr;
  } else if (t_pend_a != nullptr) {  // no launch consumed the pair: record it empty
    (void)hipEventRecord(t_pend_a, s);
    (void)hipEventRecord(t_pend_b, s);
    t_pend_a = t_pend_b = nullptr;
  }
}
}  // namespace qmoe

// ---------------------------------------------------------------------------
// launch shapes (occupancy and CU count), cached per device and kernel
// ---------------------------------------------------------------------------
namespace qmoe {
namespace {
struct ShapeEntry {
  int dev;
  const void* kernel;
  int lds_bytes;  // -1: the entry only records that the LDS limit was raised
  int blocks_per_cu, n_cus;
};
std::mutex g_shape_mu;
std::vector<ShapeEntry> g_shapes;
}  // namespace

hipError_t launch_shape(const void* kernel, int threads, int lds_bytes, int lds_max, int* blocks_per_cu,
                        int* n_cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_shape_mu);
  bool raised = false;
  for (const ShapeEntry& x : g_shapes) {
    if (x.dev != dev || x.kernel != kernel) continue;
    if (x.lds_bytes == lds_bytes) {
      *blocks_per_cu = x.blocks_per_cu;
      *n_cus = x.n_cus;
      return hipSuccess;
    }
    raised = true;
  }
  if (!raised && kernel != nullptr && lds_max > 0) {
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds_max);
    if (e != hipSuccess) return e;
  }
  int nb = 0, cus = 0;
  if (kernel != nullptr) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, lds_bytes);
    if (e != hipSuccess) return e;
  }
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  ShapeEntry x{dev, kernel, lds_bytes, nb > 0 ? nb : 1, cus > 0 ? cus : 1};
  g_shapes.push_back(x);
  *blocks_per_cu = x.blocks_per_cu;
  *n_cus = x.n_cus;
  return hipSuccess;
}
}  // namespace qmoe

extern "C" int moe_profile_enable(int32_t on) {
  g_prof_on = on != 0;
  return ok();
}

extern "C" int moe_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof) {
    (void)hipEventSynchronize(r.b);
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  return ok();
}

extern "C" int moe_profile_collect(int32_t max_kernels, char* names, int64_t* launches, double* total_ms,
                                   int32_t* n_kernels) {
  if (!names || !launches || !total_ms || !n_kernels || max_kernels < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_profile_collect: null output");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<std::string> keys;
  std::vector<double> ms;
  std::vector<int64_t> cnt;
  for (auto& r : g_prof) {
    HIP_CHECK(hipEventSynchronize(r.b), "hipEventSynchronize");
    float t = 0.f;
    HIP_CHECK(hipEventElapsedTime(&t, r.a, r.b), "hipEventElapsedTime");
    size_t i = 0;
    while (i < keys.size() && keys[i] != r.name) i++;
    if (i == keys.size()) {
      keys.push_back(r.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += t;
    cnt[i] += 1;
  }
  const int n = (int)keys.size() < max_kernels ? (int)keys.size() : max_kernels;
  for (int i = 0; i < n; i++) {
    strncpy(names + 48 * i, keys[i].c_str(), 47);
    names[48 * i + 47] = 0;
    launches[i] = cnt[i];
    total_ms[i] = ms[i];
  }
  *n_kernels = n;
  return ok();
}

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }
static bool fmt_known(int f) {
  return f == MOE_FMT_IQ2XXS_L || f == MOE_FMT_Q2K_L || f == MOE_FMT_Q8_0_L || f == MOE_FMT_Q4K_L ||
         f == MOE_FMT_MXFP4_L || f == MOE_FMT_VQ12_L || f == MOE_FMT_VQ13_L;
}
static_assert(MOE_FMT_VQ12_L == FMT_VQ12 && MOE_FMT_VQ13_L == FMT_VQ13 && MOE_FMT_MXFP4_L == FMT_MX4,
              "format ids of the header and of the kernels agree");

#define NEED_PTR(p, what)                                                                       \
  do {                                                                                          \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s: %s is null", fn, what);                     \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, what); \
  } while (0)

static int check_dims(const char* fn, int E, int d, int k) {
  if (E < 1 || E > MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "%s: n_experts %d not in [1, %d]", fn, E, MAX_EXPERTS);
  if (!pow2_in(d, 256, 8192)) return fail(MOE_ERR_INVALID_ARG, "%s: d_model %d is not a power of two in [256, 8192]", fn, d);
  if (k < 1 || k > TOPK_MAX_K || k > E)
    return fail(MOE_ERR_INVALID_ARG, "%s: top_k %d not in [1, min(n_experts, %d)]", fn, k, TOPK_MAX_K);
  return MOE_OK;
}

static int check_T(const char* fn, int T) {
  if (T < 0 || T > 65536) return fail(MOE_ERR_INVALID_ARG, "%s: T %d not in [0, 65536]", fn, T);
  return MOE_OK;
}

// The prefill GEMMs address x16 [T][d] and H [T*k][f] (fp16) with 32-bit
// byte offsets; checked before anything is enqueued.
static int check_prefill_size(const char* fn, int T, int k, int d, int f) {
  if (!prefill_fits(T, k, d, f))
    return fail(MOE_ERR_INVALID_ARG,
                "%s: T %d with top_k %d, d_model %d, d_ff %d exceeds the prefill path's 2^31-byte activation "
                "buffers (T*d*2 and T*top_k*d_ff*2 must stay below 2^31)", fn, T, k, d, f);
  return MOE_OK;
}

static int check_dtype(const char* fn, int x_dtype) {
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown activation dtype %d", fn, x_dtype);
  return MOE_OK;
}

// Checks every field of a layer that the compute paths read (the weights in
// `want_layout`: the compute entry points read only the device layout).
static int check_layer(const char* fn, const moe_layer* L, bool need_router, int want_layout = MOE_LAYOUT_DEVICE) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "%s: layer is null", fn);
  if (L->abi_version != MOE_ABI_VERSION)
    return fail(MOE_ERR_UNSUPPORTED, "%s: layer abi_version %u, library speaks %d", fn, L->abi_version, MOE_ABI_VERSION);
  int rc = check_dims(fn, L->n_experts, L->d_model, L->top_k);
  if (rc) return rc;
  if (!pow2_in(L->d_ff, 256, 8192)) return fail(MOE_ERR_INVALID_ARG, "%s: d_ff %d is not a power of two in [256, 8192]", fn, L->d_ff);
  if (!fmt_known(L->fmt_gate_up)) return fail(MOE_ERR_UNSUPPORTED, "%s: unknown gate/up format %d", fn, L->fmt_gate_up);
  if (!fmt_known(L->fmt_down)) return fail(MOE_ERR_UNSUPPORTED, "%s: unknown down format %d", fn, L->fmt_down);
  if (L->layout != want_layout) {
    if (L->layout == MOE_LAYOUT_CANONICAL)
      return fail(MOE_ERR_UNSUPPORTED,
                  "%s: weights must be in MOE_LAYOUT_DEVICE (convert with moe_prepare_weights or moe_repack)", fn);
    if (L->layout == MOE_LAYOUT_DEVICE)
      return fail(MOE_ERR_UNSUPPORTED, "%s: the layer's weights are already in MOE_LAYOUT_DEVICE", fn);
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown layout %d", fn, L->layout);
  }
  if (L->has_shared != 0 && L->has_shared != 1) return fail(MOE_ERR_INVALID_ARG, "%s: has_shared must be 0 or 1", fn);
  NEED_PTR(L->w_gate, "w_gate");
  NEED_PTR(L->w_up, "w_up");
  NEED_PTR(L->w_down, "w_down");
  bool iq2 = L->fmt_gate_up == MOE_FMT_IQ2XXS_L || L->fmt_down == MOE_FMT_IQ2XXS_L;
  if (is_vq(L->fmt_gate_up) || is_vq(L->fmt_down)) {
    if (is_vq(L->fmt_gate_up) != is_vq(L->fmt_down))
      return fail(MOE_ERR_UNSUPPORTED,
                  "%s: the VQ formats cover a layer's routed gate/up and down together (one codebook per layer); "
                  "gate/up format %d with down format %d", fn, L->fmt_gate_up, L->fmt_down);
    NEED_PTR(L->vq_codebook, "vq_codebook");
    if (L->vq_codes != 4096 && L->vq_codes != 8192)
      return fail(MOE_ERR_INVALID_ARG, "%s: vq_codes %d is neither 4096 nor 8192", fn, L->vq_codes);
    const int need = max(is_vq(L->fmt_gate_up) ? vq_codes(L->fmt_gate_up) : 0,
                         is_vq(L->fmt_down) ? vq_codes(L->fmt_down) : 0);
    if (L->vq_codes < need)
      return fail(MOE_ERR_INVALID_ARG, "%s: a 13-bit VQ matrix needs 8192 codewords, the codebook has %d", fn,
                  L->vq_codes);
  }
  if (L->has_shared) {
    if (!fmt_known(L->fmt_shared)) return fail(MOE_ERR_UNSUPPORTED, "%s: unknown shared format %d", fn, L->fmt_shared);
    if (L->fmt_shared == MOE_FMT_Q4K_L || L->fmt_shared == MOE_FMT_MXFP4_L || is_vq(L->fmt_shared))
      return fail(MOE_ERR_UNSUPPORTED,
                  "%s: Q4K_L, MXFP4_L and the VQ formats are routed-expert formats (shared expert: IQ2XXS_L, "
                  "Q2K_L or Q8_0_L)", fn);
    NEED_PTR(L->s_gate, "s_gate");
    NEED_PTR(L->s_up, "s_up");
    NEED_PTR(L->s_down, "s_down");
    iq2 = iq2 || L->fmt_shared == MOE_FMT_IQ2XXS_L;
  }
  if (iq2) NEED_PTR(L->iq2_grid, "iq2_grid");
  if (need_router) NEED_PTR(L->w_router, "w_router");
  if (L->router_bias && ((uintptr_t)L->router_bias & 3u))
    return fail(MOE_ERR_INVALID_ARG, "%s: router_bias is not 4-byte aligned", fn);
  if (L->down_gain && !aligned16(L->down_gain))
    return fail(MOE_ERR_INVALID_ARG, "%s: down_gain is not 16-byte aligned", fn);
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// workspace
// ---------------------------------------------------------------------------
namespace {
struct Carve {
  size_t off = 0;
  uint8_t* base = nullptr;
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

struct RouteWs {
  float* z;
};
struct DecodeWs {
  void* quant;
};
struct PrefillWs {
  int32_t *counts, *offsets, *tile_start, *perm, *pos;
  int32_t* bucket_hist;  // the bucketing's chunk histograms
  uint16_t* x16;
  float *xs, *route_xs;
  void *H, *Hs;
  int8_t *Hexp, *Hsexp;
  float *Hsc, *Hssc;
  float *Ye, *Ysh;
  uint16_t *Wgu, *Wdn;  // the dense shared expert's fp16 weights (null without)
  float *colsc, *Dgu;
};
struct LayerWs {
  float* z;
  float* zkey;  // selection keys under a router bias
  int32_t* idx;
  float* wt;
};

void carve_route(Carve& c, RouteWs& w, int E, int T) { w.z = (float*)c.take((size_t)T * E * 4); }
void carve_decode(Carve& c, DecodeWs& w, int T, int k, int d, int f) { w.quant = c.take(decode_quant_bytes(T, k, d, f)); }
void carve_prefill(Carve& c, PrefillWs& w, int E, int T, int k, int d, int f, int has_shared, bool dense,
                   bool bucket_out) {
  const size_t n = (size_t)T * k;
  if (!bucket_out) {
    w.counts = (int32_t*)c.take((size_t)E * 4);
    w.offsets = (int32_t*)c.take((size_t)(E + 1) * 4);
    w.perm = (int32_t*)c.take(n * 4);
  }
  w.tile_start = (int32_t*)c.take((size_t)(E + 1) * 4);
  w.pos = (int32_t*)c.take(n * 4);
  w.bucket_hist = (int32_t*)c.take(bucket_scratch_ints((int)n, E) * 4);
  const size_t Tg = dense && has_shared ? dense_rows(T) : T;  // rows of the dense shared GEMMs' operands
  w.x16 = (uint16_t*)c.take(Tg * d * 2);
  w.xs = (float*)c.take((size_t)T * 4);
  w.route_xs = (float*)c.take(n * 4);
  w.H = c.take(n * f * 2);
  w.Hexp = (int8_t*)c.take(n * (f / PREFILL_HCHUNK));
  w.Hsc = (float*)c.take(n * 4);
  w.Ye = (float*)c.take(n * d * 4);
  if (has_shared) {
    w.Hs = c.take(Tg * f * 2);
    w.Hsexp = (int8_t*)c.take((size_t)T * (f / PREFILL_HCHUNK));
    w.Hssc = (float*)c.take((size_t)T * 4);
    w.Ysh = (float*)c.take(Tg * d * 4);
  } else {
    w.Hs = nullptr;
    w.Hsexp = nullptr;
    w.Hssc = nullptr;
    w.Ysh = nullptr;
  }
  w.Wgu = w.Wdn = nullptr;
  w.colsc = w.Dgu = nullptr;
  if (has_shared && dense) {
    w.Wgu = (uint16_t*)c.take((size_t)2 * f * d * 2);
    w.Wdn = (uint16_t*)c.take((size_t)d * f * 2);
    w.colsc = (float*)c.take((size_t)(2 * f + d) * 4);
    w.Dgu = (float*)c.take(Tg * 2 * f * 4);
  }
}
void carve_layer_routes(Carve& c, LayerWs& w, int E, int T, int k) {
  w.z = (float*)c.take((size_t)T * E * 4);
  w.zkey = (float*)c.take((size_t)T * E * 4);
  w.idx = (int32_t*)c.take((size_t)T * k * 4);
  w.wt = (float*)c.take((size_t)T * k * 4);
}

size_t ws_route(int E, int T) {
  Carve c;
  RouteWs w;
  carve_route(c, w, E, T);
  return c.off;
}
size_t ws_decode(int T, int k, int d, int f) {
  Carve c;
  DecodeWs w;
  carve_decode(c, w, T, k, d, f);
  return c.off;
}
size_t ws_prefill(int E, int T, int k, int d, int f, int sh, bool dense) {
  Carve c;
  PrefillWs w;
  carve_prefill(c, w, E, T, k, d, f, sh, dense, false);
  return c.off;
}
size_t ws_layer(int E, int T, int k, int d, int f, int sh, bool dense, int path) {
  Carve c;
  LayerWs lw;
  carve_layer_routes(c, lw, E, T, k);
  if (path == MOE_PATH_DECODE) {  // (calls above the decode limit run in chunks of at most that many tokens)
    DecodeWs w;
    carve_decode(c, w, T < DECODE_MAX_T ? T : DECODE_MAX_T, k, d, f);
  } else {
    PrefillWs w;
    carve_prefill(c, w, E, T, k, d, f, sh, dense, false);
  }
  return c.off;
}
}  // namespace

// The shared expert of a prefill call as dense fp16 GEMMs (dense.hip): a Q8
// shared expert and a caller's workspace (the fp16 weights do not fit the
// fixed no-alloc array, and the library GEMM's first use allocates).
static bool dense_shared(const moe_layer* L, bool noalloc) {
  return !noalloc && L->has_shared && L->fmt_shared == FMT_Q8;
}

static int resolve_path(int path, int T) {
  if (path == MOE_PATH_AUTO) return T <= AUTO_DECODE_MAX_T ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
  return path;
}

// ---------------------------------------------------------------------------
// exported entry points
// ---------------------------------------------------------------------------
extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

extern "C" const char* moe_last_error(void) { return g_err.c_str(); }

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "unknown status";
  }
}

extern "C" int moe_matrix_bytes(int32_t fmt, int32_t n_experts, int32_t rows, int32_t K, size_t* bytes) {
  const char* fn = "moe_matrix_bytes";
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "%s: bytes is null", fn);
  if (!fmt_known(fmt)) return fail(MOE_ERR_UNSUPPORTED, "%s: unknown format %d", fn, fmt);
  if (n_experts < 1 || rows < 1 || K < 1 || K % k_multiple(fmt) != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: bad shape (%d experts, %d rows, K %d)", fn, n_experts, rows, K);
  *bytes = (size_t)matrix_bytes(fmt, n_experts, rows, K);
  return ok();
}

extern "C" int moe_workspace_bytes(const moe_layer* L, int32_t T, int32_t op, size_t* bytes) {
  const char* fn = "moe_workspace_bytes";
  if (!L || !bytes) return fail(MOE_ERR_INVALID_ARG, "%s: null argument", fn);
  int rc = check_T(fn, T);
  if (rc) return rc;
  if (op == MOE_OP_ROUTE) {
    if (L->n_experts < 1 || L->n_experts > MAX_EXPERTS)
      return fail(MOE_ERR_INVALID_ARG, "%s: n_experts %d not in [1, %d]", fn, L->n_experts, MAX_EXPERTS);
    *bytes = ws_route(L->n_experts, T);
    return ok();
  }
  rc = check_dims(fn, L->n_experts, L->d_model, L->top_k);
  if (rc) return rc;
  if (!pow2_in(L->d_ff, 256, 8192)) return fail(MOE_ERR_INVALID_ARG, "%s: d_ff %d is not a power of two in [256, 8192]", fn, L->d_ff);
  const int E = L->n_experts, d = L->d_model, f = L->d_ff, k = L->top_k, sh = L->has_shared ? 1 : 0;
  switch (op) {
    case MOE_OP_DECODE: *bytes = ws_decode(T, k, d, f); break;
    case MOE_OP_PREFILL: *bytes = ws_prefill(E, T, k, d, f, sh, dense_shared(L, false)); break;
    case MOE_OP_LAYER: {
      size_t b = ws_layer(E, T, k, d, f, sh, dense_shared(L, false), MOE_PATH_PREFILL);
      if (T <= AUTO_DECODE_MAX_T) {
        const size_t b2 = ws_layer(E, T, k, d, f, sh, false, MOE_PATH_DECODE);
        if (b2 > b) b = b2;
      }
      *bytes = b;
      break;
    }
    default: return fail(MOE_ERR_INVALID_ARG, "%s: unknown op %d", fn, op);
  }
  return ok();
}

extern "C" int moe_repack(int32_t fmt, int32_t n_experts, int32_t rows, int32_t K, const void* src, void* dst,
                          int32_t direction, void* stream) {
  const char* fn = "moe_repack";
  if (!fmt_known(fmt)) return fail(MOE_ERR_UNSUPPORTED, "%s: unknown format %d", fn, fmt);
  if (n_experts < 1 || rows < 1 || K < 1 || K % k_multiple(fmt) != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: bad shape (%d experts, %d rows, K %d)", fn, n_experts, rows, K);
  if (direction != MOE_REPACK_TO_DEVICE && direction != MOE_REPACK_TO_CANONICAL)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown direction %d", fn, direction);
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "%s: null buffer", fn);
  if (src == dst) return fail(MOE_ERR_INVALID_ARG, "%s: src and dst must be distinct buffers", fn);
  hipStream_t s = (hipStream_t)stream;
  const int pid = prof_begin("repack", s);
  hipError_t e = launch_repack(fmt, (int64_t)n_experts * rows, K, src, dst, direction == MOE_REPACK_TO_DEVICE, s);
  prof_end(pid, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

extern "C" int moe_prepare_weights(const moe_layer* canonical, moe_layer* device_out, void* stream) {
  const char* fn = "moe_prepare_weights";
  int rc = check_layer(fn, canonical, false, MOE_LAYOUT_CANONICAL);
  if (rc) return rc;
  if (!device_out) return fail(MOE_ERR_INVALID_ARG, "%s: device_out is null", fn);
  const moe_layer& C = *canonical;
  struct Job {
    const char* name;
    const void* src;
    const void* dst;
    int fmt, E, rows, K;
  };
  Job jobs[6] = {
      {"w_gate", C.w_gate, device_out->w_gate, C.fmt_gate_up, C.n_experts, C.d_ff, C.d_model},
      {"w_up", C.w_up, device_out->w_up, C.fmt_gate_up, C.n_experts, C.d_ff, C.d_model},
      {"w_down", C.w_down, device_out->w_down, C.fmt_down, C.n_experts, C.d_model, C.d_ff},
      {"s_gate", C.s_gate, device_out->s_gate, C.fmt_shared, 1, C.d_ff, C.d_model},
      {"s_up", C.s_up, device_out->s_up, C.fmt_shared, 1, C.d_ff, C.d_model},
      {"s_down", C.s_down, device_out->s_down, C.fmt_shared, 1, C.d_model, C.d_ff},
  };
  const int n_jobs = C.has_shared ? 6 : 3;
  for (int i = 0; i < n_jobs; i++) {  // every destination, before anything is enqueued
    const Job& j = jobs[i];
    if (!j.dst) return fail(MOE_ERR_INVALID_ARG, "%s: device_out->%s is null", fn, j.name);
    if (!aligned16(j.dst)) return fail(MOE_ERR_INVALID_ARG, "%s: device_out->%s is not 16-byte aligned", fn, j.name);
    const size_t bytes = (size_t)matrix_bytes(j.fmt, j.E, j.rows, j.K);
    const uintptr_t d0 = (uintptr_t)j.dst, d1 = d0 + bytes;
    for (int k = 0; k < n_jobs; k++) {  // no destination may overlap a source or another destination
      const Job& o = jobs[k];
      const size_t ob = (size_t)matrix_bytes(o.fmt, o.E, o.rows, o.K);
      const uintptr_t s0 = (uintptr_t)o.src, s1 = s0 + ob;
      if (d0 < s1 && s0 < d1)
        return fail(MOE_ERR_INVALID_ARG, "%s: device_out->%s overlaps the canonical %s", fn, j.name, o.name);
      if (k != i) {
        const uintptr_t t0 = (uintptr_t)o.dst, t1 = t0 + ob;
        if (o.dst && d0 < t1 && t0 < d1)
          return fail(MOE_ERR_INVALID_ARG, "%s: device_out->%s overlaps device_out->%s", fn, j.name, o.name);
      }
    }
  }
  hipStream_t s = (hipStream_t)stream;
  for (int i = 0; i < n_jobs; i++) {
    const Job& j = jobs[i];
    const int pid = prof_begin("repack", s);
    hipError_t e = launch_repack(j.fmt, (int64_t)j.E * j.rows, j.K, j.src, const_cast<void*>(j.dst), 1, s);
    prof_end(pid, s);
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  moe_layer out = C;
  out.layout = MOE_LAYOUT_DEVICE;
  out.w_gate = jobs[0].dst;
  out.w_up = jobs[1].dst;
  out.w_down = jobs[2].dst;
  out.s_gate = C.has_shared ? jobs[3].dst : nullptr;
  out.s_up = C.has_shared ? jobs[4].dst : nullptr;
  out.s_down = C.has_shared ? jobs[5].dst : nullptr;
  *device_out = out;
  return ok();
}

extern "C" int moe_route_topk(const float* w_router, const float* bias, int32_t E, int32_t d, const void* x,
                              int32_t x_dtype, int32_t T, int32_t k, int32_t* idx, float* wt, void* ws,
                              size_t ws_bytes, void* stream) {
  const char* fn = "moe_route_topk";
  int rc = check_dims(fn, E, d, k);
  if (rc) return rc;
  if ((rc = check_T(fn, T)) || (rc = check_dtype(fn, x_dtype))) return rc;
  if (T == 0) return ok();
  NEED_PTR(w_router, "w_router");
  if (bias && ((uintptr_t)bias & 3u)) return fail(MOE_ERR_INVALID_ARG, "%s: bias is not 4-byte aligned", fn);
  NEED_PTR(x, "x");
  NEED_PTR(idx, "idx");
  NEED_PTR(wt, "wt");
  NEED_PTR(ws, "workspace");
  const size_t need = ws_route(E, T);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  Carve c;
  c.base = (uint8_t*)ws;
  RouteWs w;
  carve_route(c, w, E, T);
  hipStream_t s = (hipStream_t)stream;
  int pid = prof_begin(T <= ROUTER_ROWS_MAX_T ? "router_rows" : "router_tiled", s);
  hipError_t e = launch_router(w_router, E, d, x, x_dtype, T, w.z, s);
  prof_end(pid, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  pid = prof_begin("topk", s);
  e = launch_topk(w.z, T, E, k, bias, idx, wt, nullptr, nullptr, s);
  prof_end(pid, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

extern "C" int moe_bucket(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* pos, void* stream) {
  const char* fn = "moe_bucket";
  if (E < 1 || E > MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "%s: n_experts %d not in [1, %d]", fn, E, MAX_EXPERTS);
  if (k < 1 || k > TOPK_MAX_K || k > E) return fail(MOE_ERR_INVALID_ARG, "%s: top_k %d out of range", fn, k);
  int rc = check_T(fn, T);
  if (rc) return rc;
  if (T == 0) return ok();
  NEED_PTR(idx, "idx");
  NEED_PTR(counts, "counts");
  NEED_PTR(offsets, "offsets");
  NEED_PTR(perm, "perm");
  NEED_PTR(pos, "pos");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_bucket(idx, T, k, E, counts, offsets, perm, pos, nullptr, 1, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

static DecodeLaunch decode_launch(const moe_layer* L, const void* x, int x_dtype, int T) {
  DecodeLaunch D{};
  D.E = L->n_experts;
  D.d = L->d_model;
  D.f = L->d_ff;
  D.k = L->top_k;
  D.T = T;
  D.fmt_gate_up = L->fmt_gate_up;
  D.fmt_down = L->fmt_down;
  D.fmt_shared = L->fmt_shared;
  D.has_shared = L->has_shared;
  D.w_gate = L->w_gate;
  D.w_up = L->w_up;
  D.w_down = L->w_down;
  D.s_gate = L->s_gate;
  D.s_up = L->s_up;
  D.s_down = L->s_down;
  D.grid = L->iq2_grid;
  D.vq_cb = L->vq_codebook;
  D.w_router = L->w_router;
  D.x = x;
  D.x_dtype = x_dtype;
  D.router_bias = L->router_bias;
  D.down_gain = L->down_gain;
  return D;
}

static PrefillLaunch prefill_launch(const moe_layer* L, const void* x, int x_dtype, int T) {
  PrefillLaunch P{};
  P.E = L->n_experts;
  P.d = L->d_model;
  P.f = L->d_ff;
  P.k = L->top_k;
  P.T = T;
  P.fmt_gate_up = L->fmt_gate_up;
  P.fmt_down = L->fmt_down;
  P.fmt_shared = L->fmt_shared;
  P.has_shared = L->has_shared;
  P.w_gate = L->w_gate;
  P.w_up = L->w_up;
  P.w_down = L->w_down;
  P.s_gate = L->s_gate;
  P.s_up = L->s_up;
  P.s_down = L->s_down;
  P.grid = L->iq2_grid;
  P.vq_cb = L->vq_codebook;
  P.x = x;
  P.x_dtype = x_dtype;
  P.down_gain = L->down_gain;
  return P;
}

// bucketing + grouped GEMMs + combine for routes already in device memory
static int run_prefill(const char* fn, const moe_layer* L, const void* x, int x_dtype, int T, const int32_t* idx,
                       const float* wt, float* y, int32_t* bucket_out, bool dense, Carve& c, hipStream_t s) {
  const int E = L->n_experts, k = L->top_k;
  PrefillWs w;
  carve_prefill(c, w, E, T, k, L->d_model, L->d_ff, L->has_shared, dense, bucket_out != nullptr);
  if (bucket_out) {
    w.counts = bucket_out;
    w.offsets = bucket_out + E;
    w.perm = bucket_out + 2 * E + 1;
  }
  PrefillLaunch P = prefill_launch(L, x, x_dtype, T);
  P.counts = w.counts;
  P.offsets = w.offsets;
  P.tile_start = w.tile_start;
  P.perm = w.perm;
  P.pos = w.pos;
  P.idx = idx;
  P.wt = wt;
  P.x16 = w.x16;
  P.xs = w.xs;
  P.route_xs = w.route_xs;
  P.H = w.H;
  P.Hs = w.Hs;
  P.Hexp = w.Hexp;
  P.Hsexp = w.Hsexp;
  P.Hsc = w.Hsc;
  P.Hssc = w.Hssc;
  P.Ye = w.Ye;
  P.Ysh = w.Ysh;
  P.Wgu = w.Wgu;
  P.Wdn = w.Wdn;
  P.colsc = w.colsc;
  P.Dgu = w.Dgu;
  P.y = y;
  const int tile_m = PREFILL_BM;
  hipError_t e = launch_bucket(idx, T, k, E, w.counts, w.offsets, w.perm, w.pos, w.tile_start, tile_m, w.bucket_hist, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  e = launch_prefill_gemms(P, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

extern "C" int moe_expert_ffn_decode(const moe_layer* L, const void* x, int32_t x_dtype, int32_t T, const int32_t* idx,
                                     const float* wt, float* y, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_expert_ffn_decode";
  int rc = check_layer(fn, L, false);
  if (rc) return rc;
  if ((rc = check_T(fn, T)) || (rc = check_dtype(fn, x_dtype))) return rc;
  if (T > DECODE_MAX_T) return fail(MOE_ERR_INVALID_ARG, "%s: T %d above the decode limit %d", fn, T, DECODE_MAX_T);
  if (T == 0) return ok();
  NEED_PTR(x, "x");
  NEED_PTR(idx, "idx");
  NEED_PTR(wt, "wt");
  NEED_PTR(y, "y");
  NEED_PTR(ws, "workspace");
  const size_t need = ws_decode(T, L->top_k, L->d_model, L->d_ff);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  Carve c;
  c.base = (uint8_t*)ws;
  DecodeWs w;
  carve_decode(c, w, T, L->top_k, L->d_model, L->d_ff);
  DecodeLaunch D = decode_launch(L, x, x_dtype, T);
  D.idx = const_cast<int32_t*>(idx);
  D.wt = const_cast<float*>(wt);
  D.quant = w.quant;
  D.y = y;
  D.fused_topk = 0;
  hipError_t e = launch_decode(D, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

extern "C" int moe_expert_ffn_prefill(const moe_layer* L, const void* x, int32_t x_dtype, int32_t T,
                                      const int32_t* idx, const float* wt, float* y, int32_t* bucket_out, void* ws,
                                      size_t ws_bytes, void* stream) {
  const char* fn = "moe_expert_ffn_prefill";
  int rc = check_layer(fn, L, false);
  if (rc) return rc;
  if ((rc = check_T(fn, T)) || (rc = check_dtype(fn, x_dtype))) return rc;
  if ((rc = check_prefill_size(fn, T, L->top_k, L->d_model, L->d_ff))) return rc;
  if (T == 0) return ok();
  NEED_PTR(x, "x");
  NEED_PTR(idx, "idx");
  NEED_PTR(wt, "wt");
  NEED_PTR(y, "y");
  NEED_PTR(ws, "workspace");
  if (bucket_out && ((uintptr_t)bucket_out & 3u)) return fail(MOE_ERR_INVALID_ARG, "%s: bucket_out misaligned", fn);
  const bool dense = dense_shared(L, false);
  const size_t need = ws_prefill(L->n_experts, T, L->top_k, L->d_model, L->d_ff, L->has_shared, dense);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  Carve c;
  c.base = (uint8_t*)ws;
  return run_prefill(fn, L, x, x_dtype, T, idx, wt, y, bucket_out, dense, c, (hipStream_t)stream);
}

// The device array behind moe_layer_forward_noalloc: a fixed workspace in
// every device's memory, held until the process ends.  Its host-side name
// is only a stand-in; kernels get the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

// The address of the current device's `scratch`, looked up once per device
// (under a lock) and kept.
static int scratch_address(const char* fn, void** out) {
  static std::mutex mu;
  static std::vector<std::pair<int, void*>> addrs;
  int dev = 0;
  HIP_CHECK(hipGetDevice(&dev), fn);
  std::lock_guard<std::mutex> lk(mu);
  for (const auto& a : addrs)
    if (a.first == dev) {
      *out = a.second;
      return MOE_OK;
    }
  void* ptr = nullptr;
  HIP_CHECK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), fn);
  addrs.emplace_back(dev, ptr);
  *out = ptr;
  return MOE_OK;
}

// moe_layer_forward and moe_layer_forward_noalloc: validation, then the
// launches on the caller's workspace or (noalloc) on `scratch`.
static int layer_forward(const char* fn, const moe_layer* L, const void* x, int32_t x_dtype, int32_t T, float* y,
                         int32_t* idx_out, float* wt_out, int32_t path, void* ws, size_t ws_bytes, bool noalloc,
                         void* stream) {
  int rc = check_layer(fn, L, true);
  if (rc) return rc;
  if ((rc = check_T(fn, T)) || (rc = check_dtype(fn, x_dtype))) return rc;
  if (path != MOE_PATH_AUTO && path != MOE_PATH_DECODE && path != MOE_PATH_PREFILL)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  const int p = resolve_path(path, T);
  if (path == MOE_PATH_DECODE && T > DECODE_MAX_T)
    return fail(MOE_ERR_INVALID_ARG, "%s: T %d above the decode limit %d", fn, T, DECODE_MAX_T);
  if (p == MOE_PATH_PREFILL && (rc = check_prefill_size(fn, T, L->top_k, L->d_model, L->d_ff))) return rc;
  if (T == 0) return ok();
  NEED_PTR(x, "x");
  NEED_PTR(y, "y");
  if (!noalloc) NEED_PTR(ws, "workspace");
  if (idx_out && !aligned16(idx_out)) return fail(MOE_ERR_INVALID_ARG, "%s: idx_out is not 16-byte aligned", fn);
  if (wt_out && !aligned16(wt_out)) return fail(MOE_ERR_INVALID_ARG, "%s: wt_out is not 16-byte aligned", fn);
  const int E = L->n_experts, k = L->top_k;
  const bool dense = p == MOE_PATH_PREFILL && dense_shared(L, noalloc);
  const size_t need = ws_layer(E, T, k, L->d_model, L->d_ff, L->has_shared, dense, p);
  if (noalloc) {
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
      return fail(MOE_ERR_WORKSPACE,
                  "%s: this call needs %zu bytes of workspace, above the library's fixed %u-byte scratch array "
                  "(fewer tokens, or moe_layer_forward with a workspace)", fn, need, (unsigned)MOE_NOALLOC_SCRATCH_BYTES);
    if ((rc = scratch_address(fn, &ws))) return rc;
  } else if (ws_bytes < need) {
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  }
  Carve c;
  c.base = (uint8_t*)ws;
  LayerWs lw;
  carve_layer_routes(c, lw, E, T, k);
  hipStream_t s = (hipStream_t)stream;
  if (p == MOE_PATH_DECODE) {
    // MOE_PATH_AUTO may pick the decode path above its per-call limit: then
    // consecutive chunks of at most DECODE_MAX_T tokens, each a whole decode
    // call on its slices of x, y, the routes and the workspace's quantized
    // activations (reused by every chunk, in stream order)
    const int d = L->d_model;
    const int Tc = T < DECODE_MAX_T ? T : DECODE_MAX_T;
    DecodeWs w;
    carve_decode(c, w, Tc, k, d, L->d_ff);
    const size_t x_el = x_dtype == MOE_BF16 ? 2 : 4;
    for (int t0 = 0; t0 < T; t0 += Tc) {
      const int n = T - t0 < Tc ? T - t0 : Tc;
      DecodeLaunch D = decode_launch(L, static_cast<const uint8_t*>(x) + (size_t)t0 * d * x_el, x_dtype, n);
      D.z = lw.z + (size_t)t0 * E;
      D.zkey = lw.zkey + (size_t)t0 * E;
      D.idx = lw.idx + (size_t)t0 * k;
      D.wt = lw.wt + (size_t)t0 * k;
      D.idx_out = idx_out ? idx_out + (size_t)t0 * k : nullptr;
      D.wt_out = wt_out ? wt_out + (size_t)t0 * k : nullptr;
      D.quant = w.quant;
      D.y = y + (size_t)t0 * d;
      D.fused_topk = 1;
      hipError_t e = launch_decode(D, s);
      if (e != hipSuccess) return hip_fail(e, fn);
    }
    return ok();
  }
  int pid = prof_begin(T <= ROUTER_ROWS_MAX_T ? "router_rows" : "router_tiled", s);
  hipError_t e = launch_router(L->w_router, E, L->d_model, x, x_dtype, T, lw.z, s);
  prof_end(pid, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  pid = prof_begin("topk", s);
  e = launch_topk(lw.z, T, E, k, L->router_bias, lw.idx, lw.wt, idx_out, wt_out, s);
  prof_end(pid, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return run_prefill(fn, L, x, x_dtype, T, lw.idx, lw.wt, y, nullptr, dense, c, s);
}

extern "C" int moe_layer_forward(const moe_layer* L, const void* x, int32_t x_dtype, int32_t T, float* y,
                                 int32_t* idx_out, float* wt_out, int32_t path, void* ws, size_t ws_bytes,
                                 void* stream) {
  return layer_forward("moe_layer_forward", L, x, x_dtype, T, y, idx_out, wt_out, path, ws, ws_bytes, false, stream);
}

extern "C" int moe_layer_forward_noalloc(const moe_layer* L, const void* x, int32_t x_dtype, int32_t T, float* y,
                                         int32_t* idx_out, float* wt_out, int32_t path, void* stream) {
  return layer_forward("moe_layer_forward_noalloc", L, x, x_dtype, T, y, idx_out, wt_out, path, nullptr, 0, true,
                       stream);
}
