// Canonical <-> device layout of a weight tensor (a bijection on bytes).
// Device copies with aligned quant streams follow the load-time payload
// re-alignment described on "YoungAi -- DeepSeek V4.1 Flash on one DGX
// Spark", section 4.4 (decode, VQ expert kernel): the file layout stays as
// it is, only the device copy changes.
#include "common.hpp"
#include "kernels.hpp"

namespace qmoe {

// A tensor is a sequence of units (blocks; whole rows for the VQ formats) of
// `ub` bytes, each cut into up to three segments; segment s of every unit
// goes, in unit order, to plane s of the device layout.
struct Segs {
  int n, ub;
  int off[3], len[3];
  int64_t start[3];  // byte offset of each plane in the device layout
};

static Segs segments(int fmt, int K, int64_t n_units) {
  Segs g{};
  auto add = [&](int len) {
    g.off[g.n] = g.n ? g.off[g.n - 1] + g.len[g.n - 1] : 0;
    g.len[g.n] = len;
    g.start[g.n] = g.n ? g.start[g.n - 1] + n_units * g.len[g.n - 1] : 0;
    g.n++;
  };
  switch (fmt) {
    case FMT_IQ2: add(2); add(64); break;
    case FMT_Q2K: add(4); add(16); add(64); break;
    case FMT_Q4K: add(4); add(12); add(128); break;
    case FMT_MX4: add(1); add(16); break;
    case FMT_Q8: add(2); add(32); break;
    default:  // VQ rows: gain, index stream, (13 bits) bit plane
      add(2);
      add(3 * K / 16);
      if (fmt == FMT_VQ13) add(K / 64);
  }
  g.ub = g.off[g.n - 1] + g.len[g.n - 1];
  return g;
}

// One thread per byte of the tensor (index c in the canonical order).
__global__ __launch_bounds__(256) void repack_kernel(Segs g, int64_t total, const uint8_t* __restrict__ src,
                                                     uint8_t* __restrict__ dst, int to_device) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total) return;
  const int64_t u = c / g.ub;
  const int o = (int)(c - u * g.ub);
  int s = 0;
  while (s + 1 < g.n && o >= g.off[s + 1]) s++;
  const int64_t dev = g.start[s] + u * g.len[s] + (o - g.off[s]);
  if (to_device)
    dst[dev] = src[c];
  else
    dst[c] = src[dev];
}

hipError_t launch_repack(int fmt, int64_t n_rows, int K, const void* src, void* dst, int to_device, hipStream_t s) {
  const int64_t n_units = is_vq(fmt) ? n_rows : n_rows * (K / block_weights(fmt));
  const Segs g = segments(fmt, K, n_units);
  const int64_t total = n_units * g.ub;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t grid = (total + threads - 1) / threads;
  QMOE_LAUNCH(repack_kernel, dim3((unsigned)grid), dim3(threads), 0, s, g, total, static_cast<const uint8_t*>(src),
              static_cast<uint8_t*>(dst), to_device);
  return hipGetLastError();
}

}  // namespace qmoe
