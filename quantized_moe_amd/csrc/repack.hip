// Canonical <-> device layout of a weight tensor (a bijection on bytes).
// Device copies with aligned quant streams follow the load-time payload
// re-alignment described on "YoungAi -- DeepSeek V4.1 Flash on one DGX
// Spark", section 4.4 (decode, VQ expert kernel): the file layout stays as
// it is, only the device copy changes.
#include "common.hpp"
#include "kernels.hpp"

namespace qmoe {

// One thread per block.  Block b of the canonical stream corresponds to
// entry b of every plane, because both are ordered [expert][row][block].
__global__ void repack_kernel(int fmt, int64_t n_blocks, const uint8_t* __restrict__ src,
                              uint8_t* __restrict__ dst, int to_device) {
  int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_blocks) return;
  const int bb = block_bytes(fmt);
  // (offset inside the canonical block, plane start, bytes per plane entry)
  int64_t plane0 = 0;
  int seg_off[3], seg_len[3], nseg;
  if (fmt == FMT_IQ2) {
    nseg = 2;
    seg_off[0] = 0; seg_len[0] = 2;
    seg_off[1] = 2; seg_len[1] = 64;
  } else if (fmt == FMT_Q2K) {
    nseg = 3;
    seg_off[0] = 0; seg_len[0] = 4;
    seg_off[1] = 4; seg_len[1] = 16;
    seg_off[2] = 20; seg_len[2] = 64;
  } else if (fmt == FMT_Q4K) {
    nseg = 3;
    seg_off[0] = 0; seg_len[0] = 4;
    seg_off[1] = 4; seg_len[1] = 12;
    seg_off[2] = 16; seg_len[2] = 128;
  } else if (fmt == FMT_MX4) {
    nseg = 2;
    seg_off[0] = 0; seg_len[0] = 1;
    seg_off[1] = 1; seg_len[1] = 16;
  } else {
    nseg = 2;
    seg_off[0] = 0; seg_len[0] = 2;
    seg_off[1] = 2; seg_len[1] = 32;
  }
  for (int s = 0; s < nseg; s++) {
    const int64_t canon = b * bb + seg_off[s];
    const int64_t dev = plane0 + b * seg_len[s];
    for (int i = 0; i < seg_len[s]; i++) {
      if (to_device)
        dst[dev + i] = src[canon + i];
      else
        dst[canon + i] = src[dev + i];
    }
    plane0 += n_blocks * seg_len[s];
  }
}

hipError_t launch_repack(int fmt, int64_t n_blocks, const void* src, void* dst, int to_device, hipStream_t s) {
  if (n_blocks == 0) return hipSuccess;
  const int threads = 256;
  const int64_t grid = (n_blocks + threads - 1) / threads;
  QMOE_LAUNCH(repack_kernel, dim3((unsigned)grid), dim3(threads), 0, s, fmt, n_blocks, static_cast<const uint8_t*>(src),
              static_cast<uint8_t*>(dst), to_device);
  return hipGetLastError();
}

}  // namespace qmoe
