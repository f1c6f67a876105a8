// Token-to-expert bucketing: a stable counting sort of the T*k routes by
// expert, so that each expert's tokens form one contiguous group and one
// pass over the expert's weights serves all of them ("YoungAi -- DeepSeek
// V4.1 Flash on one DGX Spark", section 4.4: the verify batch reads each
// chosen expert's bits once for all of its rows).
//
// One block per expert e.  Every block builds the full histogram in LDS
// (integer counts, so the order of the atomic increments cannot change the
// result), derives its own offset and M-tile start, then scans the routes
// in order and places those with key e with a wave ballot + block prefix,
// which keeps them in route order (stable).  No global atomics, no host
// round trip: the GEMMs that follow read counts, offsets and tile starts
// from device memory.
#include "common.hpp"
#include "kernels.hpp"

namespace qmoe {

__device__ __forceinline__ int block_sum_256(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(256) void bucket_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ pos,
                                                     int32_t* __restrict__ tile_start, int tile_m) {
  __shared__ int hist[MAX_EXPERTS];
  __shared__ int red[4];
  __shared__ int wcnt[4];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < E; i += 256) hist[i] = 0;
  __syncthreads();
  for (int r = tid; r < n; r += 256) {
    const int key = idx[r];
    if ((unsigned)key < (unsigned)E)
      atomicAdd(&hist[key], 1);
    else if (e == 0)
      pos[r] = n;  // an out-of-range route is dropped: no place in perm (pos = n marks it)
  }
  __syncthreads();
  int part_off = 0, part_tiles = 0;
  for (int i = tid; i < e; i += 256) {
    part_off += hist[i];
    part_tiles += (hist[i] + tile_m - 1) / tile_m;
  }
  const int off_e = block_sum_256(part_off, red);
  const int tiles_e = block_sum_256(part_tiles, red);
  const int cnt = hist[e];
  if (tid == 0) {
    counts[e] = cnt;
    offsets[e] = off_e;
    if (tile_start) tile_start[e] = tiles_e;
    if (e == E - 1) {
      offsets[E] = n;
      if (tile_start) tile_start[E] = tiles_e + (cnt + tile_m - 1) / tile_m;
    }
  }
  if (cnt == 0) return;
  int running = 0;
  for (int base = 0; base < n; base += 256) {
    const int r = base + tid;
    const bool match = r < n && idx[r] == e;
    const unsigned long long mask = __ballot(match);
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) wcnt[wave] = __popcll(mask);
    __syncthreads();
    int prefix = running;
    for (int w = 0; w < wave; w++) prefix += wcnt[w];
    if (match) {
      const int p = off_e + prefix + rank;
      perm[p] = r;
      pos[r] = p;
    }
    running += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    if (running >= cnt) break;  // uniform across the block
  }
}

hipError_t launch_bucket(const int32_t* idx, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* pos, int32_t* tile_start, int tile_m, hipStream_t s) {
  const int n = T * k;
  QMOE_LAUNCH(bucket_kernel, dim3(E), dim3(256), 0, s, idx, n, E, counts, offsets, perm, pos, tile_start,
              tile_m > 0 ? tile_m : 1);
  return hipGetLastError();
}

}  // namespace qmoe
