// Token-to-expert bucketing: a stable counting sort of the T*k routes by
// expert, so that each expert's tokens form one contiguous group and one
// pass over the expert's weights serves all of them ("YoungAi -- DeepSeek
// V4.1 Flash on one DGX Spark", section 4.4: the verify batch reads each
// chosen expert's bits once for all of its rows).
//
// Four small launches, each reading the routes once (O(T k + C E) work for
// C chunks of consecutive routes):
//   1. per chunk, the histogram of its keys (LDS integer counts: the order
//      of the increments cannot change them), stored in `pos`, which is
//      free until the last launch (C E <= T k by the choice of C; a single
//      chunk writes `counts` directly);
//   2. one block: counts[e] (sum over chunks), each chunk's count of key e
//      turned into the number of earlier routes with key e, offsets and the
//      M-tile starts;
//   3. one wave per chunk walks its routes in order, 64 at a time: lanes
//      with equal keys are grouped by ballots, each lane's rank in its group
//      is the number of lower lanes in it, and one lane per group claims the
//      group's places from the chunk's running count of that key in LDS
//      (distinct keys per claim, batches in route order: stable);
//   4. pos = the inverse of perm (and n for an out-of-range key, which has
//      no place).
// No global atomics, no host round trip.
#include "common.hpp"
#include "kernels.hpp"

namespace qmoe {

namespace {

// chunks: C <= T k / E (the histograms fit in pos), at most 1024, at least 1
int bucket_chunks(int n, int E) {
  int c = n / E;
  return c < 1 ? 1 : (c > 1024 ? 1024 : c);
}

__global__ __launch_bounds__(64) void bucket_count_kernel(const int32_t* __restrict__ idx, int n, int E, int ch,
                                                          int32_t* __restrict__ hist_out) {
  __shared__ int hist[MAX_EXPERTS];
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int i = lane; i < E; i += 64) hist[i] = 0;
  __syncthreads();
  const int r0 = c * ch, r1 = min(n, r0 + ch);
  for (int r = r0 + lane; r < r1; r += 64) {
    const int key = idx[r];
    if ((unsigned)key < (unsigned)E) atomicAdd(&hist[key], 1);
  }
  __syncthreads();
  for (int i = lane; i < E; i += 64) hist_out[(int64_t)c * E + i] = hist[i];
}

// One block of 1024 threads: thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void bucket_scan_kernel(int n, int E, int C, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ hist, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ tile_start, int tile_m) {
  __shared__ int wsum[2][16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  int cnt = 0;
  if (e < E) {
    if (C == 1) {
      cnt = counts[e];
    } else {
#pragma unroll 8
      for (int c = 0; c < C; c++) {  // chunk c's count -> routes of key e in chunks before c
        const int h = hist[(int64_t)c * E + e];
        hist[(int64_t)c * E + e] = cnt;
        cnt += h;
      }
      counts[e] = cnt;
    }
  }
  // exclusive scans over e of the counts and of the M tiles
  const int tiles = (cnt + tile_m - 1) / tile_m;
  int a = cnt, b = tiles;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ya = __shfl_up(a, o, 64), yb = __shfl_up(b, o, 64);
    if (lane >= o) {
      a += ya;
      b += yb;
    }
  }
  if (lane == 63) {
    wsum[0][wave] = a;
    wsum[1][wave] = b;
  }
  __syncthreads();
  int pa = 0, pb = 0;
  for (int w = 0; w < wave; w++) {
    pa += wsum[0][w];
    pb += wsum[1][w];
  }
  if (e < E) {
    offsets[e] = pa + a - cnt;
    if (tile_start) tile_start[e] = pb + b - tiles;
    if (e == E - 1) {
      offsets[E] = n;
      if (tile_start) tile_start[E] = pb + b;
    }
  }
}

// One wave per chunk.
__global__ __launch_bounds__(64) void bucket_place_kernel(const int32_t* __restrict__ idx, int n, int E, int ch, int C,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ hist, int32_t* __restrict__ perm) {
  __shared__ int next[MAX_EXPERTS];  // next place of key e in this chunk
  const int c = blockIdx.x, lane = threadIdx.x;
  for (int i = lane; i < E; i += 64) next[i] = offsets[i] + (C == 1 ? 0 : hist[(int64_t)c * E + i]);
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
  const int r0 = c * ch, r1 = min(n, r0 + ch);
  for (int base = r0; base < r1; base += 64) {
    const int r = base + lane;
    const int key = r < r1 ? idx[r] : -1;
    const bool ok = (unsigned)key < (unsigned)E;
    // group the lanes by key: one ballot per distinct key of the batch
    unsigned long long todo = __ballot(ok);
    int rank = 0, leader = 0, gsize = 0;
    while (todo) {
      const int l = __builtin_ctzll(todo);
      const int kl = __builtin_amdgcn_readlane(key, l);
      const unsigned long long m = __ballot(ok && key == kl);
      if (ok && key == kl) {
        rank = __popcll(m & below);
        leader = l;
        gsize = __popcll(m);
      }
      todo &= ~m;
    }
    // each group's lowest lane claims its places (distinct keys: no two
    // lanes of the wave touch one counter)
    int first = 0;
    if (ok && rank == 0) first = atomicAdd(&next[key], gsize);
    first = __shfl(first, leader, 64);
    if (ok) perm[first + rank] = r;
  }
}

__global__ __launch_bounds__(256) void bucket_inverse_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ pos) {
  const int placed = offsets[E - 1] + counts[E - 1];  // routes with a key in range
  const int stride = gridDim.x * 256;
  for (int p = blockIdx.x * 256 + threadIdx.x; p < n; p += stride) {
    if (p < placed) pos[perm[p]] = p;
    if ((unsigned)idx[p] >= (unsigned)E) pos[p] = n;  // an out-of-range route is dropped (pos = n marks it)
  }
}

}  // namespace

hipError_t launch_bucket(const int32_t* idx, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* pos, int32_t* tile_start, int tile_m, hipStream_t s) {
  const int n = T * k;
  const int C = bucket_chunks(n, E);
  const int ch = (n + C - 1) / C;
  int32_t* hist = C == 1 ? counts : pos;  // C E <= n when C > 1
  QMOE_LAUNCH(bucket_count_kernel, dim3(C), dim3(64), 0, s, idx, n, E, ch, hist);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  QMOE_LAUNCH(bucket_scan_kernel, dim3(1), dim3(1024), 0, s, n, E, C, counts, hist, offsets, tile_start,
              tile_m > 0 ? tile_m : 1);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  QMOE_LAUNCH(bucket_place_kernel, dim3(C), dim3(64), 0, s, idx, n, E, ch, C, offsets, hist, perm);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  QMOE_LAUNCH(bucket_inverse_kernel, dim3(blocks), dim3(256), 0, s, idx, n, E, counts, offsets, perm, pos);
  return hipGetLastError();
}

}  // namespace qmoe
