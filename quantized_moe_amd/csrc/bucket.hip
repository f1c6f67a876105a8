// Token-to-expert bucketing: a stable counting sort of the T*k routes by
// expert, so that each expert's tokens form one contiguous group and one
// pass over the expert's weights serves all of them ("YoungAi -- DeepSeek
// V4.1 Flash on one DGX Spark", section 4.4: the verify batch reads each
// chosen expert's bits once for all of its rows).
//
// Small launches, each reading the routes once (O(T k + C E) work for C
// chunks of consecutive routes):
//   1. per chunk, the histogram of its keys (LDS integer counts: the order
//      of the increments cannot change them), stored in a scratch array of
//      C E counts: the caller's (the prefill workspace), or else `pos`,
//      which is free until the last launch (then C E <= T k by the choice
//      of C; a single chunk writes `counts` directly);
//   2. one block: counts[e] (sum over chunks), each chunk's count of key e
//      turned into the number of earlier routes with key e, offsets and the
//      M-tile starts;
//   3. one block per chunk: a route's place is its key's offset, plus the
//      routes with that key in earlier chunks, plus those earlier in the
//      chunk (counted from the chunk's keys in LDS): stable, no atomics;
//      with a scratch array it also writes pos;
//   4. (histograms in pos) pos = the inverse of perm.
// An out-of-range key has no place (pos = n marks it).  No global atomics,
// no host round trip.
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
#pragma unroll 8
  for (int r = r0 + lane; r < r1; r += 64) {
    const int key = idx[r];
    if ((unsigned)key < (unsigned)E) atomicAdd(&hist[key], 1);
  }
  __syncthreads();
  for (int i = lane; i < E; i += 64) hist_out[(int64_t)c * E + i] = hist[i];
}

// One block of 1024 threads (E <= 1024).  Each chunk's count of key e
// becomes the number of routes with key e in the chunks before it, either
// by thread e walking the C chunks (eight loads in flight: about C / 8
// dependent load rounds), or, when that is the longer (few keys, many
// routes), by wave w taking keys w, w + 16, ... with its lanes on 64 chunks
// at a time (four loads in flight per lane, ceil(E / 16) ceil(C / 256)
// rounds) and a wave prefix sum.
__global__ __launch_bounds__(1024) void bucket_scan_kernel(int n, int E, int C, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ hist, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ tile_start, int tile_m) {
  __shared__ int wsum[2][16];
  __shared__ int s_cnt[MAX_EXPERTS];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  int cnt = 0;
  if (C == 1 || ((E + 15) / 16) * ((C + 255) / 256) * 8 >= C) {  // (uniform)
    if (e < E) {
      if (C == 1) {
        cnt = counts[e];
      } else {
#pragma unroll 8
        for (int c = 0; c < C; c++) {
          const int h = hist[(int64_t)c * E + e];
          hist[(int64_t)c * E + e] = cnt;
          cnt += h;
        }
        counts[e] = cnt;
      }
    }
  } else {
    for (int key = wave; key < E; key += 16) {  // (uniform per wave)
      int carry = 0;
      for (int c0 = 0; c0 < C; c0 += 256) {
        int h[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int c = c0 + 64 * j + lane;
          h[j] = c < C ? hist[(int64_t)c * E + key] : 0;
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
          int v = h[j];  // inclusive prefix over the wave's 64 chunks
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(v, o, 64);
            if (lane >= o) v += y;
          }
          const int c = c0 + 64 * j + lane;
          if (c < C) hist[(int64_t)c * E + key] = carry + v - h[j];
          carry += __shfl(v, 63, 64);
        }
      }
      if (lane == 0) s_cnt[key] = carry;
    }
    __syncthreads();
    if (e < E) {
      cnt = s_cnt[e];
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

// One block per chunk (ch <= PLACE_MAX_CH routes); pos_out (nullable)
// receives pos directly.  A route's place is the chunk's base for its key
// plus its rank: the number of earlier routes of the chunk with that key,
// counted from the chunk's keys in LDS (every lane of a wave reads the same
// word at a step: no bank conflicts).
constexpr int PLACE_MAX_CH = 2048;
__global__ __launch_bounds__(256) void bucket_place_kernel(const int32_t* __restrict__ idx, int n, int E, int ch, int C,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ hist, int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ pos_out) {
  __shared__ __align__(16) int skey[PLACE_MAX_CH + 4];
  __shared__ int base[MAX_EXPERTS];
  const int c = blockIdx.x, tid = threadIdx.x;
  const int r0 = c * ch, len = min(n, r0 + ch) - r0;
  for (int i = tid; i < E; i += 256) base[i] = offsets[i] + (C == 1 ? 0 : hist[(int64_t)c * E + i]);
  for (int i = tid; i < len; i += 256) skey[i] = idx[r0 + i];
  if (tid < 4) skey[len + tid] = -1;  // (a whole last quad)
  __syncthreads();
  for (int t = tid; t < len; t += 256) {
    const int key = skey[t];
    if ((unsigned)key >= (unsigned)E) {
      if (pos_out) pos_out[r0 + t] = n;
      continue;
    }
    int rank = 0;
    for (int i = 0; i < (t & ~3); i += 4) {  // whole quads before t, then the rest
      const int4 q = *reinterpret_cast<const int4*>(skey + i);
      rank += (q.x == key) + (q.y == key) + (q.z == key) + (q.w == key);
    }
    for (int i = t & ~3; i < t; i++) rank += skey[i] == key;
    const int p = base[key] + rank;
    perm[p] = r0 + t;
    if (pos_out) pos_out[r0 + t] = p;
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
                         int32_t* pos, int32_t* tile_start, int tile_m, int32_t* scratch, hipStream_t s) {
  const int n = T * k;
  const int C = bucket_chunks(n, E);
  const int ch = (n + C - 1) / C;  // <= 1.5 E + 1 for 2 <= C < 1024, < 2 E for C = 1, n / 1024 at the cap
  if (ch > PLACE_MAX_CH) return hipErrorInvalidValue;
  int32_t* hist = C == 1 ? counts : scratch ? scratch : pos;  // pos: C E <= n when C > 1
  int pid = prof_begin("bucket_count", s);
  QMOE_LAUNCH(bucket_count_kernel, dim3(C), dim3(64), 0, s, idx, n, E, ch, hist);
  prof_end(pid, s);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  pid = prof_begin("bucket_scan", s);
  QMOE_LAUNCH(bucket_scan_kernel, dim3(1), dim3(1024), 0, s, n, E, C, counts, hist, offsets, tile_start,
              tile_m > 0 ? tile_m : 1);
  prof_end(pid, s);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const bool direct = C == 1 || scratch != nullptr;  // pos is not the histogram store: written by the placement
  pid = prof_begin("bucket_place", s);
  QMOE_LAUNCH(bucket_place_kernel, dim3(C), dim3(256), 0, s, idx, n, E, ch, C, offsets, hist, perm,
              direct ? pos : nullptr);
  prof_end(pid, s);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (direct) return hipSuccess;
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  pid = prof_begin("bucket_inverse", s);
  QMOE_LAUNCH(bucket_inverse_kernel, dim3(blocks), dim3(256), 0, s, idx, n, E, counts, offsets, perm, pos);
  prof_end(pid, s);
  return hipGetLastError();
}

// Scratch counts that launch_bucket can take for n routes and E keys.
size_t bucket_scratch_ints(int n, int E) { return (size_t)bucket_chunks(n, E) * (size_t)E; }

}  // namespace qmoe
