// Achievable-peak probes for the measurement harness (not part of the MoE
// layer's C ABI; built as libqmoe_probe.so).  They give the denominators
// that the kernels' roofline fractions are quoted against beside the spec
// peaks, in the spirit of the "mem_ceiling" probe of "YoungAi -- DeepSeek
// V4.1 Flash on one DGX Spark", section 4.1 (full-line loads against
// partial-line loads on that machine).
//
//   qmoe_probe_read : streams `bytes` once with 16-byte nontemporal loads,
//                     each wave reading 1 KB contiguous per load (the decode
//                     kernels' access shape), and folds them into one word
//                     per block so nothing is dead;
//   qmoe_probe_mfma : back-to-back v_mfma_f32_16x16x32_f16 on registers,
//                     eight independent accumulators per wave, no memory;
//   qmoe_probe_mfma32: the same with v_mfma_f32_32x32x16_f16, four
//                     accumulators per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_kernel(const uint8_t* __restrict__ p, size_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  // four loads in flight per thread
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i);
    const u32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i + stride);
    const u32x4_t c = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i + 2 * stride);
    const u32x4_t d = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a[i] = (_Float16)(0.001f * (float)((lane + i) & 7));
    b[i] = (_Float16)(0.001f * (float)((lane * 3 + i) & 7));
  }
  f32x4_t c[8];
#pragma unroll
  for (int j = 0; j < 8; j++) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < 8; j++) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j++) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (s == 12345.678f) sink[blockIdx.x] = s;  // (never true: keeps the chains live)
}

__global__ __launch_bounds__(256) void mfma32_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  f16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a[i] = (_Float16)(0.001f * (float)((lane + i) & 7));
    b[i] = (_Float16)(0.001f * (float)((lane * 3 + i) & 7));
  }
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  f32x16_t c[4];
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) c[j][r] = 0.f;
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < 4; j++) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) s += c[j][r];
  if (s == 12345.678f) sink[blockIdx.x] = s;  // (never true: keeps the chains live)
}

}  // namespace

extern "C" {

// Streams bytes (a multiple of 16, 16-byte aligned device buffer) with
// `blocks` blocks of 256 threads; sink holds `blocks` words.  Returns a
// hipError_t.
int qmoe_probe_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, void* stream) {
  if (!buf || !sink || blocks < 1 || (bytes & 15) || ((uintptr_t)buf & 15)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint8_t*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}

// iters x 8 MFMAs of 16x16x32 (16384 flops each) per wave, `blocks` blocks
// of 256 threads (4 waves).  Flops = blocks * 4 * iters * 8 * 16384.
int qmoe_probe_mfma(int iters, int blocks, float* sink, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return (int)hipGetLastError();
}

// iters x 4 MFMAs of 32x32x16 (32768 flops each) per wave, `blocks` blocks
// of 256 threads.  Flops = blocks * 4 * iters * 4 * 32768.
int qmoe_probe_mfma32(int iters, int blocks, float* sink, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma32_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
