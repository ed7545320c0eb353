// Measurement probes: this device's practical ceilings, against which the path's kernels are
// reported beside the published peaks.  None of them is part of the search; each computes a
// throwaway value that exists only so that the compiler keeps the work.
//
//   k_probe_mfma      back-to-back v_mfma_f32_32x32x16_f16 on register operands, eight waves
//                     a block (two a SIMD, as in the loss product), eight independent
//                     accumulators a wave; the first wave of each block reads the shader-clock
//                     counter and the 100 MHz real-time counter around its loop, so the host
//                     gets the clock the matrix cores ran at under that load.
//   k_probe_lds       every wave of an eight-wave block streams conflict-free 16-byte LDS
//                     reads (lane l reads bytes 16 l .. 16 l + 15 of a 1 KiB row); same clocks.
//   k_probe_read      a streaming read of a device buffer with 16-byte loads, sixteen in
//                     flight a lane, each block over its own contiguous range.
//   k_probe_write     the same with 16-byte stores; k_probe_copy reads and writes (eight
//                     loads in flight, then their stores).
#include <hip/hip_runtime.h>

#include "awq_internal.h"

namespace awq {

// Written only when a probe's throwaway value hits an impossible pattern.  The array has
// external linkage (the host could read it), so the compiler cannot treat these stores, or
// the work whose result feeds them, as dead.
__device__ unsigned g_probe_sink[4];

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 512;

// The shader-clock counter and the 100 MHz real-time counter, read in one asm block that
// also waits for them (both return through lgkmcnt).  `dep` is an in/out operand: at the
// start of a loop the loop's input passes through it, at the end the loop's result, so the
// compiler can move neither the loop nor the reads across each other.
struct Stamp {
  unsigned long long shader, real;
};
__device__ __forceinline__ Stamp stamp(unsigned& dep) {
  Stamp t;
  asm volatile(
      "s_memtime %0\n\t"
      "s_memrealtime %1\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=s"(t.shader), "=s"(t.real), "+v"(dep));
  return t;
}

// clocks[2 b] = shader-clock ticks, clocks[2 b + 1] = 100 MHz ticks of block b's loop.
__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma(int iters, float seed,
                                                             unsigned long long* clocks) {
  const int lane = threadIdx.x & 63;
  floatx16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
  __syncthreads();
  // the operands are formed from the seed after the first stamp
  unsigned dep = __builtin_bit_cast(unsigned, seed);
  const Stamp t0 = stamp(dep);
  const float sd = __builtin_bit_cast(float, dep);
  half8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(sd * (float)(lane + i));
    b[i] = (_Float16)(sd * (float)(lane - i));
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  unsigned res = __builtin_bit_cast(unsigned, s);
  const Stamp t1 = stamp(res);  // after this wave's products have all completed
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1.shader - t0.shader;
    clocks[2 * blockIdx.x + 1] = t1.real - t0.real;
  }
  if (res == 0x12345678u) g_probe_sink[0] = 1u;  // never true for the host's seed
}

constexpr int kLdsBytes = 64 * 1024;

__global__ __launch_bounds__(kProbeThreads) void k_probe_lds(int iters, int step,
                                                            unsigned long long* clocks) {
  __shared__ __attribute__((aligned(16))) unsigned lds[kLdsBytes / 4];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += kProbeThreads) lds[i] = (unsigned)i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned dep = (unsigned)step;
  const Stamp t0 = stamp(dep);  // the addresses below depend on the stamp's output
  step = (int)dep;
  u32x4 x = {0u, 0u, 0u, 0u};
  // each wave walks the 64 rows of 1 KiB from its own starting row, 16 reads an iteration
  // (step = 16 from the host: a runtime value, so the reads cannot be folded)
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = (wave * 8 + it * step + j) & 63;
      const u32x4 v = *(const u32x4*)((const char*)lds + row * 1024 + lane * 16);
      x ^= v;
    }
  }
  unsigned h = x[0] ^ x[1] ^ x[2] ^ x[3];
  const Stamp t1 = stamp(h);  // after this wave's reads have all returned
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1.shader - t0.shader;
    clocks[2 * blockIdx.x + 1] = t1.real - t0.real;
  }
  if (h == 0x9e3779b9u && lane == 7) g_probe_sink[1] = h;
}

constexpr int kStreamThreads = 256;

// The stream probes give each block one contiguous 1/gridDim of the buffer (a block-wide
// stride over a contiguous range moves 6.1-6.3 TB/s here, a grid-wide stride 4.1-5.3).
__device__ __forceinline__ void block_range(long long n16, long long& b0, long long& b1) {
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  b0 = (long long)blockIdx.x * per;
  b1 = b0 + per < n16 ? b0 + per : n16;
}

constexpr int kReadBatch = 16;  // 16-byte loads in flight a lane

__global__ __launch_bounds__(kStreamThreads) void k_probe_read(const u32x4* __restrict__ src,
                                                              long long n16) {
  long long b0, b1;
  block_range(n16, b0, b1);
  u32x4 x = {0u, 0u, 0u, 0u};
  long long i = b0 + threadIdx.x;
  for (; i + (kReadBatch - 1) * kStreamThreads < b1; i += kReadBatch * kStreamThreads) {
    u32x4 v[kReadBatch];
#pragma unroll
    for (int u = 0; u < kReadBatch; ++u) v[u] = src[i + u * kStreamThreads];
#pragma unroll
    for (int u = 0; u < kReadBatch; ++u) x ^= v[u];
  }
  for (; i < b1; i += kStreamThreads) x ^= src[i];
  const unsigned h = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (h == 0x9e3779b9u) g_probe_sink[2] = h;  // keeps the loads
}

__global__ __launch_bounds__(kStreamThreads) void k_probe_write(u32x4* __restrict__ dst,
                                                               long long n16) {
  long long b0, b1;
  block_range(n16, b0, b1);
  const u32x4 v = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
  for (long long i = b0 + threadIdx.x; i < b1; i += kStreamThreads) dst[i] = v;
}

constexpr int kCopyBatch = 8;

__global__ __launch_bounds__(kStreamThreads) void k_probe_copy(const u32x4* __restrict__ src,
                                                              u32x4* __restrict__ dst,
                                                              long long n16) {
  long long b0, b1;
  block_range(n16, b0, b1);
  long long i = b0 + threadIdx.x;
  for (; i + (kCopyBatch - 1) * kStreamThreads < b1; i += kCopyBatch * kStreamThreads) {
    u32x4 v[kCopyBatch];
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) v[u] = src[i + u * kStreamThreads];
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) dst[i + u * kStreamThreads] = v[u];
  }
  for (; i < b1; i += kStreamThreads) dst[i] = src[i];
}

}  // namespace

hipError_t launch_probe_mfma(int blocks, int iters, unsigned long long* clocks,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(kProbeThreads), 0, stream, iters,
                     0.0009765625f, clocks);
  return hipGetLastError();
}

hipError_t launch_probe_lds(int blocks, int iters, unsigned long long* clocks,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_probe_lds, dim3(blocks), dim3(kProbeThreads), 0, stream, iters, 16,
                     clocks);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, long long bytes, hipStream_t stream) {
  const long long n16 = bytes / 16;
  hipLaunchKernelGGL(k_probe_read, dim3(kProbeStreamBlocks), dim3(kStreamThreads), 0, stream,
                     (const u32x4*)src, n16);
  return hipGetLastError();
}

hipError_t launch_probe_write(void* dst, long long bytes, hipStream_t stream) {
  const long long n16 = bytes / 16;
  hipLaunchKernelGGL(k_probe_write, dim3(kProbeStreamBlocks), dim3(kStreamThreads), 0, stream,
                     (u32x4*)dst, n16);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, long long bytes, hipStream_t stream) {
  const long long n16 = bytes / 16;
  hipLaunchKernelGGL(k_probe_copy, dim3(kProbeStreamBlocks), dim3(kStreamThreads), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

}  // namespace awq
