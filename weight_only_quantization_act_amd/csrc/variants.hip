// Variants around the scale search: percentile-threshold fixed-factor scales and a
// blockwise Hadamard rotation of weights or activations.
//
// Pages: "AWQ量化" tutorial, 显著识别 (an indicator of channels above a percentile
// threshold of the importance scores), 缩放保护 and Python 演示 (scale those channels by a
// fixed factor, 70th percentile and factor 2 in the demo); "AWQ" scholia-log notes §5.1
// (an orthogonal R keeps WX = (WR)(R^T X); a normalised Hadamard spreads an outlier
// channel over many) and §5.2 (structured rotations in O(d log d)).
#include <hip/hip_runtime.h>

#include <math.h>

#include "awq_internal.h"
#include "quantizer.h"

namespace awq {

namespace {

constexpr int kSortThreads = 1024;

// One block: bitonic sort of a (non-finite values sort last), the linear-interpolation
// percentile in fp64 (position p/100 * (K-1) between order statistics), then
// s_i = factor if a_i > threshold else 1, decided in fp64 exactly as the reference does.
__global__ __launch_bounds__(kSortThreads) void k_threshold_scales(const float* __restrict__ a,
                                                                   int K, int P, double percentile,
                                                                   float factor,
                                                                   float* __restrict__ s_out) {
  __shared__ float key[kMaxThresholdK];
  __shared__ double tau_sh;
  const int tid = threadIdx.x;
  for (int i = tid; i < P; i += kSortThreads) {
    float v = (i < K) ? a[i] : INFINITY;
    if (v != v) v = INFINITY;
    key[i] = v;
  }
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      __syncthreads();
      for (int i = tid; i < P; i += kSortThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool ascending = (i & k) == 0;
          const float x = key[i], y = key[ixj];
          if ((x > y) == ascending) {
            key[i] = y;
            key[ixj] = x;
          }
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    const double pos = percentile / 100.0 * (double)(K - 1);
    int lo = (int)floor(pos);
    if (lo > K - 1) lo = K - 1;
    const int hi = lo + 1 < K ? lo + 1 : K - 1;
    const double frac = pos - (double)lo;
    const double vlo = (double)key[lo], vhi = (double)key[hi];
    tau_sh = vlo + frac * (vhi - vlo);
  }
  __syncthreads();
  const double tau = tau_sh;
  for (int i = tid; i < K; i += kSortThreads) s_out[i] = ((double)a[i] > tau) ? factor : 1.0f;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp64 -> fp16, correctly rounded (nearest, ties to even): round to odd into fp32
// (toward zero, then set the last bit if anything was cut off), then nearest-even into
// fp16.  fp32 carries 13 more bits than fp16, so the second rounding sees the exact
// value's position relative to every fp16 midpoint and the two steps round once.
__device__ __forceinline__ uint16_t d2h_rn(double d) {
  float f = (float)d;
  if (fabs((double)f) > fabs(d)) f = nextafterf(f, 0.0f);
  if ((double)f != d) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f2h(f);
}

// Fast Walsh-Hadamard transform within aligned blocks of BLOCK channels (Sylvester order:
// butterflies (x_j + x_{j+h}, x_j - x_{j+h}) for h = 1, 2, 4, ...), scaled by 1/sqrt(BLOCK).
// A thread holds 8 consecutive channels (h < 8 in registers); a block of BLOCK channels
// spans BLOCK/8 consecutive lanes of one wave (h >= 8 by xor shuffles).  The butterflies
// run in fp64, where they are exact (fp16 values are multiples of 2^-24 below 2^16, so a
// sum of up to 512 of them needs at most 49 significant bits); the scaling is the one
// rounding, and the fp16 result is the correctly rounded value of that.  In-place use is
// safe: every thread reads its 16 bytes before any write and writes only those.
template <int BLOCK>
__global__ __launch_bounds__(256) void k_hadamard(const uint16_t* __restrict__ A, long long chunks,
                                                  double scale, uint16_t* __restrict__ out) {
  const long long chunk = (long long)blockIdx.x * 256 + threadIdx.x;
  const bool ok = chunk < chunks;
  const int lane = threadIdx.x & 63;
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (ok) raw = *(const u32x4*)(A + chunk * 8);
  double x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = (double)h2f((uint16_t)(raw[j] & 0xffffu));
    x[2 * j + 1] = (double)h2f((uint16_t)(raw[j] >> 16));
  }
  constexpr int IN = BLOCK < 8 ? BLOCK : 8;
#pragma unroll
  for (int h = 1; h < IN; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0) {
        const double p = x[i], q = x[i + h];
        x[i] = p + q;
        x[i + h] = p - q;
      }
#pragma unroll
  for (int d = 1; d < BLOCK / 8; d <<= 1) {
    const bool upper = (lane & d) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double p = __shfl_xor(x[i], d);
      x[i] = upper ? (p - x[i]) : (x[i] + p);
    }
  }
  if (ok) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = (uint32_t)d2h_rn(x[2 * j] * scale) | ((uint32_t)d2h_rn(x[2 * j + 1] * scale) << 16);
    *(u32x4*)(out + chunk * 8) = r;
  }
}

template <int BLOCK>
hipError_t launch_h(const uint16_t* A, long long chunks, double scale, uint16_t* out,
                    hipStream_t stream) {
  const long long blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(k_hadamard<BLOCK>, dim3((unsigned)blocks), dim3(256), 0, stream, A, chunks,
                     scale, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_threshold_scales(const float* a, int K, double percentile, float factor,
                                   float* s_out, hipStream_t stream) {
  if (K <= 0) return hipSuccess;
  if (K > kMaxThresholdK) return hipErrorInvalidValue;
  int P = 1;
  while (P < K) P <<= 1;
  hipLaunchKernelGGL(k_threshold_scales, dim3(1), dim3(kSortThreads), 0, stream, a, K, P,
                     percentile, factor, s_out);
  return hipGetLastError();
}

hipError_t launch_hadamard(const uint16_t* A, int rows, int K, int block, uint16_t* out,
                           hipStream_t stream) {
  if (rows <= 0 || K <= 0) return hipSuccess;
  const long long chunks = (long long)rows * K / 8;
  const double scale = 1.0 / sqrt((double)block);
  switch (block) {
    case 2: return launch_h<2>(A, chunks, scale, out, stream);
    case 4: return launch_h<4>(A, chunks, scale, out, stream);
    case 8: return launch_h<8>(A, chunks, scale, out, stream);
    case 16: return launch_h<16>(A, chunks, scale, out, stream);
    case 32: return launch_h<32>(A, chunks, scale, out, stream);
    case 64: return launch_h<64>(A, chunks, scale, out, stream);
    case 128: return launch_h<128>(A, chunks, scale, out, stream);
    case 256: return launch_h<256>(A, chunks, scale, out, stream);
    case 512: return launch_h<512>(A, chunks, scale, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace awq
