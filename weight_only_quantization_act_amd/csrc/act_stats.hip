// Per-input-channel mean activation magnitude a_i = (1/N) sum_t |X[t][i]|.
//
// Pages: "AWQ" scholia-log notes §1.2 (a_i = E|x_i| from calibration activations);
// "AWQ量化" tutorial, 激活感知 (importance = average absolute activation over N samples).
//
// X is fp16 [N tokens][K channels], K contiguous, so a wave reading 64 consecutive
// 16-byte chunks of one token row streams 1 KiB of contiguous HBM.  Pass 1: a block owns
// 512 channels (64 chunk lanes) and one slice of tokens, which its 4 waves stride through;
// each lane accumulates |x| for its 8 channels in fp64.  The 4 waves' sums are combined in
// a fixed order through LDS and written as one fp64 partial per (slice, channel).
// Pass 2 adds the slices in order, divides by N in fp64 and rounds to fp32.
//
// fp16 values are integer multiples of 2^-24, so fp64 sums of them are exact while every
// partial sum stays below 2^29; in that range the result does not depend on the order
// of additions at all.  Outside it the fixed order still makes the result repeatable.
#include <hip/hip_runtime.h>

#include "awq_internal.h"
#include "quantizer.h"

namespace awq {

namespace {

constexpr int kThreads = 256;
constexpr int kChunkLanes = 64;                     // chunks (8 channels) per block
constexpr int kTokenLanes = kThreads / kChunkLanes;  // token strides per block
constexpr int kTargetBlocks = 1024;
constexpr int kMinTokensPerSplit = 64;
constexpr int kMaxSplits = 128;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_act_stats_partial(const uint16_t* __restrict__ X,
                                                                int N, int K,
                                                                int tokens_per_split,
                                                                double* __restrict__ part) {
  __shared__ double red[kTokenLanes][kChunkLanes][8];
  const int lc = threadIdx.x % kChunkLanes;
  const int lt = threadIdx.x / kChunkLanes;
  const int col0 = (blockIdx.x * kChunkLanes + lc) * 8;
  const int split = blockIdx.y;
  const int t0 = split * tokens_per_split;
  const int t1 = min(N, t0 + tokens_per_split);

  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;

  if (VEC) {
    if (col0 < K) {
      for (int t = t0 + lt; t < t1; t += kTokenLanes) {
        const u32x4 raw = *(const u32x4*)(X + (size_t)t * K + col0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += fabs((double)h2f((uint16_t)(raw[j] & 0xffffu)));
          acc[2 * j + 1] += fabs((double)h2f((uint16_t)(raw[j] >> 16)));
        }
      }
    }
  } else {
    for (int t = t0 + lt; t < t1; t += kTokenLanes) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (col0 + i < K) acc[i] += fabs((double)h2f(X[(size_t)t * K + col0 + i]));
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) red[lt][lc][i] = acc[i];
  __syncthreads();
  if (lt == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double s = red[0][lc][i];
#pragma unroll
      for (int u = 1; u < kTokenLanes; ++u) s += red[u][lc][i];
      if (col0 + i < K) part[(size_t)split * K + col0 + i] = s;
    }
  }
}

// Pass 2: a block owns 64 channels; its 4 waves take interleaved slices of the splits
// (wave u sums splits u, u+4, u+8, ... in order) and the 4 sums are added in a fixed
// order.  Reads are 64 consecutive doubles per wave instruction.
__global__ __launch_bounds__(kThreads) void k_act_stats_finalize(const double* __restrict__ part,
                                                                 int splits, int N, int K,
                                                                 float* __restrict__ a) {
  __shared__ double red[kTokenLanes][kChunkLanes];
  const int lc = threadIdx.x % kChunkLanes;
  const int lt = threadIdx.x / kChunkLanes;
  const int i = blockIdx.x * kChunkLanes + lc;
  double s = 0.0;
  if (i < K) {
#pragma unroll 4
    for (int p = lt; p < splits; p += kTokenLanes) s += part[(size_t)p * K + i];
  }
  red[lt][lc] = s;
  __syncthreads();
  if (lt == 0 && i < K) {
    double t = red[0][lc];
#pragma unroll
    for (int u = 1; u < kTokenLanes; ++u) t += red[u][lc];
    a[i] = (float)(t / (double)N);
  }
}

}  // namespace

int stats_splits(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 1;
  const int64_t col_blocks = (K + kChunkLanes * 8 - 1) / (kChunkLanes * 8);
  int64_t by_blocks = (kTargetBlocks + col_blocks - 1) / col_blocks;
  int64_t by_tokens = (N + kMinTokensPerSplit - 1) / kMinTokensPerSplit;
  int64_t s = by_blocks < by_tokens ? by_blocks : by_tokens;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_act_stats(const uint16_t* X, int N, int K, float* a_out, double* partials,
                            int splits, hipStream_t stream) {
  if (K <= 0) return hipSuccess;
  const int tps = (N + splits - 1) / splits;
  const int col_blocks = (K + kChunkLanes * 8 - 1) / (kChunkLanes * 8);
  dim3 grid(col_blocks, splits);
  if (K % 8 == 0)
    hipLaunchKernelGGL(k_act_stats_partial<true>, grid, dim3(kThreads), 0, stream, X, N, K, tps,
                       partials);
  else
    hipLaunchKernelGGL(k_act_stats_partial<false>, grid, dim3(kThreads), 0, stream, X, N, K,
                       tps, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_act_stats_finalize, dim3((K + kChunkLanes - 1) / kChunkLanes),
                     dim3(kThreads), 0, stream, partials, splits, N, K, a_out);
  return hipGetLastError();
}

}  // namespace awq
