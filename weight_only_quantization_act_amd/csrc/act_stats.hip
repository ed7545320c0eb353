// Per-input-channel mean activation magnitude a_i = (1/N) sum_t |X[t][i]|.
//
// Pages: "AWQ" scholia-log notes §1.2 (a_i = E|x_i| from calibration activations);
// "AWQ量化" tutorial, 激活感知 (importance = average absolute activation over N samples);
// ewbang.com GPTQ与AWQ §3 二.2 (max |A|); kwkr.cn AWQ 技术解析 §1.2 (E|a| / sqrt(E a^2)) and
// §2.1 (EMA of batch means with momentum 0.9, running max).
//
// X is fp16 [N tokens][K channels], K contiguous, so a wave reading 64 consecutive
// 16-byte chunks of one token row streams 1 KiB of contiguous HBM.  Pass 1: a block owns
// 512 channels (64 chunk lanes) and one slice of tokens, which its 4 waves stride through;
// each lane accumulates |x| for its 8 channels in fp64.  The 4 waves' sums are combined in
// a fixed order through LDS and written as one fp64 partial per (slice, channel).
// Pass 2 adds the slices in order, divides by N in fp64 and rounds to fp32.
//
// The same two passes compute the other statistics the pages name: max |x| (a running
// max instead of a sum), E|x| / sqrt(E x^2) (a second fp64 sum of squares), and an
// exponential moving average of per-batch mean |x| over consecutive token batches (the
// splits are then whole batches cut into pieces, and pass 2 runs the recurrence over the
// batches in order).
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
constexpr int kMinTokensPerSplit = 32;
constexpr int kMaxSplits = 128;
#ifndef AWQ_STATS_LOAD_BATCH
#define AWQ_STATS_LOAD_BATCH 4
#endif
// token rows a lane loads at once (same-device graph replays of the pass over 65536 x 8192
// activations: 196.5 us for 1, 175.8 for 4, 186.2 for 8, 191.9 for 16; 12.4 to 14.2 us
// for all four at 4096 x 4096)
constexpr int kLoadBatch = AWQ_STATS_LOAD_BATCH;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// max that keeps a NaN once one is seen (a plain fmax would drop it), so a NaN activation
// propagates into the statistic as it does for the sums.
__device__ __forceinline__ double nan_max(double m, double v) {
  return (v > m || v != v) ? v : m;
}

// Quantities a statistic needs per (split, channel): q0 = sum |x| (or max |x| for the max
// statistic) and, for the RMS ratio, q1 = sum x^2.
template <int MODE>
struct StatQ {
  static constexpr int NQ = (MODE == kStatRmsRatio) ? 2 : 1;
};

// Split s covers tokens [b*B + j*tpb, min(+tpb, (b+1)*B, N)) with b = s / sub, j = s % sub:
// whole batches of B tokens, each cut into `sub` pieces (B = N, one batch, except for the
// EMA statistic).
template <bool VEC, int MODE>
__global__ __launch_bounds__(kThreads) void k_act_stats_partial(const uint16_t* __restrict__ X,
                                                                int N, int K, int B, int sub,
                                                                int tpb,
                                                                double* __restrict__ part,
                                                                int splits) {
  constexpr int NQ = StatQ<MODE>::NQ;
  __shared__ double red[NQ][kTokenLanes][kChunkLanes][8];
  const int lc = threadIdx.x % kChunkLanes;
  const int lt = threadIdx.x / kChunkLanes;
  const int col0 = (blockIdx.x * kChunkLanes + lc) * 8;
  const int split = blockIdx.y;
  const int b = split / sub, j = split - (split / sub) * sub;
  const long long t0l = (long long)b * B + (long long)j * tpb;
  const int t0 = (int)min(t0l, (long long)N);
  const int t1 = (int)min(min(t0l + tpb, (long long)(b + 1) * B), (long long)N);

  double q0[8], q1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q0[i] = q1[i] = 0.0;

  auto add = [&](int i, float xf) {
    const double x = (double)xf;
    if constexpr (MODE == kStatMaxAbs) {
      q0[i] = nan_max(q0[i], fabs(x));
    } else {
      q0[i] += fabs(x);
      if constexpr (MODE == kStatRmsRatio) q1[i] += x * x;
    }
  };

  if (VEC) {
    if (col0 < K) {
      // kLoadBatch rows are loaded before any is added, so a wave keeps that many 1 KiB
      // reads in flight (one at a time leaves a short split waiting out each round trip).
      // Rows past the split's end load as zeros, which change no statistic: |0| adds
      // nothing to a sum or a sum of squares and never exceeds a running max.
      const uint16_t* xc = X + col0;
      for (int t = t0 + lt; t < t1; t += kLoadBatch * kTokenLanes) {
        u32x4 raw[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
          const int tt = t + u * kTokenLanes;
          raw[u] = tt < t1 ? *(const u32x4*)(xc + (size_t)tt * K) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            add(2 * jj, h2f((uint16_t)(raw[u][jj] & 0xffffu)));
            add(2 * jj + 1, h2f((uint16_t)(raw[u][jj] >> 16)));
          }
      }
    }
  } else {
    for (int t = t0 + lt; t < t1; t += kTokenLanes) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (col0 + i < K) add(i, h2f(X[(size_t)t * K + col0 + i]));
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    red[0][lt][lc][i] = q0[i];
    if constexpr (NQ > 1) red[NQ - 1][lt][lc][i] = q1[i];
  }
  __syncthreads();
  if (lt == 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        double v = red[q][0][lc][i];
#pragma unroll
        for (int u = 1; u < kTokenLanes; ++u)
          v = (MODE == kStatMaxAbs) ? nan_max(v, red[q][u][lc][i]) : v + red[q][u][lc][i];
        if (col0 + i < K) part[((size_t)q * splits + split) * K + col0 + i] = v;
      }
  }
}

// Pass 2 (mean, max, RMS ratio): a block owns 64 channels; its 4 waves take interleaved
// slices of the splits (wave u: splits u, u+4, ... in order) and the 4 partial results are
// combined in a fixed order.
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_act_stats_finalize(const double* __restrict__ part,
                                                                 int splits, int N, int K,
                                                                 float* __restrict__ a) {
  constexpr int NQ = StatQ<MODE>::NQ;
  __shared__ double red[NQ][kTokenLanes][kChunkLanes];
  const int lc = threadIdx.x % kChunkLanes;
  const int lt = threadIdx.x / kChunkLanes;
  const int i = blockIdx.x * kChunkLanes + lc;
  double s0 = 0.0, s1 = 0.0;
  if (i < K) {
#pragma unroll 4
    for (int p = lt; p < splits; p += kTokenLanes) {
      const double v = part[(size_t)p * K + i];
      s0 = (MODE == kStatMaxAbs) ? nan_max(s0, v) : s0 + v;
      if constexpr (NQ > 1) s1 += part[((size_t)splits + p) * K + i];
    }
  }
  red[0][lt][lc] = s0;
  if constexpr (NQ > 1) red[NQ - 1][lt][lc] = s1;
  __syncthreads();
  if (lt == 0 && i < K) {
    double t0 = red[0][0][lc], t1 = (NQ > 1) ? red[NQ - 1][0][lc] : 0.0;
#pragma unroll
    for (int u = 1; u < kTokenLanes; ++u) {
      t0 = (MODE == kStatMaxAbs) ? nan_max(t0, red[0][u][lc]) : t0 + red[0][u][lc];
      if constexpr (NQ > 1) t1 += red[NQ - 1][u][lc];
    }
    double r;
    if constexpr (MODE == kStatMeanAbs) {
      r = t0 / (double)N;
    } else if constexpr (MODE == kStatMaxAbs) {
      r = t0;
    } else {  // RMS ratio: mean |x| / sqrt(mean x^2); 0 for an all-zero channel
      const double m1 = t0 / (double)N, m2 = t1 / (double)N;
      r = (m2 > 0.0) ? m1 / sqrt(m2) : 0.0;
    }
    a[i] = (float)r;
  }
}

// Pass 2 (EMA): per channel, batch sums -> batch mean -> e = momentum * e + (1 - momentum) *
// mean, from e = 0, over the batches in order.  A wave covers 16 channels with 4 lanes
// each: lane slot q sums the batch's pieces q, q + 4, ..., and the four slots are added
// across lanes.  The pieces are exact fp64 sums of fp16 magnitudes (while a batch's sum
// stays below 2^29), so any order of these additions gives the same batch sum; every lane
// of a channel then runs the same recurrence and slot 0 writes the result.
constexpr int kEmaSlots = 4;
constexpr int kEmaChannelsPerBlock = kThreads / kEmaSlots;
__global__ __launch_bounds__(kThreads) void k_act_stats_ema(const double* __restrict__ part,
                                                            int n_batches, int sub, int N, int B,
                                                            int K, double momentum,
                                                            float* __restrict__ a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4;  // slot 0..3
  const int i = blockIdx.x * kEmaChannelsPerBlock + wave * 16 + (lane & 15);
  const bool ok = i < K;
  const double keep = 1.0 - momentum;
  double e = 0.0;
  for (int b = 0; b < n_batches; ++b) {
    double sum = 0.0;
    if (ok)
      for (int j = q; j < sub; j += kEmaSlots) sum += part[(size_t)(b * sub + j) * K + i];
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    const int cnt = (int)min((long long)B, (long long)N - (long long)b * B);
    const double m = sum / (double)cnt;
    e = momentum * e + keep * m;
  }
  if (ok && q == 0) a[i] = (float)e;
}

}  // namespace

StatsPlan stats_plan(int64_t N, int64_t K, int mode, int64_t batch_tokens) {
  StatsPlan p{};
  p.nq = (mode == kStatRmsRatio) ? 2 : 1;
  if (N <= 0 || K <= 0) {
    p.B = (int)(N > 0 ? N : 1); p.n_batches = 1; p.sub = 1; p.tpb = p.B; p.splits = 1;
    return p;
  }
  const int64_t col_blocks = (K + kChunkLanes * 8 - 1) / (kChunkLanes * 8);
  const int64_t target = (kTargetBlocks + col_blocks - 1) / col_blocks;
  if (mode == kStatEmaMean) {
    const int64_t B = batch_tokens < N ? batch_tokens : N;  // one batch if it covers all
    p.B = (int)B;
    p.n_batches = (int)((N + B - 1) / B);
    int64_t sub = target / p.n_batches;
    const int64_t by_tokens = (B + kMinTokensPerSplit - 1) / kMinTokensPerSplit;
    if (sub > by_tokens) sub = by_tokens;
    if (sub < 1) sub = 1;
    p.sub = (int)sub;
    p.tpb = (int)((B + sub - 1) / sub);
    p.splits = p.n_batches * p.sub;
  } else {
    int64_t by_tokens = (N + kMinTokensPerSplit - 1) / kMinTokensPerSplit;
    int64_t s = target < by_tokens ? target : by_tokens;
    if (s > kMaxSplits) s = kMaxSplits;
    if (s < 1) s = 1;
    p.B = (int)N;
    p.n_batches = 1;
    p.sub = (int)s;
    p.tpb = (int)((N + s - 1) / s);
    p.splits = (int)s;
  }
  return p;
}

template <int MODE>
static hipError_t launch_stats_mode(const uint16_t* X, int N, int K, const StatsPlan& p,
                                    double momentum, float* a_out, double* partials,
                                    hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int col_blocks = (K + kChunkLanes * 8 - 1) / (kChunkLanes * 8);
  dim3 grid(col_blocks, p.splits);
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, stream);
    if (e != hipSuccess) return e;
  }
  if (K % 8 == 0)
    hipLaunchKernelGGL((k_act_stats_partial<true, MODE>), grid, dim3(kThreads), 0, stream, X, N, K,
                       p.B, p.sub, p.tpb, partials, p.splits);
  else
    hipLaunchKernelGGL((k_act_stats_partial<false, MODE>), grid, dim3(kThreads), 0, stream, X, N,
                       K, p.B, p.sub, p.tpb, partials, p.splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  if constexpr (MODE == kStatEmaMean) {
    hipLaunchKernelGGL(k_act_stats_ema,
                       dim3((K + kEmaChannelsPerBlock - 1) / kEmaChannelsPerBlock), dim3(kThreads), 0,
                       stream, partials, p.n_batches, p.sub, N, p.B, K, momentum, a_out);
  } else {
    hipLaunchKernelGGL(k_act_stats_finalize<MODE>, dim3((K + kChunkLanes - 1) / kChunkLanes),
                       dim3(kThreads), 0, stream, partials, p.splits, N, K, a_out);
  }
  return hipGetLastError();
}

hipError_t launch_act_stats(const uint16_t* X, int N, int K, int mode, const StatsPlan& plan,
                            double momentum, float* a_out, double* partials, hipStream_t stream,
                            hipEvent_t ev0, hipEvent_t ev1) {
  if (K <= 0) return hipSuccess;
  switch (mode) {
    case kStatMeanAbs:
      return launch_stats_mode<kStatMeanAbs>(X, N, K, plan, momentum, a_out, partials, stream,
                                             ev0, ev1);
    case kStatMaxAbs:
      return launch_stats_mode<kStatMaxAbs>(X, N, K, plan, momentum, a_out, partials, stream,
                                            ev0, ev1);
    case kStatRmsRatio:
      return launch_stats_mode<kStatRmsRatio>(X, N, K, plan, momentum, a_out, partials, stream,
                                              ev0, ev1);
    case kStatEmaMean:
      return launch_stats_mode<kStatEmaMean>(X, N, K, plan, momentum, a_out, partials, stream,
                                             ev0, ev1);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace awq
