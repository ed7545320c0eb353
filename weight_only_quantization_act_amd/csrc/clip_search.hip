// Clip search after the scale search: for every (row, group) of the scaled weight, the
// ratio rho of a grid that shrinks the group's quantisation range with the smallest output
// error of the group's own partial product.
//
// Pages: "AWQ" scholia-log notes, closing note (the practical algorithm searches a
// restricted family and may add clipping) and §2.3 (the quantiser rounds and clips); §1.1
// (the output error is the weight error times the activations).
//
// The group error is e = sum_t (sum_{i in G} d_i x_{t,i})^2 = d^T G_j d, with d the group's
// weight error and G_j = X_j^T X_j the Gram matrix of the group's activation columns.
// Forming the g x g Gram matrices once (N K g multiply-adds) and then one g x g quadratic
// form per (row, group, ratio) (M K g n_ratio) costs g / N of the direct products, and all
// ratios share the Gram matrix.
//
//   k_group_gram   fp64 sums of fp16 products (exact products, fp64 accumulation) over
//                  token splits, one 64 x 64 (or g x g) tile of one group per block, a
//                  4 x 4 (2 x 2) register tile per thread; k_gram_reduce adds the splits
//                  in order and rounds to fp32.
//   k_clip_search  one block per (group, row range).  A lane owns one (row, ratio) pair:
//                  it quantises the row's group with its ratio in fp32 exactly as the pack
//                  does, forms d = (v - Q(v)) / s, and evaluates d^T G d in fp32.  Every
//                  lane needs the same Gram element at the same time, so G is read with
//                  scalar loads into SGPRs, which the FMAs take as an operand (an LDS
//                  broadcast would still return 1 KiB per wave per 16 bytes of G through the
//                  LDS port and bound the kernel there).  Pairs of one row sit in one wave,
//                  so the first smallest error is picked through LDS.
#include <hip/hip_runtime.h>

#include <math.h>

#include "awq_internal.h"
#include "quantizer.h"

namespace awq {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGramThreads = 256;
constexpr int kGramTT = 32;  // tokens per LDS stage
constexpr int kGramTargetBlocks = 1024;

// partials[sp][j][a][b] = sum over the split's tokens of X[t][j g + a] X[t][j g + b].
template <int TS>
__global__ __launch_bounds__(kGramThreads) void k_group_gram(const uint16_t* __restrict__ X,
                                                             int N, int K, int g, int splits,
                                                             int tokens_per_split,
                                                             double* __restrict__ partials) {
  constexpr int R = TS / 16;  // outputs per thread along each side
  __shared__ float As[kGramTT][TS];
  __shared__ float Bs[kGramTT][TS];
  const int tiles_side = g / TS;
  const int tiles = tiles_side * tiles_side;
  const int j = blockIdx.x / tiles;
  const int tile = blockIdx.x - j * tiles;
  const int ta = tile / tiles_side, tb = tile - (tile / tiles_side) * tiles_side;
  const int ca = j * g + ta * TS, cb = j * g + tb * TS;
  const int sp = blockIdx.y;
  const int t_begin = sp * tokens_per_split;
  const int t_end = min(N, t_begin + tokens_per_split);
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid - (tid / 16) * 16;

  double acc[R][R];
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < R; ++b) acc[a][b] = 0.0;

  constexpr int kChunksPerRow = TS / 8;                // 16-byte loads per token row
  constexpr int kLoaders = kGramTT * kChunksPerRow;    // threads that load one tile
  for (int t0 = t_begin; t0 < t_end; t0 += kGramTT) {
    if (tid < kLoaders) {
      const int r = tid / kChunksPerRow, c = (tid - r * kChunksPerRow) * 8;
      const int t = t0 + r;
      u32x4 ra = {0u, 0u, 0u, 0u}, rb = {0u, 0u, 0u, 0u};
      if (t < t_end) {
        ra = *(const u32x4*)(X + (size_t)t * K + ca + c);
        rb = *(const u32x4*)(X + (size_t)t * K + cb + c);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        As[r][c + 2 * e] = h2f((uint16_t)(ra[e] & 0xffffu));
        As[r][c + 2 * e + 1] = h2f((uint16_t)(ra[e] >> 16));
        Bs[r][c + 2 * e] = h2f((uint16_t)(rb[e] & 0xffffu));
        Bs[r][c + 2 * e + 1] = h2f((uint16_t)(rb[e] >> 16));
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int t = 0; t < kGramTT; ++t) {
      double av[R], bv[R];
#pragma unroll
      for (int a = 0; a < R; ++a) av[a] = (double)As[t][ty * R + a];
#pragma unroll
      for (int b = 0; b < R; ++b) bv[b] = (double)Bs[t][tx * R + b];
#pragma unroll
      for (int a = 0; a < R; ++a)
#pragma unroll
        for (int b = 0; b < R; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
  double* out = partials + ((size_t)sp * (K / g) + j) * (size_t)g * g;
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int b = 0; b < R; ++b)
      out[(size_t)(ta * TS + ty * R + a) * g + tb * TS + tx * R + b] = acc[a][b];
}

__global__ __launch_bounds__(256) void k_gram_reduce(const double* __restrict__ partials,
                                                     long long n, int splits,
                                                     float* __restrict__ G) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  double v = partials[i];
  for (int sp = 1; sp < splits; ++sp) v += partials[(size_t)sp * n + i];
  G[i] = (float)v;
}

constexpr int kClipThreads = 256;
constexpr int kClipWaves = kClipThreads / 64;

// One (row, ratio) pair per lane; rows_per_wave = 64 / n_ratio rows of pairs per wave.
// red: [kClipWaves][64] errors of the current pass.
template <int GS>
__global__ __launch_bounds__(kClipThreads) void k_clip_search(
    const uint16_t* __restrict__ W, const float* __restrict__ s_in, const float* __restrict__ G,
    int M, int K, int w_bit, int zero_point, ClipList ratios, int n_ratio, int rows_per_block,
    float* __restrict__ clip_out, int32_t* __restrict__ best_out, float* __restrict__ errors) {
  __shared__ float ss[GS], rs[GS];
  __shared__ float red[kClipWaves][64];
  const int j = blockIdx.x;
  const int ngroups = K / GS;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* __restrict__ Gj = G + (size_t)j * GS * GS;
  for (int i = tid; i < GS; i += kClipThreads) {
    const float sv = s_in[j * GS + i];
    ss[i] = sv;
    rs[i] = 1.0f / sv;
  }
  __syncthreads();

  const int rows_per_wave = 64 / n_ratio;
  const int r_local = lane / n_ratio;
  const int k = lane - r_local * n_ratio;
  const bool active = r_local < rows_per_wave;
  const int rows_per_pass = rows_per_wave * kClipWaves;
  const int m_begin = blockIdx.y * rows_per_block;
  const int m_end = min(M, m_begin + rows_per_block);
  const bool zp = zero_point != 0;
  const float rho = active ? ratios.v[k] : 1.0f;

  for (int p0 = m_begin; p0 < m_end; p0 += rows_per_pass) {
    const int m = p0 + wave * rows_per_wave + r_local;
    const bool live = active && m < m_end;
    float e = 0.0f;
    if (live) {
      float d[GS];
      // scaled weights v = w * s (one rounding, as the pack computes them)
      const uint16_t* wr = W + (size_t)m * K + (size_t)j * GS;
#pragma unroll
      for (int c = 0; c < GS; c += 8) {
        const u32x4 raw = *(const u32x4*)(wr + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          d[c + 2 * q] = h2f((uint16_t)(raw[q] & 0xffffu)) * ss[c + 2 * q];
          d[c + 2 * q + 1] = h2f((uint16_t)(raw[q] >> 16)) * ss[c + 2 * q + 1];
        }
      }
      // the group's step and zero with the range shrunk by rho, as in the pack
      float st, z, lo_code, hi_code;
      if (zp) {
        float hi = d[0], lo = d[0];
#pragma unroll
        for (int i = 1; i < GS; ++i) {
          hi = fmaxf(hi, d[i]);
          lo = fminf(lo, d[i]);
        }
        hi = fmaxf(hi, 0.0f) * rho;
        lo = fminf(lo, 0.0f) * rho;
        const float top = (float)((1 << w_bit) - 1);
        st = (hi - lo) / top;
        if (st == 0.0f) st = 1.0f;
        z = fminf(fmaxf(rintf(-lo / st), 0.0f), top);
        lo_code = 0.0f;
        hi_code = top;
      } else {
        float mag = fabsf(d[0]);
#pragma unroll
        for (int i = 1; i < GS; ++i) mag = fmaxf(mag, fabsf(d[i]));
        mag *= rho;
        const float qmax = (float)((1 << (w_bit - 1)) - 1);
        st = mag / qmax;
        if (st == 0.0f) st = 1.0f;
        z = (float)(1 << (w_bit - 1));
        lo_code = z - qmax;
        hi_code = z + qmax;
      }
      // d = (v - (code - z) * step) / s
#pragma unroll
      for (int i = 0; i < GS; ++i) {
        const float code = fminf(fmaxf(rintf(d[i] / st) + z, lo_code), hi_code);
        d[i] = (d[i] - (code - z) * st) * rs[i];
      }
      // e = d^T G d; row a of G is wave-uniform (scalar loads), d[a + 1] is fetched one
      // row ahead
      float da = d[0];
      for (int a = 0; a < GS; ++a) {
        const float dn = d[a + 1 < GS ? a + 1 : a];
        const float* __restrict__ Ga = Gj + a * GS;
        float u = 0.0f;
#pragma unroll
        for (int b = 0; b < GS; ++b) u = fmaf(Ga[b], d[b], u);
        e = fmaf(da, u, e);
        da = dn;
      }
      if (errors) errors[((size_t)k * M + m) * ngroups + j] = e;
    }
    red[wave][lane] = e;
    __syncthreads();
    if (live && k == 0) {
      int best = -1;
      float be = 0.0f;
      for (int q = 0; q < n_ratio; ++q) {
        const float v = red[wave][r_local * n_ratio + q];
        if (v == v && fabsf(v) != INFINITY && (best < 0 || v < be)) {
          best = q;
          be = v;
        }
      }
      clip_out[(size_t)m * ngroups + j] = best >= 0 ? ratios.v[best] : 1.0f;
      if (best_out) best_out[(size_t)m * ngroups + j] = best;
    }
    __syncthreads();
  }
}

}  // namespace

int gram_splits(int64_t N, int64_t K, int group_size) {
  const int ts = group_size < 64 ? group_size : 64;
  const int64_t blocks = (K / group_size) * (int64_t)(group_size / ts) * (group_size / ts);
  int64_t sp = blocks > 0 ? (kGramTargetBlocks + blocks - 1) / blocks : 1;
  const int64_t by_tokens = (N + 255) / 256;  // at least 256 tokens per split
  if (sp > by_tokens) sp = by_tokens;
  if (sp < 1) sp = 1;
  if (sp > 64) sp = 64;
  return (int)sp;
}

hipError_t launch_group_gram(const uint16_t* X, int N, int K, int group_size, int splits,
                             double* partials, float* G, hipStream_t stream) {
  if (K <= 0) return hipSuccess;
  const int ts = group_size < 64 ? group_size : 64;
  const int tiles = (group_size / ts) * (group_size / ts);
  const int tps = (N + splits - 1) / splits;
  dim3 grid((K / group_size) * tiles, splits);
  if (ts == 64)
    hipLaunchKernelGGL(k_group_gram<64>, grid, dim3(kGramThreads), 0, stream, X, N, K,
                       group_size, splits, tps, partials);
  else if (ts == 32)
    hipLaunchKernelGGL(k_group_gram<32>, grid, dim3(kGramThreads), 0, stream, X, N, K,
                       group_size, splits, tps, partials);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = (long long)K * group_size;
  hipLaunchKernelGGL(k_gram_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     partials, n, splits, G);
  return hipGetLastError();
}

hipError_t launch_clip_search(const uint16_t* W, const float* s, const float* G, int M, int K,
                              int w_bit, int group_size, int zero_point, const ClipList& ratios,
                              int n_ratio, float* clip_out, int32_t* best_out, float* errors,
                              hipStream_t stream) {
  if (M <= 0 || K <= 0) return hipSuccess;
  if (n_ratio < 1 || n_ratio > 64) return hipErrorInvalidValue;
  const int rows_per_pass = (64 / n_ratio) * kClipWaves;
  // about 4 passes per block, and enough blocks to fill the chip
  int rows = rows_per_pass * 4;
  const int ngroups = K / group_size;
  while (rows > rows_per_pass && (int64_t)ngroups * ((M + rows - 1) / rows) < 2048)
    rows -= rows_per_pass;
  dim3 grid(ngroups, (M + rows - 1) / rows);
#define AWQ_CLIP(GS)                                                                        \
  hipLaunchKernelGGL(k_clip_search<GS>, grid, dim3(kClipThreads), 0, stream, W, s, G, M, K, \
                     w_bit, zero_point, ratios, n_ratio, rows, clip_out, best_out, errors)
  switch (group_size) {
    case 32: AWQ_CLIP(32); break;
    case 64: AWQ_CLIP(64); break;
    case 128: AWQ_CLIP(128); break;
    default: return hipErrorInvalidValue;
  }
#undef AWQ_CLIP
  return hipGetLastError();
}

}  // namespace awq
