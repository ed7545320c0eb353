// The output-error loss through the Gram matrix of the calibration activations, for layers
// with many more tokens than input channels.
//
// Pages: "AWQ" scholia-log notes §1.1 (the output error is Delta W X) and §4.1 (its squared
// Frobenius norm is the search objective).
//
// ||Delta W X^T||_F^2 = sum over rows r of Delta W_r G Delta W_r^T with G = X^T X (K x K).
// Forming G costs N K^2 multiply-adds once (the upper triangle); each grid point then
// costs about M K^2 / 2 (the block upper triangle of G below) instead of M K N, which
// pays once N is about as large as K.
//
//   k_transpose_x      Xt = X^T (fp16 [K][ld], tokens contiguous, ld = N rounded up to 8,
//                      the padding tokens zero), so that G = Xt Xt^T is a product of two
//                      row-contiguous operands like the loss product itself.
//   k_loss_gemm (G build mode, loss_gemm.hip)
//                      G's upper block triangle in 256 x 256 tiles on the matrix cores:
//                      fp16 products (exact in fp32) summed in fp32 over one token split
//                      of at most kGramSplitTokens tokens (at most 512 accumulator additions of
//                      32x32x16 products, so within 2^-15 of the sum of |products|).
//   k_gram_combine     with several splits: each entry the fp64 sum of its split partials
//                      in split order, rounded to fp32; each quarter tile's largest |G|.
//   k_gram_full_split  one power of two 2^-ex for the whole matrix (its largest magnitude
//                      into [2^13, 2^14)) and the operand of the per-grid-point product:
//                      G' 2^-ex in fp16, where G' is G with its blocks of kLossBN x kLossBN
//                      above the diagonal doubled (exact), those below it zero and its
//                      diagonal zero; each diagonal block has the same structure at half
//                      size (upper-right half block doubled, lower-left zero).  With d the
//                      rows of dW,
//                      sum_r d_r G d_r^T = sum over column blocks a of d_a . (G' d)_a
//                                          + sum_c (sum_r d_rc^2) G_cc,
//                      the product for column block a only runs over k from block a on
//                      (its upper half of channels from the half block on),
//                      and the diagonal term, which carries most of the sum, is taken in
//                      fp32 from gdiag = diag(G) 2^-ex (fp32) in the product's epilogue,
//                      so that only the off-diagonal entries are rounded to fp16.
//                      Only G's upper block triangle is read, and only that of G' is written.
#include <hip/hip_runtime.h>

#include <math.h>

#include "awq_internal.h"
#include "quantizer.h"

namespace awq {

namespace {

constexpr int kGfSplitChunk = 4096;  // entries per block of the split pass
constexpr int kTrTile = 64;          // tokens and channels of a transpose tile
constexpr int kCombineRows = 64;     // tile rows per block of the combine pass

__device__ __forceinline__ float nan_maxf(float m, float a) {
  return (a > m || a != a) ? a : m;
}

// Block (bx, by): tokens [64 bx, 64 bx + 64) x channels [64 by, 64 by + 64).  Loads are
// 16-byte runs of 8 channels of one token, stores 16-byte runs of 8 tokens of one channel;
// the tile passes through LDS with a row pitch of 66 halves (33 banks), so the column
// reads of the store phase spread over the banks.
__global__ __launch_bounds__(256) void k_transpose_x(const uint16_t* __restrict__ X, int N,
                                                     int K, int ld, uint16_t* __restrict__ Xt) {
  constexpr int P = kTrTile + 2;
  __shared__ uint16_t t[kTrTile * P];
  const int t0 = blockIdx.x * kTrTile, c0 = blockIdx.y * kTrTile;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = tid + 256 * i;         // 512 runs: token u / 8, channels 8 (u mod 8) ..
    const int tr = u >> 3, cc = (u & 7) * 8;
    const int tok = t0 + tr, ch = c0 + cc;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (tok < N && ch < K) v = *(const uint4*)(X + (size_t)tok * K + ch);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[tr * P + cc + 2 * j] = (uint16_t)(w[j] & 0xffffu);
      t[tr * P + cc + 2 * j + 1] = (uint16_t)(w[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = tid + 256 * i;         // 512 runs: channel u / 8, tokens 8 (u mod 8) ..
    const int cr = u >> 3, tt = (u & 7) * 8;
    const int ch = c0 + cr, tok = t0 + tt;
    if (ch < K && tok < ld) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)t[(tt + 2 * j) * P + cr] | ((uint32_t)t[(tt + 2 * j + 1) * P + cr] << 16);
      *(uint4*)(Xt + (size_t)ch * ld + tok) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Block (quarter q of pair p): rows [64 q, 64 q + 64) of tile pair p = (tm, tn): each entry
// the fp64 sum over splits of the partial tiles [split][pair][256][256] in split order,
// rounded to fp32, written to G; the quarter's largest |entry| to tmax[4 p + q].
__global__ __launch_bounds__(256) void k_gram_combine(const float* __restrict__ part,
                                                      int splits, int npairs, int T, int K,
                                                      float* __restrict__ G,
                                                      float* __restrict__ tmax) {
  __shared__ float wm[4];
  const int p = blockIdx.x >> 2, qr = blockIdx.x & 3;
  int tm = 0, left = p;
  while (left >= T - tm) {
    left -= T - tm;
    ++tm;
  }
  const int tn = tm + left;
  const int tid = threadIdx.x;
  const int col = tn * kLossBN + tid;
  float mx = 0.0f;
  for (int rr = 0; rr < kCombineRows; ++rr) {
    const int rl = qr * kCombineRows + rr;
    const int row = tm * kLossBM + rl;
    if (row >= K || col >= K) continue;
    double acc = 0.0;
    for (int sp = 0; sp < splits; ++sp)
      acc += (double)part[(((size_t)sp * npairs + p) * kLossBM + rl) * kLossBN + tid];
    const float v = (float)acc;
    G[(size_t)row * K + col] = v;
    mx = nan_maxf(mx, fabsf(v));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = nan_maxf(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) wm[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0) tmax[blockIdx.x] = nan_maxf(nan_maxf(wm[0], wm[1]), nan_maxf(wm[2], wm[3]));
}

// Block c: entries [c chunk, (c + 1) chunk) of G (K x K), eight consecutive entries of one
// row a thread (K is a multiple of 8).  Every block derives the same exponent from all tile
// maxima (NaN if any entry is NaN: then ex = 0 and the NaN reaches the losses); block 0
// publishes it.  Runs in the blocks below the diagonal are skipped: the product never reads
// them (a tile row of channels runs over k from its own diagonal block on), so G' there is
// left unwritten.
__global__ __launch_bounds__(256) void k_gram_full_split(const float* __restrict__ G, int K,
                                                         int64_t KK,
                                                         const float* __restrict__ tmax,
                                                         int ntiles, uint16_t* __restrict__ Gh,
                                                         float* __restrict__ gdiag,
                                                         int32_t* __restrict__ gexp) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  float m = 0.0f;
  for (int i = tid; i < ntiles; i += 256) m = nan_maxf(m, tmax[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = nan_maxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = nan_maxf(nan_maxf(red[0], red[1]), nan_maxf(red[2], red[3]));
  int ex = 0;
  if (m > 0.0f && m < INFINITY) {
    int e2;
    frexpf(m, &e2);  // m = f 2^e2, f in [0.5, 1)
    ex = e2 - 14;    // m 2^-ex in [2^13, 2^14)
  }
  if (blockIdx.x == 0 && tid == 0) gexp[0] = ex;
  const int64_t base = (int64_t)blockIdx.x * kGfSplitChunk;
#pragma unroll
  for (int run = 0; run < kGfSplitChunk / (256 * 8); ++run) {
    const int64_t j0 = base + (int64_t)(run * 256 + tid) * 8;
    if (j0 >= KK) break;
    const int64_t row = j0 / K, col0 = j0 - (j0 / K) * K;
    const int64_t ra = row / kLossBN, cb = col0 / kLossBN;
    if (cb < ra) continue;
    const float4 g0 = *(const float4*)(G + j0), g1 = *(const float4*)(G + j0 + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    // inside a diagonal block, the same at half size: its upper-right half block doubled,
    // its lower-left half zero (so the product's waves holding a tile's upper 128
    // channels start at the half block's diagonal)
    const int64_t hr = (row % kLossBN) / (kLossBN / 2), hc = (col0 % kLossBN) / (kLossBN / 2);
    const float f = (cb > ra || hc > hr) ? 2.0f : (hc < hr ? 0.0f : 1.0f);  // exact
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      uint16_t lo = f2h(ldexpf(f * g[i], -ex)), hi = f2h(ldexpf(f * g[i + 1], -ex));
      if (col0 + i == row) {
        gdiag[row] = ldexpf(g[i], -ex);
        lo = 0;
      }
      if (col0 + i + 1 == row) {
        gdiag[row] = ldexpf(g[i + 1], -ex);
        hi = 0;
      }
      h[i >> 1] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    *(uint4*)(Gh + j0) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

}  // namespace

GramPlan gram_plan(int64_t N, int64_t K) {
  GramPlan g;
  g.ld = (N + 7) / 8 * 8;
  g.splits = (N + kGramSplitTokens - 1) / kGramSplitTokens;
  const int64_t T = loss_tiles_m(K);
  g.pairs = T * (T + 1) / 2;
  g.tmax = g.splits > 1 ? 4 * g.pairs : g.pairs;
  return g;
}

hipError_t launch_gram_full(const uint16_t* X, int N, int K, uint16_t* Xt, float* part,
                            float* G, float* tmax, uint16_t* Gh, float* gdiag, int32_t* gexp,
                            hipStream_t stream) {
  if (K <= 0) return hipSuccess;
  if (K % 8 != 0 || N <= 0) return hipErrorInvalidValue;
  const GramPlan g = gram_plan(N, K);
  hipLaunchKernelGGL(k_transpose_x, dim3((unsigned)((g.ld + kTrTile - 1) / kTrTile),
                                         (unsigned)((K + kTrTile - 1) / kTrTile)),
                     dim3(256), 0, stream, X, N, K, (int)g.ld, Xt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_gram_build(Xt, N, (int)g.ld, K, kGramSplitTokens, (int)g.splits, g.splits > 1 ? part : G,
                        tmax, stream);
  if (e != hipSuccess) return e;
  if (g.splits > 1) {
    const int T = (int)loss_tiles_m(K);
    hipLaunchKernelGGL(k_gram_combine, dim3((unsigned)(4 * g.pairs)), dim3(256), 0, stream, part,
                       (int)g.splits, (int)g.pairs, T, K, G, tmax);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t KK = (int64_t)K * K;
  const int64_t blocks = (KK + kGfSplitChunk - 1) / kGfSplitChunk;
  hipLaunchKernelGGL(k_gram_full_split, dim3((unsigned)blocks), dim3(256), 0, stream, G, K, KK,
                     tmax, (int)g.tmax, Gh, gdiag, gexp);
  return hipGetLastError();
}

}  // namespace awq
