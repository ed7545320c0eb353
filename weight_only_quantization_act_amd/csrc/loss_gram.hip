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
//                      G's upper block triangle in 256 x 256 tiles on the matrix cores,
//                      one block per (token split, tile): fp16 products (exact in fp32)
//                      summed in fp32 over a split of at most kGramSplitTokens tokens (at
//                      most 512 accumulator additions of 32x32x16 products, so within
//                      2^-15 of the sum of |products|), written as that split's partial
//                      tile with its largest |entry|.  The split length is planned so
//                      that the blocks fill the compute units (gram_split_tokens).
//   k_gram_combine_split
//                      each entry of G the fp64 sum of its split partials in split order,
//                      rounded to fp32; one power of two 2^-ex for the whole matrix (a
//                      bound on its largest magnitude into [2^13, 2^14)) and the operand
//                      of the per-grid-point product:
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

#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "awq_internal.h"
#include "quantizer.h"

namespace awq {

namespace {

constexpr int kTrTile = 64;          // tokens and channels of a transpose tile
constexpr int kSplitRows = 64;       // tile rows per block of the split pass

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

// The tile pair p of G's upper block triangle in row-major order: (tm, tn), tm <= tn.
__device__ __forceinline__ void pair_tiles(int p, int T, int& tm, int& tn) {
  int t = 0, left = p;
  while (left >= T - t) {
    left -= T - t;
    ++t;
  }
  tm = t;
  tn = t + left;
}

// Block (quarter q of pair p): rows [64 q, 64 q + 64) of tile pair p = (tm, tn); a thread
// takes eight consecutive columns of one row at a time (32 threads a row, 8 rows a pass).
// Each entry of G is the fp64 sum of the split partials [split][pair][256][256] in split
// order, rounded to fp32 (one split: the partial itself).  One power of two 2^-ex serves
// the whole matrix: every block derives it from the tile maxima of the partials (the sum
// over splits of a tile's largest |partial| bounds its largest |G|; NaN if any entry is
// NaN, and then ex = 0 and the NaN reaches the losses).  Then G' 2^-ex goes to Gh (fp16,
// row-major [K][K]) and diag(G) 2^-ex to gdiag (fp32); block 0 publishes ex.  Blocks
// below the diagonal are not formed: the product never reads them.
__global__ __launch_bounds__(256) void k_gram_combine_split(
    const float* __restrict__ part, int splits, int npairs, int T, int K,
    const float* __restrict__ tmax, uint16_t* __restrict__ Gh, float* __restrict__ gdiag,
    int32_t* __restrict__ gexp) {
  __shared__ double red[4];
  const int tid = threadIdx.x;
  double m = 0.0;
  for (int p = tid; p < npairs; p += 256) {
    double ub = 0.0;
    for (int sp = 0; sp < splits; ++sp) ub += (double)tmax[(size_t)sp * npairs + p];
    m = (ub > m || ub != ub) ? ub : m;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double v = __shfl_xor(m, o);
    m = (v > m || v != v) ? v : m;
  }
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) m = (red[w] > m || red[w] != red[w]) ? red[w] : m;
  int ex = 0;
  if (m > 0.0 && m < INFINITY) {
    int e2;
    frexp(m, &e2);  // m = f 2^e2, f in [0.5, 1)
    ex = e2 - 14;   // m 2^-ex in [2^13, 2^14)
  }
  if (blockIdx.x == 0 && tid == 0) gexp[0] = ex;

  const int p = blockIdx.x >> 2, qr = blockIdx.x & 3;
  int tm, tn;
  pair_tiles(p, T, tm, tn);
  const int cl = (tid & 31) * 8;
  const int col0 = tn * kLossBN + cl;
  if (col0 >= K) return;  // K is a multiple of 8, so a run is wholly in or out
  const size_t split_stride = (size_t)npairs * kLossBM * kLossBN;
  const float* src = part + (size_t)p * kLossBM * kLossBN + cl;
  for (int it = 0; it < kSplitRows / 8; ++it) {
    const int rl = qr * kSplitRows + it * 8 + (tid >> 5);
    const int row = tm * kLossBM + rl;
    if (row >= K) break;
    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    for (int sp = 0; sp < splits; ++sp) {
      const float* q = src + sp * split_stride + (size_t)rl * kLossBN;
      const float4 a = *(const float4*)q, b = *(const float4*)(q + 4);
      acc[0] += (double)a.x; acc[1] += (double)a.y; acc[2] += (double)a.z; acc[3] += (double)a.w;
      acc[4] += (double)b.x; acc[5] += (double)b.y; acc[6] += (double)b.z; acc[7] += (double)b.w;
    }
    // G' = G with the blocks above the diagonal doubled; inside a diagonal block the same
    // at half size: its upper-right half block doubled, its lower-left half zero (so the
    // product's waves holding a tile's upper 128 channels start at the half block's
    // diagonal); the diagonal itself zero, kept in fp32 apart
    const int hr = rl / (kLossBN / 2), hc = cl / (kLossBN / 2);
    const float f = (tn > tm || hc > hr) ? 2.0f : (hc < hr ? 0.0f : 1.0f);  // exact
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float g0 = (float)acc[i], g1 = (float)acc[i + 1];
      uint16_t lo = f2h(ldexpf(f * g0, -ex)), hi = f2h(ldexpf(f * g1, -ex));
      if (col0 + i == row) {
        gdiag[row] = ldexpf(g0, -ex);
        lo = 0;
      }
      if (col0 + i + 1 == row) {
        gdiag[row] = ldexpf(g1, -ex);
        hi = 0;
      }
      h[i >> 1] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    *(uint4*)(Gh + (size_t)row * K + col0) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

}  // namespace

// Tokens per split.  A block of the build runs one tile over one split; the blocks go out
// split by split, round-robin over the 8 XCDs, each XCD filling its 32 compute units as
// they free up.  Candidates: s splits for s from the fewest that keep every split within
// kGramSplitTokens to 6 more, the last split a whole, 2/3, 1/2 or 1/3 share of the others
// (so that the short blocks fill the units the long ones leave idle).  Each is priced by
// list-scheduling the busiest XCD's blocks in that order (its longest unit, in block-time
// per token) plus the partial tiles written and read back (about 4.3 token-times per
// 256 x 256 fp32 tile: 512 KiB of traffic at about 5 TB/s against about 0.024 us a token
// for a block).  The cheapest wins; ties keep fewer splits.  The host computes this once
// per (tokens, tile pairs) and keeps the last few answers.
static int64_t gram_split_tokens_uncached(int64_t N, int64_t pairs) {
  constexpr int kUnits = 32;
  constexpr double kTileCost = 4.3;
  const int64_t cap = kGramSplitTokens;
  const int64_t s_min = (N + cap - 1) / cap;
  const int64_t per_xcd = (pairs + 7) / 8;
  int64_t best_k = N < cap ? ((N + 63) / 64) * 64 : cap;
  double best = -1.0;
  for (int64_t sp = s_min; sp <= s_min + 6; ++sp) {
    for (const int sixths : {6, 4, 3, 2}) {
      if (sp == 1 && sixths != 6) continue;
      int64_t k = (6 * N + 6 * (sp - 1) + sixths - 1) / (6 * (sp - 1) + sixths);
      k = ((k + 63) / 64) * 64;
      if (k > cap) k = cap;
      const int64_t splits = (N + k - 1) / k;
      const int64_t last = N - (splits - 1) * k;
      // the units' busy times as a min-heap: each block goes to the first unit free
      std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> busy;
      for (int v = 0; v < kUnits; ++v) busy.push(0);
      int64_t span = 0;
      for (int64_t jj = 0; jj < splits; ++jj) {
        const int64_t len = jj + 1 == splits ? last : k;
        for (int64_t b = 0; b < per_xcd; ++b) {
          const int64_t t = busy.top() + len;
          busy.pop();
          busy.push(t);
          span = t > span ? t : span;
        }
      }
      const double cost = (double)span + kTileCost * (double)(splits * pairs);
      if (best < 0.0 || cost < best) {
        best = cost;
        best_k = k;
      }
    }
  }
  return best_k;
}

int64_t gram_split_tokens(int64_t N, int64_t pairs) {
  struct Entry {
    int64_t n, pairs, k;
  };
  static std::mutex mu;
  static Entry cache[8] = {};
  static int next = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : cache)
      if (e.k > 0 && e.n == N && e.pairs == pairs) return e.k;
  }
  const int64_t k = gram_split_tokens_uncached(N, pairs);
  std::lock_guard<std::mutex> lock(mu);
  cache[next] = Entry{N, pairs, k};
  next = (next + 1) % 8;
  return k;
}

GramPlan gram_plan(int64_t N, int64_t K) {
  GramPlan g;
  g.ld = (N + 7) / 8 * 8;
  const int64_t T = loss_tiles_m(K);
  g.pairs = T * (T + 1) / 2;
  g.kchunk = N > 0 ? gram_split_tokens(N, g.pairs) : 64;
  g.splits = N > 0 ? (N + g.kchunk - 1) / g.kchunk : 1;
  g.tmax = g.splits * g.pairs;
  return g;
}

hipError_t launch_gram_full(const uint16_t* X, int N, int K, uint16_t* Xt, float* part,
                            float* tmax, uint16_t* Gh, float* gdiag, int32_t* gexp,
                            hipStream_t stream) {
  if (K <= 0) return hipSuccess;
  if (K % 8 != 0 || N <= 0) return hipErrorInvalidValue;
  const GramPlan g = gram_plan(N, K);
  hipLaunchKernelGGL(k_transpose_x, dim3((unsigned)((g.ld + kTrTile - 1) / kTrTile),
                                         (unsigned)((K + kTrTile - 1) / kTrTile)),
                     dim3(256), 0, stream, X, N, K, (int)g.ld, Xt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_gram_build(Xt, N, (int)g.ld, K, (int)g.kchunk, (int)g.splits, part, tmax, stream);
  if (e != hipSuccess) return e;
  const int T = (int)loss_tiles_m(K);
  hipLaunchKernelGGL(k_gram_combine_split, dim3((unsigned)(4 * g.pairs)), dim3(256), 0, stream,
                     part, (int)g.splits, (int)g.pairs, T, K, tmax, Gh, gdiag, gexp);
  return hipGetLastError();
}

}  // namespace awq
