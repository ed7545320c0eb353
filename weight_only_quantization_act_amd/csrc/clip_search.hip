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
//                  4 x 4 (2 x 2) register tile per thread.
//   k_gram_sum     adds the splits in order (over split 0) and takes per-chunk maxima;
//   k_gram_split   scales the group's matrix by a power of two into [2^13, 2^14) and
//                  splits it into fp16 hi + lo (G ~ hi + lo to about 2^-22 relative), with
//                  the exponent kept per group.
//   k_clip_mfma    the quadratic forms on the matrix cores.  A lane pair (l, l ^ 32) owns one
//                  (row, ratio) pair: it quantises the row's group with its ratio in fp32
//                  exactly as the pack does, forms d = (v - Q(v)) / s, scales d by a power
//                  of two into [2^9, 2^10) and splits it into fp16 hi + lo.  Then
//                  U^T = G D^T comes from v_mfma_f32_32x32x16_f16 in three passes
//                  (G_hi D_hi + G_hi D_lo + G_lo D_hi; every product is exact in fp32),
//                  G's 32-row tiles as the A operand (from LDS) and 32 pairs as the B
//                  operand.  The k-slots of each 16-channel step are permuted so that lane
//                  half h supplies the channels whose bit 2 is h -- exactly the rows of U^T
//                  it receives in C -- so e = sum_c U^T[c] d[c] is a lane-local sum plus one
//                  exchange with the partner lane.  The power-of-two scales are undone
//                  exactly; the first smallest error per row is picked through LDS.
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

constexpr int kGramChunk = 1024;  // Gram entries per block of the two passes below

__device__ __forceinline__ double nan_max64(double m, double a) {
  return (a > m || a != a) ? a : m;
}

// Pass 1, block (group j, chunk c): G = sum of the split partials in order, written over
// split 0, and the chunk's largest magnitude (NaN if any entry is NaN).
__global__ __launch_bounds__(256) void k_gram_sum(double* __restrict__ partials, int g,
                                                  int ngroups, int splits,
                                                  double* __restrict__ cmax) {
  __shared__ double mx[256];
  const int j = blockIdx.x, c = blockIdx.y, nc = gridDim.y;
  const int tid = threadIdx.x;
  const size_t gg = (size_t)g * g;
  const size_t base = (size_t)j * gg + (size_t)c * kGramChunk;
  const size_t stride = (size_t)ngroups * gg;  // one split's partials
  const int n = (int)min((size_t)kGramChunk, gg - (size_t)c * kGramChunk);
  double m = 0.0;
  for (int i = tid; i < n; i += 256) {
    double v = partials[base + i];
    for (int sp = 1; sp < splits; ++sp) v += partials[sp * stride + base + i];
    partials[base + i] = v;
    m = nan_max64(m, fabs(v));
  }
  mx[tid] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) mx[tid] = nan_max64(mx[tid], mx[tid + o]);
    __syncthreads();
  }
  if (tid == 0) cmax[(size_t)j * nc + c] = mx[0];
}

// Pass 2, block (group j, chunk c): the group's largest magnitude from its chunks, the
// power of two 2^-ex that brings it into [2^13, 2^14), and the fp16 split of G 2^-ex.  A
// non-finite group keeps ex = 0, and its NaN / inf reaches the errors.
__global__ __launch_bounds__(256) void k_gram_split(const double* __restrict__ G64, int g,
                                                    const double* __restrict__ cmax,
                                                    uint16_t* __restrict__ Ghi,
                                                    uint16_t* __restrict__ Glo,
                                                    int32_t* __restrict__ gexp) {
  const int j = blockIdx.x, c = blockIdx.y, nc = gridDim.y;
  const int tid = threadIdx.x;
  double top = 0.0;
  for (int q = 0; q < nc; ++q) top = nan_max64(top, cmax[(size_t)j * nc + q]);
  int ex = 0;
  if (top > 0.0 && top < INFINITY) {
    int e2;
    frexp(top, &e2);  // top = f 2^e2, f in [0.5, 1)
    ex = e2 - 14;     // top 2^-ex in [2^13, 2^14)
  }
  if (c == 0 && tid == 0) gexp[j] = ex;
  const size_t gg = (size_t)g * g;
  const size_t base = (size_t)j * gg + (size_t)c * kGramChunk;
  const int n = (int)min((size_t)kGramChunk, gg - (size_t)c * kGramChunk);
  for (int i = tid; i < n; i += 256) {
    const float vs = (float)ldexp(G64[base + i], -ex);
    const uint16_t hi = f2h(vs);
    Ghi[base + i] = hi;
    Glo[base + i] = f2h(vs - h2f(hi));
  }
}

constexpr int kClipThreads = 256;
constexpr int kClipWaves = kClipThreads / 64;
constexpr int kClipPairs = kClipWaves * 32;  // (row, ratio) pairs per pass of a block

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Block: group j, rows [m_begin, m_end) in passes of kClipPairs / n_ratio rows.  Lane l of
// wave w: pair 32 w + (l mod 32) of the pass, half h = l div 32, channels 8 b + 4 h + i of the
// group (b < GS / 8, i < 4).  MFMA k-slot (h, e) of step s is channel 16 s + 4 h + e for
// e < 4 and 16 s + 8 + 4 h + (e - 4) otherwise, in both operands.
template <int GS>
__global__ __launch_bounds__(kClipThreads) void k_clip_mfma(
    const uint16_t* __restrict__ W, const float* __restrict__ s_in,
    const uint16_t* __restrict__ Ghi, const uint16_t* __restrict__ Glo,
    const int32_t* __restrict__ gexp, int M, int K, int w_bit, int zero_point,
    ClipList ratios, int n_ratio, int rows_per_block, float* __restrict__ clip_out,
    int32_t* __restrict__ best_out, float* __restrict__ errors) {
  constexpr int GP = GS + 4;  // padded LDS row (fp16): 8-byte fragment reads hit 32 banks pairs
  constexpr int KS = GS / 16;
  constexpr int RT = GS / 32;
  constexpr int NB = GS / 8;
  __shared__ __attribute__((aligned(16))) uint16_t gh[GS * GP];
  __shared__ __attribute__((aligned(16))) uint16_t gl[GS * GP];
  __shared__ float ss[GS], rs[GS];
  __shared__ float esh[kClipPairs];
  const int j = blockIdx.x;
  const int G = K / GS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, pl = lane & 31;
  const size_t gbase = (size_t)j * GS * GS;
  for (int i = tid; i < GS * GS / 8; i += kClipThreads) {
    const int r = i / (GS / 8), c8 = (i - r * (GS / 8)) * 8;
    const u32x4 a = *(const u32x4*)(Ghi + gbase + (size_t)r * GS + c8);
    const u32x4 b = *(const u32x4*)(Glo + gbase + (size_t)r * GS + c8);
    *(uint2*)(gh + r * GP + c8) = make_uint2(a[0], a[1]);
    *(uint2*)(gh + r * GP + c8 + 4) = make_uint2(a[2], a[3]);
    *(uint2*)(gl + r * GP + c8) = make_uint2(b[0], b[1]);
    *(uint2*)(gl + r * GP + c8 + 4) = make_uint2(b[2], b[3]);
  }
  __shared__ float rs_max_sh;
  for (int i = tid; i < GS; i += kClipThreads) {
    const float sv = s_in[j * GS + i];
    ss[i] = sv;
    rs[i] = 1.0f / sv;
  }
  __syncthreads();
  if (tid == 0) {
    float mx = 0.0f;
    for (int i = 0; i < GS; ++i) mx = fmaxf(mx, fabsf(rs[i]));
    rs_max_sh = mx;
  }
  __syncthreads();
  const float rs_max = rs_max_sh;
  const int ex = gexp[j];
  const int rows_per_pass = kClipPairs / n_ratio;
  const int pair = wave * 32 + pl;
  const int r_local = pair / n_ratio;
  const int k = pair - r_local * n_ratio;
  const float rho = ratios.v[k];
  const bool zp = zero_point != 0;
  const int m_begin = blockIdx.y * rows_per_block;
  const int m_end = min(M, m_begin + rows_per_block);

  for (int p0 = m_begin; p0 < m_end; p0 += rows_per_pass) {
    const int m = p0 + r_local;
    const bool live = r_local < rows_per_pass && m < m_end;
    // ---- the pair's weight error on the lane's channels ----------------------------------
    uint2 raw[NB];
    const uint16_t* wr = W + (size_t)(live ? m : 0) * K + (size_t)j * GS + 4 * h;
#pragma unroll
    for (int b = 0; b < NB; ++b) raw[b] = live ? *(const uint2*)(wr + 8 * b) : make_uint2(0u, 0u);
    // scaled weights v = w s (one rounding) of block b; s read 4 at a time from LDS
    auto vblock = [&](int b, float (&v)[4]) {
      const float4 sv = *(const float4*)&ss[8 * b + 4 * h];
      v[0] = h2f((uint16_t)(raw[b].x & 0xffffu)) * sv.x;
      v[1] = h2f((uint16_t)(raw[b].x >> 16)) * sv.y;
      v[2] = h2f((uint16_t)(raw[b].y & 0xffffu)) * sv.z;
      v[3] = h2f((uint16_t)(raw[b].y >> 16)) * sv.w;
    };
    // the group's step and zero with the range shrunk by rho, as in the pack
    float hi = -INFINITY, lo = INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v[4];
      vblock(b, v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi = fmaxf(hi, v[i]);
        lo = fminf(lo, v[i]);
      }
      if ((b & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound the hoisted LDS reads
    }
    hi = fmaxf(hi, __shfl_xor(hi, 32));
    lo = fminf(lo, __shfl_xor(lo, 32));
    const float vmax = fmaxf(fabsf(hi), fabsf(lo));
    float st, z, lo_code, hi_code;
    if (zp) {
      const float top = (float)((1 << w_bit) - 1);
      const float hr = fmaxf(hi, 0.0f) * rho, lr = fminf(lo, 0.0f) * rho;
      st = (hr - lr) / top;
      if (st == 0.0f) st = 1.0f;
      z = fminf(fmaxf(rintf(-lr / st), 0.0f), top);
      lo_code = 0.0f;
      hi_code = top;
    } else {
      const float qmax = (float)((1 << (w_bit - 1)) - 1);
      st = vmax * rho / qmax;
      if (st == 0.0f) st = 1.0f;
      z = (float)(1 << (w_bit - 1));
      lo_code = z - qmax;
      hi_code = z + qmax;
    }
    // |d| = |v - Q(v)| / s <= 2 max|v| max(1/s) = bound: scale by 2^kd so that the bound is
    // below 2^14 (no fp16 overflow; values far below it only lose precision in terms that
    // contribute little to e), then split d 2^kd into fp16 hi + lo (the B operand).
    const float bound = 2.0f * vmax * rs_max;
    int kd = 0;
    if (bound > 0.0f && bound < INFINITY) {
      int e2;
      frexpf(bound, &e2);  // bound = f 2^e2, f in [0.5, 1)
      kd = 14 - e2;
    }
    // k-step sk, dword q = channels of block b = 2 sk + (q >> 1), i = 2 (q & 1) .. + 1
    uint32_t bhi[KS][4], blo[KS][4];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v[4], dd[4];
      vblock(b, v);
      const float4 rv = *(const float4*)&rs[8 * b + 4 * h];
      const float r4[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float code = fminf(fmaxf(rintf(v[i] / st) + z, lo_code), hi_code);
        dd[i] = ldexpf((v[i] - (code - z) * st) * r4[i], kd);
      }
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const uint16_t h0 = f2h(dd[i]), h1 = f2h(dd[i + 1]);
        const uint16_t l0 = f2h(dd[i] - h2f(h0)), l1 = f2h(dd[i + 1] - h2f(h1));
        bhi[b >> 1][(b & 1) * 2 + (i >> 1)] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        blo[b >> 1][(b & 1) * 2 + (i >> 1)] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
      __builtin_amdgcn_sched_barrier(0);  // one block at a time
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- U^T = G D^T per 32-row tile of G, and e = sum_c U^T[c] d[c] ---------------------
    float e_lane = 0.0f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      floatx16 c = {};
      const uint16_t* rh = gh + (32 * rt + pl) * GP + 4 * h;
      const uint16_t* rl = gl + (32 * rt + pl) * GP + 4 * h;
#pragma unroll
      for (int sk = 0; sk < KS; ++sk) {
        const uint2 h0 = *(const uint2*)(rh + 16 * sk), h1 = *(const uint2*)(rh + 16 * sk + 8);
        const uint2 l0 = *(const uint2*)(rl + 16 * sk), l1 = *(const uint2*)(rl + 16 * sk + 8);
        const u32x4 hv = {h0.x, h0.y, h1.x, h1.y}, lv = {l0.x, l0.y, l1.x, l1.y};
        const half8 ahi = __builtin_bit_cast(half8, hv), alo = __builtin_bit_cast(half8, lv);
        const u32x4 bh = {bhi[sk][0], bhi[sk][1], bhi[sk][2], bhi[sk][3]};
        const u32x4 bl = {blo[sk][0], blo[sk][1], blo[sk][2], blo[sk][3]};
        const half8 bhv = __builtin_bit_cast(half8, bh), blv = __builtin_bit_cast(half8, bl);
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, bhv, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi, blv, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo, bhv, c, 0, 0, 0);
      }
      // C element i: row (channel) 32 rt + 8 (i div 4) + 4 h + (i mod 4) = channel 8 b + 4 h + i'
      // of this lane with b = 4 rt + i div 4, i' = i mod 4
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int b = 4 * rt + (i >> 2), ii = i & 3;
        const uint32_t ph = bhi[b >> 1][(b & 1) * 2 + (ii >> 1)];
        const uint32_t pq = blo[b >> 1][(b & 1) * 2 + (ii >> 1)];
        const int sh = (ii & 1) * 16;
        const float dv = h2f((uint16_t)(ph >> sh)) + h2f((uint16_t)(pq >> sh));
        e_lane = fmaf(c[i], dv, e_lane);
      }
      // one row tile at a time: keeps a single accumulator tile and its fragments live
      __builtin_amdgcn_sched_barrier(0);
    }
    e_lane += __shfl_xor(e_lane, 32);
    const float e = ldexpf(e_lane, ex - 2 * kd);
    if (live && h == 0) {
      esh[pair] = e;
      if (errors) errors[((size_t)k * M + m) * G + j] = e;
    }
    __syncthreads();
    if (live && h == 0 && k == 0) {
      int best = -1;
      float be = 0.0f;
      for (int q = 0; q < n_ratio; ++q) {
        const float v = esh[r_local * n_ratio + q];
        if (v == v && fabsf(v) != INFINITY && (best < 0 || v < be)) {
          best = q;
          be = v;
        }
      }
      clip_out[(size_t)m * G + j] = best >= 0 ? ratios.v[best] : 1.0f;
      if (best_out) best_out[(size_t)m * G + j] = best;
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

int gram_chunks(int group_size) {
  return (group_size * group_size + kGramChunk - 1) / kGramChunk;
}

hipError_t launch_group_gram(const uint16_t* X, int N, int K, int group_size, int splits,
                             double* partials, double* cmax, uint16_t* Ghi, uint16_t* Glo,
                             int32_t* gexp, hipStream_t stream) {
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
  const int nc = gram_chunks(group_size);
  dim3 g2(K / group_size, nc);
  hipLaunchKernelGGL(k_gram_sum, g2, dim3(256), 0, stream, partials, group_size,
                     K / group_size, splits, cmax);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gram_split, g2, dim3(256), 0, stream, partials, group_size, cmax, Ghi,
                     Glo, gexp);
  return hipGetLastError();
}

hipError_t launch_clip_search(const uint16_t* W, const float* s, const uint16_t* Ghi,
                              const uint16_t* Glo, const int32_t* gexp, int M, int K, int w_bit,
                              int group_size, int zero_point, const ClipList& ratios,
                              int n_ratio, float* clip_out, int32_t* best_out, float* errors,
                              hipStream_t stream) {
  if (M <= 0 || K <= 0) return hipSuccess;
  if (n_ratio < 1 || n_ratio > kClipPairs / 2) return hipErrorInvalidValue;
  const int rows_per_pass = kClipPairs / n_ratio;
  // about 96 rows per block (the Gram matrix is staged once per block), fewer when the
  // layer is small, so that the grid still fills the chip
  const int ngroups = K / group_size;
  int passes = (96 + rows_per_pass - 1) / rows_per_pass;
  while (passes > 1 && (int64_t)ngroups * ((M + passes * rows_per_pass - 1) /
                                           (passes * rows_per_pass)) < 1024)
    --passes;
  const int rows = passes * rows_per_pass;
  dim3 grid(ngroups, (M + rows - 1) / rows);
#define AWQ_CLIP(GS)                                                                        \
  hipLaunchKernelGGL(k_clip_mfma<GS>, grid, dim3(kClipThreads), 0, stream, W, s, Ghi, Glo,   \
                     gexp, M, K, w_bit, zero_point, ratios, n_ratio, rows, clip_out,          \
                     best_out, errors)
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
