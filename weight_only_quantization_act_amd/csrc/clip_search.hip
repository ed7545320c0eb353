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
//   k_gram_mfma    the Gram sums on the matrix cores: fp16 products (exact in fp32) summed
//                  in fp32 over at most 256 tokens, added in fp64, one 128-channel span and
//                  token split per block (the stage transposed into LDS on the way in);
//   k_gram_sum     adds the split partials in fp64 in split order and takes per-chunk
//                  maxima;
//   k_gram_split   scales the group's matrix by a power of two into [2^13, 2^14) and
//                  splits it into fp16 hi + lo (G ~ hi + lo to about 2^-22 relative), with
//                  the exponent kept per group.
//   k_clip_mfma    the quadratic forms on the matrix cores.  Four lanes own one (row, ratio)
//                  pair: they quantise the row's group with its ratio in fp32 exactly as
//                  the pack does, form d = (v - Q(v)) / s, scale d by a power of two below
//                  2^14 and split it into fp16 hi + lo.  Then U^T = G' D^T comes from
//                  v_mfma_f32_16x16x32_f16 in three passes (G_hi D_hi + G_hi D_lo +
//                  G_lo D_hi; every product is exact in fp32), G' (G with its upper 16 x 16
//                  blocks doubled and lower ones dropped, so only 20 of 32 tiles are needed)
//                  as the A operand from LDS and 16 pairs as the B operand, two such slices
//                  per wave sharing each read of G'.  The k-slots of each 32-channel step
//                  are permuted so that each lane supplies the channels whose rows of U^T it
//                  receives in C, so e = sum_c U^T[c] d[c] is a lane-local sum plus two
//                  exchanges.  The power-of-two scales are undone exactly; the first smallest
//                  error per row is kept through an LDS atomic minimum.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>

#include "awq_internal.h"
#include "quantizer.h"

namespace awq {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kGramThreads = 512;
constexpr int kGramSpan = 128;   // channels of one block (128 / g groups)
constexpr int kGramStage = 64;   // tokens per LDS stage (two 32-token k-steps)
constexpr int kGramFlush = 256;  // tokens summed in fp32 before adding into fp64
constexpr int kGramXtp = 68;     // LDS row of the transposed tile (fp16, 8-byte aligned)
constexpr int kGramTargetBlocks = 512;

// partials[sp][j][a][b] = sum over split sp's tokens of X[t][j g + a] X[t][j g + b], the
// products of fp16 values exact in fp32, summed on the matrix cores (v_mfma_f32_16x16x32_f16)
// in fp32 over at most 256 tokens (error at most 2^-16 of the sum of |products|), those
// sums added in fp64 and the split's total rounded to fp32.
//
// Block: channels [c0, c0 + 128) of the layer and split sp.  A stage of 64 tokens is stored
// transposed in LDS, xt[channel][token]: lane l of wave w loads the channel pair
// (2 l, 2 l + 1) of tokens 8 w .. 8 w + 7 (coalesced 256-byte token rows) and interleaves
// the halves with v_perm.  The MFMA fragment of channel block b (16 channels) and k-step ks
// is then lane (p, q)'s 16 bytes xt[16 b + p][32 ks + 8 q ..], the A operand of tile row b
// and the B operand of tile column b alike.  Wave w owns tile row w and the g / 16 tile
// columns of its group.
template <int GS>
__global__ __launch_bounds__(kGramThreads) void k_gram_mfma(const uint16_t* __restrict__ X,
                                                            int N, int K, int tokens_per_split,
                                                            float* __restrict__ partials) {
  constexpr int TC = GS / 16;  // tile columns of a group
  __shared__ __attribute__((aligned(16))) uint16_t xt[kGramSpan * kGramXtp];
  const int c0 = blockIdx.x * kGramSpan;
  const int sp = blockIdx.y;
  const int t_begin = sp * tokens_per_split;
  const int t_end = min(N, t_begin + tokens_per_split);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, pl = lane & 15;
  const int ngroups = K / GS;
  const int grp = (c0 + 16 * wave) / GS;  // the group of the wave's tile row
  const int tc0 = (grp * GS - c0) / 16;   // the group's first tile column (span blocks)
  const bool active = grp < ngroups;
  const bool pair_ok = c0 + 2 * lane < K;

  floatx4 acc[TC];
  double acc64[TC][4];
#pragma unroll
  for (int tc = 0; tc < TC; ++tc) {
    acc[tc] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc64[tc][e] = 0.0;
  }

  // the lane's 8 token values of its channel pair for a stage; the next stage's load is
  // in flight during this stage's matrix work
  uint32_t d[8];
  auto load_stage = [&](int t0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = t0 + 8 * wave + e;
      d[e] = (pair_ok && t < t_end) ? *(const uint32_t*)(X + (size_t)t * K + c0 + 2 * lane)
                                    : 0u;
    }
  };
  if (t_begin < t_end) load_stage(t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += kGramStage) {
    {
      uint2 lo0, lo1, hi0, hi1;  // channel 2 l (low halves) and 2 l + 1 (high halves)
      lo0.x = __builtin_amdgcn_perm(d[1], d[0], 0x05040100u);
      lo0.y = __builtin_amdgcn_perm(d[3], d[2], 0x05040100u);
      lo1.x = __builtin_amdgcn_perm(d[5], d[4], 0x05040100u);
      lo1.y = __builtin_amdgcn_perm(d[7], d[6], 0x05040100u);
      hi0.x = __builtin_amdgcn_perm(d[1], d[0], 0x07060302u);
      hi0.y = __builtin_amdgcn_perm(d[3], d[2], 0x07060302u);
      hi1.x = __builtin_amdgcn_perm(d[5], d[4], 0x07060302u);
      hi1.y = __builtin_amdgcn_perm(d[7], d[6], 0x07060302u);
      uint16_t* r0 = xt + (2 * lane) * kGramXtp + 8 * wave;
      *(uint2*)r0 = lo0;
      *(uint2*)(r0 + 4) = lo1;
      *(uint2*)(r0 + kGramXtp) = hi0;
      *(uint2*)(r0 + kGramXtp + 4) = hi1;
    }
    __syncthreads();
    if (t0 + kGramStage < t_end) load_stage(t0 + kGramStage);
    if (active) {
      auto frag = [&](int blk, int ks) {
        const uint16_t* src = xt + (16 * blk + pl) * kGramXtp + 32 * ks + 8 * q4;
        const uint2 u0 = *(const uint2*)src, u1 = *(const uint2*)(src + 4);
        const u32x4 v = {u0.x, u0.y, u1.x, u1.y};
        return __builtin_bit_cast(half8, v);
      };
#pragma unroll
      for (int ks = 0; ks < kGramStage / 32; ++ks) {
        const half8 fa = frag(wave, ks);
#pragma unroll
        for (int tc = 0; tc < TC; ++tc)
          acc[tc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, frag(tc0 + tc, ks), acc[tc], 0,
                                                           0, 0);
      }
    }
    __syncthreads();
    if ((t0 + kGramStage - t_begin) % kGramFlush == 0 || t0 + kGramStage >= t_end) {
#pragma unroll
      for (int tc = 0; tc < TC; ++tc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc64[tc][e] += (double)acc[tc][e];
        acc[tc] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  }
  if (!active) return;
  // C element e of tile (wave, tc0 + tc): G row 16 wave + 4 q + e, column
  // 16 (tc0 + tc) + (l mod 16), both relative to the span; minus the group's offset
  float* out = partials + ((size_t)sp * ngroups + grp) * (size_t)GS * GS;
  const int goff = grp * GS - c0;
#pragma unroll
  for (int tc = 0; tc < TC; ++tc)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int a = 16 * wave + 4 * q4 + e - goff;
      const int b = 16 * (tc0 + tc) + pl - goff;
      out[(size_t)a * GS + b] = (float)acc64[tc][e];
    }
}

constexpr int kGramChunk = 256;  // Gram entries per block of the two passes below (one a thread)

__device__ __forceinline__ double nan_max64(double m, double a) {
  return (a > m || a != a) ? a : m;
}

// Pass 1, block (group j, chunk c): G~ = S^-1 G S^-1, G the split partials added in fp64
// in split order and S = diag(s), and the chunk's largest magnitude (NaN if any entry is
// NaN).  With it the group error of the scaled weight error d~ = v - Q(v) = d s is
// d~^T G~ d~ = d^T G d.
__global__ __launch_bounds__(256) void k_gram_sum(const float* __restrict__ partials, int g,
                                                  int ngroups, int splits,
                                                  const float* __restrict__ s,
                                                  double* __restrict__ G64,
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
    // sixteen independent loads at a time, added in split order
    double v = 0.0;
    for (int sp0 = 0; sp0 < splits; sp0 += 16) {
      float p[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        p[u] = sp0 + u < splits ? partials[(size_t)(sp0 + u) * stride + base + i] : 0.0f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (sp0 + u < splits) v += (double)p[u];
    }
    const int e = c * kGramChunk + i;  // entry (a, b) of the group's matrix
    const int a = e / g, b = e - (e / g) * g;
    v = v / ((double)s[j * g + a] * (double)s[j * g + b]);  // (the fp32 product is exact)
    G64[base + i] = v;
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
  __shared__ double red[4];
  const int j = blockIdx.x, c = blockIdx.y, nc = gridDim.y;  // nc = g * g / 256 <= 64
  const int tid = threadIdx.x;
  double top = tid < nc ? cmax[(size_t)j * nc + tid] : 0.0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) top = nan_max64(top, __shfl_xor(top, o));
  if ((tid & 63) == 0) red[tid >> 6] = top;
  __syncthreads();
  top = nan_max64(nan_max64(red[0], red[1]), nan_max64(red[2], red[3]));
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
constexpr int kClipMaxRows = 160;  // rows of one block (its per-row LDS tables)
#ifndef AWQ_CLIP_SLICES
#define AWQ_CLIP_SLICES 2
#endif
constexpr int kClipSlices = AWQ_CLIP_SLICES;  // 16-pair slices sharing one read of G's tiles


// Order-preserving key of a finite error and its ratio index: the smallest key is the
// smallest error, and among equal errors the first ratio.
__device__ __forceinline__ unsigned long long clip_key(float e, int k) {
  const uint32_t u = __float_as_uint(e);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (uint32_t)k;
}

// Block: group j and rows [m_begin, m_begin + R).  Its R n_ratio (row, ratio) pairs, row
// major, are cut into slices of 16; wave w takes slices w, w + 4, ... with no block-wide
// synchronisation, and each row keeps its first smallest error through an LDS atomic
// minimum.  In a slice, lane l takes pair 16 slice + (l mod 16) and quarter q = l div 16,
// which owns the group's channels c with (c >> 2) & 3 == q, i.e. c = 16 b + 4 q + i
// (b < GS / 16, i < 4).  MFMA 16x16x32 f16 (A row l mod 16, k-slots 8 q + e; B column
// l mod 16, same k-slots; C column l mod 16, rows 4 q + e): k-slot (q, e) of 32-channel
// step s is channel 32 s + 16 (e div 4) + 4 q + (e mod 4) in both operands, and the C rows
// of G's 16-row tile rt are channels 16 rt + 4 q + e -- this lane's own channels, so the
// epilogue is local.
template <int GS, int NS>
__global__ __launch_bounds__(kClipThreads) void k_clip_mfma(
    const uint16_t* __restrict__ W, const float* __restrict__ s_in,
    const uint16_t* __restrict__ Ghi, const uint16_t* __restrict__ Glo,
    const int32_t* __restrict__ gexp, int M, int K, int w_bit, int zero_point,
    ClipList ratios, int n_ratio, int rows_per_block, float* __restrict__ clip_out,
    int32_t* __restrict__ best_out, float* __restrict__ errors) {
  constexpr int GP = GS + 4;  // padded LDS row (fp16) of G
  constexpr int KS = GS / 32;  // 32-channel k-steps
  constexpr int RT = GS / 16;  // 16-row tiles of G
  constexpr int NB = GS / 16;  // 16-channel blocks; a lane owns 4 channels of each
  __shared__ __attribute__((aligned(16))) uint16_t gh[GS * GP];
  __shared__ __attribute__((aligned(16))) uint16_t gl[GS * GP];
  __shared__ __attribute__((aligned(16))) float ss[GS];  // s, then s 2^kd
  __shared__ float rng_hi[kClipMaxRows], rng_lo[kClipMaxRows];  // range of v = w s per row
  __shared__ unsigned long long best_key[kClipMaxRows];
  __shared__ uint32_t vmax_bits, smax_bits;  // block maxima of max|v| (finite) and of |s|
  const int j = blockIdx.x;
  const int G = K / GS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, pl = lane & 15;
  const int m_begin = blockIdx.y * rows_per_block;
  const int R = min(M - m_begin, rows_per_block);
  const size_t gbase = (size_t)j * GS * GS;
  // G' in LDS: G's 16 x 16 blocks above the diagonal doubled (exact), those below zero, so
  // that d^T G d = sum over row tiles rt of d_rt^T (G' d)_rt and a row tile only needs the
  // k-steps from its own diagonal block on
  for (int i = tid; i < GS * GS / 8; i += kClipThreads) {
    const int r = i / (GS / 8), c8 = (i - r * (GS / 8)) * 8;
    u32x4 a = *(const u32x4*)(Ghi + gbase + (size_t)r * GS + c8);
    u32x4 b = *(const u32x4*)(Glo + gbase + (size_t)r * GS + c8);
    if (c8 / 16 < r / 16) {
      a = u32x4{0u, 0u, 0u, 0u};
      b = a;
    } else if (c8 / 16 > r / 16) {
      half8 ah = __builtin_bit_cast(half8, a), bh = __builtin_bit_cast(half8, b);
      ah = ah + ah;
      bh = bh + bh;
      a = __builtin_bit_cast(u32x4, ah);
      b = __builtin_bit_cast(u32x4, bh);
    }
    *(uint2*)(gh + r * GP + c8) = make_uint2(a[0], a[1]);
    *(uint2*)(gh + r * GP + c8 + 4) = make_uint2(a[2], a[3]);
    *(uint2*)(gl + r * GP + c8) = make_uint2(b[0], b[1]);
    *(uint2*)(gl + r * GP + c8 + 4) = make_uint2(b[2], b[3]);
  }
  for (int i = tid; i < GS; i += kClipThreads) ss[i] = s_in[j * GS + i];
  if (tid == 0) {
    vmax_bits = 0u;
    smax_bits = 0u;
  }
  __syncthreads();
  // range of the scaled weights v = w s of every row of the block (shared by its ratios),
  // one thread per row
  for (int r = tid; r < R; r += kClipThreads) {
    const uint16_t* w1 = W + (size_t)(m_begin + r) * K + (size_t)j * GS;
    float hi = -INFINITY, lo = INFINITY;
#pragma unroll 4
    for (int c8 = 0; c8 < GS; c8 += 8) {
      const u32x4 raw = *(const u32x4*)(w1 + c8);
      const float4 s0 = *(const float4*)&ss[c8], s1 = *(const float4*)&ss[c8 + 4];
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = h2f((uint16_t)(raw[i >> 1] >> (16 * (i & 1)))) * sv[i];
        hi = fmaxf(hi, v);
        lo = fminf(lo, v);
      }
    }
    rng_hi[r] = hi;
    rng_lo[r] = lo;
    best_key[r] = ~0ull;
    const float vm = fmaxf(fabsf(hi), fabsf(lo));
    if (vm < INFINITY) atomicMax(&vmax_bits, __float_as_uint(vm));
  }
  for (int i = tid; i < GS; i += kClipThreads) {
    const float a = fabsf(ss[i]);
    if (a < INFINITY) atomicMax(&smax_bits, __float_as_uint(a));
  }
  __syncthreads();
  // One power of two 2^kd for the block: |v - Q(v)| <= |v| + |Q(v)| <= 2.07 max|v|, so with
  // 2 max|v| below 2^14 the scaled errors d~ 2^kd stay far inside fp16 (65504); kd is also
  // capped so that every s 2^kd stays finite.  Scaling s by 2^kd scales v, the step and the
  // errors exactly (the quotient v / step is unchanged).
  int kd = 0;
  {
    const float bound = 2.0f * __uint_as_float(vmax_bits);
    if (bound > 0.0f) {
      int e2, es;
      frexpf(bound, &e2);  // bound = f 2^e2, f in [0.5, 1)
      kd = 14 - e2;
      frexpf(__uint_as_float(smax_bits), &es);
      kd = min(kd, 127 - es);
    }
  }
  __syncthreads();  // every thread has read the maxima; ss is rescaled next
  for (int i = tid; i < GS; i += kClipThreads) ss[i] = ldexpf(ss[i], kd);
  __syncthreads();
  const int ex = gexp[j];
  const bool zp = zero_point != 0;
  const int P = R * n_ratio;
  const int slices = (P + 15) / 16;
  const int sgroups = (slices + NS - 1) / NS;  // a wave takes NS consecutive slices at once
  // the lane's raw weights, channels 16 b + 4 q + i of the row of each of its NS pairs (a
  // dead lane past the last pair reads the last pair's row)
  uint2 raw[NS][NB];
  auto load_raw = [&](int sg) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int rr = min(16 * (sg * NS + u) + pl, P - 1) / n_ratio;
      const uint16_t* wr = W + (size_t)(m_begin + rr) * K + (size_t)j * GS + 4 * q4;
#pragma unroll
      for (int b = 0; b < NB; ++b) raw[u][b] = *(const uint2*)(wr + 16 * b);
    }
  };
  if (wave < sgroups) load_raw(wave);
  // -1 held in a register, so that d - hi stays one mixed-precision fused multiply-add
  float neg_one;
  asm volatile("s_mov_b32 %0, -1.0" : "=s"(neg_one));

  for (int sg = wave; sg < sgroups; sg += kClipWaves) {
    // B operands of the NS pairs: block b's 4 channels as two dwords of fp16 pairs,
    // hi = d~ 2^kd rounded toward zero (two per instruction) and lo = the exact remainder
    // rounded toward zero, so that |hi + lo - d~ 2^kd| <= 2^-20 |d~ 2^kd| above the fp16
    // subnormal range
    uint32_t bhi[NS][NB][2], blo[NS][NB][2];
    int rv_[NS], kv[NS];
    bool livev[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int pair = 16 * (sg * NS + u) + pl;
      const bool live = pair < P;
      const int pc = live ? pair : P - 1;
      const int r = pc / n_ratio;
      const int k = pc - r * n_ratio;
      const float rho = ratios.v[k];
      const float hi = rng_hi[r], lo = rng_lo[r];
      const float vmax = fmaxf(fabsf(hi), fabsf(lo));
      // the group's step and zero with the range shrunk by rho, as in the pack; the code
      // relative to the zero, c - z, is clamped to [clo, chi]
      float st, clo, chi;
      if (zp) {
        const float top = (float)((1 << w_bit) - 1);
        const float hr = fmaxf(hi, 0.0f) * rho, lr = fminf(lo, 0.0f) * rho;
        st = (hr - lr) / top;
        if (st == 0.0f) st = 1.0f;
        const float z = fminf(fmaxf(rintf(-lr / st), 0.0f), top);
        clo = -z;
        chi = top - z;
      } else {
        const float qmax = (float)((1 << (w_bit - 1)) - 1);
        st = vmax * rho / qmax;
        if (st == 0.0f) st = 1.0f;
        clo = -qmax;
        chi = qmax;
      }
      st = ldexpf(st, kd);  // the step in the block's scaled units
      // rint(v / st) as rint(v * (1/st)), except for a lane with an element whose product
      // lies within 2^-17 of a half-integer (or is not finite): that lane redoes its
      // elements with the correctly rounded division.  The two agree for |v / st| <= 16, and
      // beyond that the clamp gives the same code either way (the argument of the pack's
      // quantiser).  Adding the integer zero after rounding keeps the pack's tie rule.
      const float inv = step_reciprocal(st);
      auto quant_block = [&](int b, bool exact) {
        const float4 sv = *(const float4*)&ss[16 * b + 4 * q4];
        const float s4[4] = {sv.x, sv.y, sv.z, sv.w};
        const uint32_t wp[2] = {raw[u][b].x, raw[u][b].y};
        float dd[4];
        bool near = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const _Float16 wh =
              __builtin_bit_cast(_Float16, (uint16_t)(wp[i >> 1] >> (16 * (i & 1))));
          // v = w s 2^kd (a zero's sign is immaterial)
          const float v = fmaf((float)wh, s4[i], 0.0f);
          const float t = v * inv;
          float q = rintf(t);
          const bool nr = !(fabsf(t - q) < 0.5f - kTieBand);
          if (exact) {
            if (nr) q = rintf(v / st);
          } else {
            near |= nr;
          }
          const float cz = __builtin_amdgcn_fmed3f(q, clo, chi);
          dd[i] = fmaf(-cz, st, v);  // d~ 2^kd = (v - Q(v)) 2^kd
        }
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const uint32_t ph =
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(dd[i], dd[i + 1]));
          const _Float16 h0 = __builtin_bit_cast(_Float16, (uint16_t)(ph & 0xffffu));
          const _Float16 h1 = __builtin_bit_cast(_Float16, (uint16_t)(ph >> 16));
          const float l0 = fmaf((float)h0, neg_one, dd[i]);
          const float l1 = fmaf((float)h1, neg_one, dd[i + 1]);
          bhi[u][b][i >> 1] = ph;
          blo[u][b][i >> 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(l0, l1));
        }
        return near;
      };
      bool need = false;
#pragma unroll
      for (int b = 0; b < NB; ++b) need |= quant_block(b, false);
      if (need && live) {
#pragma unroll
        for (int b = 0; b < NB; ++b) quant_block(b, true);
      }
      rv_[u] = r;
      kv[u] = k;
      livev[u] = live;
    }
    // the next slices' weights load during this group's matrix phase
    if (sg + kClipWaves < sgroups) load_raw(sg + kClipWaves);
    __builtin_amdgcn_sched_barrier(0);
    // ---- U^T = G' D^T per 16-row tile of G', and e = sum_c U^T[c] d[c] -------------------
    float e_lane[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) e_lane[u] = 0.0f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      floatx4 c[NS];
#pragma unroll
      for (int u = 0; u < NS; ++u) c[u] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      const uint16_t* rh = gh + (16 * rt + pl) * GP + 4 * q4;
      const uint16_t* rl = gl + (16 * rt + pl) * GP + 4 * q4;
#pragma unroll
      for (int sk = rt / 2; sk < KS; ++sk) {
        // k-slots e < 4: channel 32 sk + 4 q + e (block 2 sk); e >= 4: 32 sk + 16 + 4 q + e - 4
        const uint2 h0 = *(const uint2*)(rh + 32 * sk), h1 = *(const uint2*)(rh + 32 * sk + 16);
        const uint2 l0 = *(const uint2*)(rl + 32 * sk), l1 = *(const uint2*)(rl + 32 * sk + 16);
        const u32x4 hv = {h0.x, h0.y, h1.x, h1.y}, lv = {l0.x, l0.y, l1.x, l1.y};
        const half8 ahi = __builtin_bit_cast(half8, hv), alo = __builtin_bit_cast(half8, lv);
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          const u32x4 bh = {bhi[u][2 * sk][0], bhi[u][2 * sk][1], bhi[u][2 * sk + 1][0],
                            bhi[u][2 * sk + 1][1]};
          const u32x4 bl = {blo[u][2 * sk][0], blo[u][2 * sk][1], blo[u][2 * sk + 1][0],
                            blo[u][2 * sk + 1][1]};
          const half8 bhv = __builtin_bit_cast(half8, bh), blv = __builtin_bit_cast(half8, bl);
          c[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bhv, c[u], 0, 0, 0);
          c[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, blv, c[u], 0, 0, 0);
          c[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bhv, c[u], 0, 0, 0);
        }
      }
      // C element e: row 16 rt + 4 q + e = channel of block rt, i = e of this lane
#pragma unroll
      for (int u = 0; u < NS; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t ph = bhi[u][rt][e >> 1], pq = blo[u][rt][e >> 1];
          const int sh = (e & 1) * 16;
          const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)(ph >> sh));
          const _Float16 dl = __builtin_bit_cast(_Float16, (uint16_t)(pq >> sh));
          e_lane[u] = fmaf(c[u][e], (float)dl, fmaf(c[u][e], (float)dh, e_lane[u]));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      float el = e_lane[u];
      el += __shfl_xor(el, 16);
      el += __shfl_xor(el, 32);
      const float e = ldexpf(el, ex - 2 * kd) + 0.0f;  // (+0 turns a -0 into +0)
      if (livev[u] && q4 == 0) {
        if (errors) errors[((size_t)kv[u] * M + m_begin + rv_[u]) * G + j] = e;
        if (fabsf(e) < INFINITY) atomicMin(&best_key[rv_[u]], clip_key(e, kv[u]));
      }
    }
  }
  __syncthreads();
  for (int r = tid; r < R; r += kClipThreads) {
    const unsigned long long key = best_key[r];
    const int best = key == ~0ull ? -1 : (int)(uint32_t)key;
    const size_t o = (size_t)(m_begin + r) * G + j;
    clip_out[o] = best >= 0 ? ratios.v[best] : 1.0f;
    if (best_out) best_out[o] = best;
  }
}

}  // namespace

int gram_tokens_per_split(int64_t N, int64_t K) {
  // enough splits to give the chip about kGramTargetBlocks blocks, each at least 256 tokens
  // (a whole number of stages), and at most 64 splits
  const int64_t spans = (K + kGramSpan - 1) / kGramSpan;
  int64_t sp = spans > 0 ? (kGramTargetBlocks + spans - 1) / spans : 1;
  const int64_t by_tokens = (N + kGramFlush - 1) / kGramFlush;
  if (sp > by_tokens) sp = by_tokens;
  if (sp > 64) sp = 64;
  if (sp < 1) sp = 1;
  int64_t tps = (N + sp - 1) / sp;
  tps = (tps + kGramStage - 1) / kGramStage * kGramStage;
  return (int)(tps > kGramStage ? tps : kGramStage);
}

int gram_splits(int64_t N, int64_t K, int group_size) {
  (void)group_size;
  const int64_t tps = gram_tokens_per_split(N, K);
  const int64_t sp = (N + tps - 1) / tps;
  return (int)(sp > 1 ? sp : 1);
}

int gram_chunks(int group_size) {
  return (group_size * group_size + kGramChunk - 1) / kGramChunk;
}

hipError_t launch_group_gram(const uint16_t* X, const float* s, int N, int K, int group_size,
                             float* partials, double* G64, double* cmax, uint16_t* Ghi,
                             uint16_t* Glo, int32_t* gexp, hipStream_t stream) {
  if (K <= 0) return hipSuccess;
  const int tps = gram_tokens_per_split(N, K);
  const int splits = gram_splits(N, K, group_size);
  dim3 grid((K + kGramSpan - 1) / kGramSpan, splits);
  switch (group_size) {
    case 32:
      hipLaunchKernelGGL(k_gram_mfma<32>, grid, dim3(kGramThreads), 0, stream, X, N, K, tps,
                         partials);
      break;
    case 64:
      hipLaunchKernelGGL(k_gram_mfma<64>, grid, dim3(kGramThreads), 0, stream, X, N, K, tps,
                         partials);
      break;
    case 128:
      hipLaunchKernelGGL(k_gram_mfma<128>, grid, dim3(kGramThreads), 0, stream, X, N, K, tps,
                         partials);
      break;
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nc = gram_chunks(group_size);
  dim3 g2(K / group_size, nc);
  hipLaunchKernelGGL(k_gram_sum, g2, dim3(256), 0, stream, partials, group_size,
                     K / group_size, splits, s, G64, cmax);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gram_split, g2, dim3(256), 0, stream, G64, group_size, cmax, Ghi, Glo,
                     gexp);
  return hipGetLastError();
}

hipError_t launch_clip_search(const uint16_t* W, const float* s, const uint16_t* Ghi,
                              const uint16_t* Glo, const int32_t* gexp, int M, int K, int w_bit,
                              int group_size, int zero_point, const ClipList& ratios,
                              int n_ratio, float* clip_out, int32_t* best_out, float* errors,
                              hipStream_t stream) {
  if (M <= 0 || K <= 0) return hipSuccess;
  if (n_ratio < 1 || n_ratio > kMaxClip) return hipErrorInvalidValue;
  const void* fn;
  switch (group_size) {
    case 32: fn = (const void*)k_clip_mfma<32, kClipSlices>; break;
    case 64: fn = (const void*)k_clip_mfma<64, kClipSlices>; break;
    case 128: fn = (const void*)k_clip_mfma<128, kClipSlices>; break;
    default: return hipErrorInvalidValue;
  }
  // rows per block: the fewest rounds of resident blocks times the work of one block
  // (its slices per wave plus about two slices' worth of staging)
  // (resident blocks per device, queried once per group size: one kind of device assumed)
  static std::atomic<int64_t> cap_cache[3];
  const int gi = group_size == 32 ? 0 : group_size == 64 ? 1 : 2;
  int64_t cap = cap_cache[gi].load(std::memory_order_relaxed);
  if (cap <= 0) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t st = hipGetDevice(&dev);
    if (st == hipSuccess)
      st = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (st == hipSuccess)
      st = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kClipThreads, 0);
    if (st != hipSuccess) return st;
    cap = (int64_t)max(1, cus) * max(1, per_cu);
    cap_cache[gi].store(cap, std::memory_order_relaxed);
  }
  const int ngroups = K / group_size;
  int rows = 1;
  int64_t best_cost = -1;
  for (int r = 1; r <= kClipMaxRows; ++r) {
    const int64_t blocks = (int64_t)ngroups * ((M + r - 1) / r);
    const int64_t rounds = (blocks + cap - 1) / cap;
    const int64_t per_wave = ((int64_t)min(r, M) * n_ratio + 16 * kClipWaves - 1) /
                             (16 * kClipWaves);  // slices per wave
    const int64_t cost = rounds * (per_wave + 2);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      rows = r;
    }
  }
  dim3 grid(ngroups, (M + rows - 1) / rows);
#define AWQ_CLIP(GS)                                                                        \
  hipLaunchKernelGGL((k_clip_mfma<GS, kClipSlices>), grid, dim3(kClipThreads), 0, stream, W, s, Ghi, Glo,   \
                     gexp, M, K, w_bit, zero_point, ratios, n_ratio, rows, clip_out,          \
                     best_out, errors)
  switch (group_size) {
    case 32: AWQ_CLIP(32); break;
    case 64: AWQ_CLIP(64); break;
    default: AWQ_CLIP(128); break;
  }
#undef AWQ_CLIP
  return hipGetLastError();
}

}  // namespace awq
