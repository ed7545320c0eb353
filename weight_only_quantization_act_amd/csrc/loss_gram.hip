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
//   k_gram_full        G's upper triangle in 128 x 128 tiles, every tile over all tokens:
//                      fp16 products (exact in fp32) summed on the matrix cores in fp32 over
//                      at most 256 tokens, those sums added in fp64, the total rounded to
//                      fp32 and written at (a, b) and (b, a); each tile's largest |G|.
//   k_gram_full_split  one power of two 2^-ex for the whole matrix (its largest magnitude
//                      into [2^13, 2^14)) and the operand of the per-grid-point product:
//                      G' 2^-ex in fp16, where G' is G with its blocks of kLossBN x kLossBN
//                      above the diagonal doubled (exact), those below it zero and its
//                      diagonal zero.  With d the rows of dW,
//                      sum_r d_r G d_r^T = sum over column blocks a of d_a . (G' d)_a
//                                          + sum_c (sum_r d_rc^2) G_cc,
//                      the product for column block a only runs over k from block a on,
//                      and the diagonal term, which carries most of the sum, is taken in
//                      fp32 from gdiag = diag(G) 2^-ex (fp32) in the product's epilogue,
//                      so that only the off-diagonal entries are rounded to fp16.
#include <hip/hip_runtime.h>

#include <math.h>

#include "awq_internal.h"
#include "quantizer.h"

namespace awq {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kGfThreads = 512;  // 8 waves, one 16-row tile row each
constexpr int kGfSpan = 128;     // channels of a tile side
#ifndef AWQ_GF_STAGE
#define AWQ_GF_STAGE 128
#endif
constexpr int kGfStage = AWQ_GF_STAGE;  // tokens per LDS stage (32-token k-steps)
constexpr int kGfOct = kGfStage / 64;   // 8-token octets a wave stages per stage
constexpr int kGfFlush = 256;           // tokens summed in fp32 before adding into fp64
constexpr int kGfXtp = kGfStage + 4;    // LDS row of a transposed stage (fp16, 8-byte aligned)
static_assert(kGfStage == 64 || kGfStage == 128, "64 or 128 tokens a stage");
constexpr int kGfSplitChunk = 4096;  // entries per block of the split pass

__device__ __forceinline__ float nan_maxf(float m, float a) {
  return (a > m || a != a) ? a : m;
}

// Block b: the b-th pair (sa <= sb) of 128-channel spans in row-major order of the upper
// triangle.  A stage of kGfStage tokens of both spans is stored transposed in LDS (xa, xb
// [channel][token]): lane l of wave w loads the channel pair (2 l, 2 l + 1) of the 8-token
// octets w (and w + 8) of each span and interleaves the halves with v_perm.  The MFMA fragment
// (16x16x32 f16) of a 16-channel block and a 32-token k-step is then lane (p, q)'s 16 bytes
// at row 16 block + p, token 32 ks + 8 q; wave w multiplies its tile row w of span a (A)
// with the 8 tile columns of span b (B).  C element e of a tile is row 4 q + e, column p.
__global__ __launch_bounds__(kGfThreads) void k_gram_full(const uint16_t* __restrict__ X,
                                                          int N, int K, int nspan,
                                                          float* __restrict__ G,
                                                          float* __restrict__ tmax) {
  __shared__ __attribute__((aligned(16))) uint16_t xa[kGfSpan * kGfXtp];
  __shared__ __attribute__((aligned(16))) uint16_t xb[kGfSpan * kGfXtp];
  __shared__ float wmax[kGfThreads / 64];
  // (sa, sb) of this block
  int sa = 0, rem = blockIdx.x;
  while (rem >= nspan - sa) {
    rem -= nspan - sa;
    ++sa;
  }
  const int sb = sa + rem;
  const int ca = sa * kGfSpan, cb = sb * kGfSpan;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, pl = lane & 15;
  const bool pa_ok = ca + 2 * lane < K, pb_ok = cb + 2 * lane < K;

  floatx4 acc[8];
  double acc64[8][4];
#pragma unroll
  for (int tc = 0; tc < 8; ++tc) {
    acc[tc] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc64[tc][e] = 0.0;
  }

  // the next stage's token values (octets wave, wave + 8), in flight during the MFMAs
  uint32_t da[kGfOct][8], db[kGfOct][8];
  auto load_stage = [&](int t0) {
#pragma unroll
    for (int o = 0; o < kGfOct; ++o)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + 8 * (wave + 8 * o) + e;
        const size_t row = (size_t)t * K;
        da[o][e] = (pa_ok && t < N) ? *(const uint32_t*)(X + row + ca + 2 * lane) : 0u;
        db[o][e] = (pb_ok && t < N) ? *(const uint32_t*)(X + row + cb + 2 * lane) : 0u;
      }
  };
  auto put = [&](uint16_t* xt, const uint32_t (&d)[8], int oct) {
    uint2 lo0, lo1, hi0, hi1;  // channel 2 l (low halves) and 2 l + 1 (high halves)
    lo0.x = __builtin_amdgcn_perm(d[1], d[0], 0x05040100u);
    lo0.y = __builtin_amdgcn_perm(d[3], d[2], 0x05040100u);
    lo1.x = __builtin_amdgcn_perm(d[5], d[4], 0x05040100u);
    lo1.y = __builtin_amdgcn_perm(d[7], d[6], 0x05040100u);
    hi0.x = __builtin_amdgcn_perm(d[1], d[0], 0x07060302u);
    hi0.y = __builtin_amdgcn_perm(d[3], d[2], 0x07060302u);
    hi1.x = __builtin_amdgcn_perm(d[5], d[4], 0x07060302u);
    hi1.y = __builtin_amdgcn_perm(d[7], d[6], 0x07060302u);
    uint16_t* r0 = xt + (2 * lane) * kGfXtp + 8 * oct;
    *(uint2*)r0 = lo0;
    *(uint2*)(r0 + 4) = lo1;
    *(uint2*)(r0 + kGfXtp) = hi0;
    *(uint2*)(r0 + kGfXtp + 4) = hi1;
  };
  auto frag = [&](const uint16_t* xt, int blk, int ks) {
    const uint16_t* src = xt + (16 * blk + pl) * kGfXtp + 32 * ks + 8 * q4;
    const uint2 u0 = *(const uint2*)src, u1 = *(const uint2*)(src + 4);
    const u32x4 v = {u0.x, u0.y, u1.x, u1.y};
    return __builtin_bit_cast(half8, v);
  };

  if (N > 0) load_stage(0);
  for (int t0 = 0; t0 < N; t0 += kGfStage) {
#pragma unroll
    for (int o = 0; o < kGfOct; ++o) {
      put(xa, da[o], wave + 8 * o);
      put(xb, db[o], wave + 8 * o);
    }
    __syncthreads();
    if (t0 + kGfStage < N) load_stage(t0 + kGfStage);
#pragma unroll
    for (int ks = 0; ks < kGfStage / 32; ++ks) {
      const half8 fa = frag(xa, wave, ks);
#pragma unroll
      for (int tc = 0; tc < 8; ++tc)
        acc[tc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, frag(xb, tc, ks), acc[tc], 0, 0, 0);
    }
    __syncthreads();
    if ((t0 + kGfStage) % kGfFlush == 0 || t0 + kGfStage >= N) {
#pragma unroll
      for (int tc = 0; tc < 8; ++tc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc64[tc][e] += (double)acc[tc][e];
        acc[tc] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  }

  // G[a][b] for a = ca + 16 w + 4 q + e, b = cb + 16 tc + p; the transposed tile as
  // 16-byte rows G[b][a .. a + 3]
  float mx = 0.0f;
  const int a0 = ca + 16 * wave + 4 * q4;
#pragma unroll
  for (int tc = 0; tc < 8; ++tc) {
    const int b = cb + 16 * tc + pl;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = (float)acc64[tc][e];
      mx = nan_maxf(mx, fabsf(v[e]));
    }
    if (b < K) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (a0 + e < K) G[(size_t)(a0 + e) * K + b] = v[e];
      if (sa != sb && a0 < K) *(float4*)(G + (size_t)b * K + a0) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = nan_maxf(mx, __shfl_xor(mx, o));
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  if (tid == 0) {
    float m = wmax[0];
#pragma unroll
    for (int w = 1; w < kGfThreads / 64; ++w) m = nan_maxf(m, wmax[w]);
    tmax[blockIdx.x] = m;
  }
}

// Block c: entries [c chunk, (c + 1) chunk) of G (K x K).  Every block derives the same
// exponent from all tile maxima (NaN if any entry is NaN: then ex = 0 and the NaN reaches
// the losses); block 0 publishes it.
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
  for (int i = tid; i < kGfSplitChunk; i += 256) {
    const int64_t j = base + i;
    if (j >= KK) break;
    const int64_t row = j / K, col = j - (j / K) * K;
    const int64_t ra = row / kLossBN, cb = col / kLossBN;
    if (row == col) {
      gdiag[row] = ldexpf(G[j], -ex);
      Gh[j] = 0;
    } else {
      const float g = cb < ra ? 0.0f : (cb > ra ? 2.0f * G[j] : G[j]);
      Gh[j] = f2h(ldexpf(g, -ex));
    }
  }
}

}  // namespace

int gram_full_tiles(int64_t K) {
  const int64_t ns = (K + kGfSpan - 1) / kGfSpan;
  return (int)(ns * (ns + 1) / 2);
}

hipError_t launch_gram_full(const uint16_t* X, int N, int K, float* G, float* tmax,
                            uint16_t* Gh, float* gdiag, int32_t* gexp, hipStream_t stream) {
  if (K <= 0) return hipSuccess;
  if (K % 2 != 0) return hipErrorInvalidValue;
  const int nspan = (K + kGfSpan - 1) / kGfSpan;
  const int ntiles = gram_full_tiles(K);
  hipLaunchKernelGGL(k_gram_full, dim3(ntiles), dim3(kGfThreads), 0, stream, X, N, K, nspan, G,
                     tmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t KK = (int64_t)K * K;
  const int64_t blocks = (KK + kGfSplitChunk - 1) / kGfSplitChunk;
  hipLaunchKernelGGL(k_gram_full_split, dim3((unsigned)blocks), dim3(256), 0, stream, G, K, KK,
                     tmax, ntiles, Gh, gdiag, gexp);
  return hipGetLastError();
}

}  // namespace awq
