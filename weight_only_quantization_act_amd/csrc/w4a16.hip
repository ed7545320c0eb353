// W4A16 product of a packed layer: y[t][m] = sum_i (c[m][i] - z[m][g(i)]) * step[m][g(i)] * x~[t][i]
//
// Pages: "AWQ量化技术解析" (kwkr.cn) §1.2 (dequantised weight = int4 code x fp16 scale) and
// §4.2 (dequantisation fused into the product); "AWQ 量化全流程拆解" (lnrq.cn) §四 (a GEMV
// kernel for single requests, a GEMM kernel for batches); "AWQ" scholia-log notes §4.3
// (S^-1 folded into the preceding operation, so the product sees x~ = x / s).
//
// Decode shape (a few tokens): the product is bound by reading the 4-bit codes from HBM
// (M*K/2 bytes) and has almost no reuse, so it runs on the vector ALUs:
//   - a thread owns 32 consecutive input channels (one 16-byte code chunk per row) and
//     keeps x~ for them in registers as fp16 pairs for every token;
//   - the 8 nibbles of a 32-bit code word become fp16 (c - z) pairs with two integer ops
//     and one packed fp16 subtraction: the fp16 bit pattern 0x6400 | c is 1024 + c, and
//     (1024 + c) - (1024 + z) is exact for integer codes and zeros below 16;
//   - v_dot2_f32_f16 multiplies each pair by the matching x~ pair and accumulates in fp32
//     (fp16 x fp16 products are exact in fp32);
//   - the lane's 32 channels lie in one quantisation group (g >= 32), so its partial sum is
//     multiplied once by the group's step; lanes are summed with DPP moves and shuffles,
//     waves in a fixed order through LDS, and the result is rounded to fp16.
// A code word's nibble n (bits 4n..4n+3) is input channel n of the word (even channel in
// the low nibble of each byte), so the pairs come out as channels (n, n + 4), n = 0..3; x~
// is loaded into registers in the same pairing.
#include <hip/hip_runtime.h>

#include "awq_internal.h"
#include "quantizer.h"

namespace awq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef AWQ_GEMV_RB
#define AWQ_GEMV_RB 2  // rows whose code loads are in flight together (256-thread blocks)
#endif
#ifndef AWQ_GEMV_TARGET_WAVES
#define AWQ_GEMV_TARGET_WAVES 4096  // waves the row split aims for
#endif
#ifndef AWQ_GEMV_MAX_ROWS
#define AWQ_GEMV_MAX_ROWS 64
#endif
#ifndef AWQ_GEMV_MIN_ROWS
// rows per block at least (a multiple of the row batch).  Same-device graph replays, one
// token, S^-1 folded / s given: 4096 x 4096 6.3 / 8.3 us against 6.7 / 8.7 for 8 rows and
// batches of 4; 28672 x 8192 28.1 / 32.9 against 30.3 / 35.4; 11008 x 4096 9.1 / 15.1
// against 9.4 / 13.5
#define AWQ_GEMV_MIN_ROWS 4
#endif

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

// x~ for channels [c0, c0 + 32) of one token, as 16 fp16 pairs in code-word order.
__device__ __forceinline__ void load_xt(const uint16_t* __restrict__ xrow,
                                        const float* __restrict__ s, int c0, h2 out[16]) {
  uint16_t v[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 r = *(const u32x4*)(xrow + c0 + 8 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * j + 2 * e] = (uint16_t)(r[e] & 0xffffu);
      v[8 * j + 2 * e + 1] = (uint16_t)(r[e] >> 16);
    }
  }
  if (s != nullptr) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 sv = *(const f32x4*)(s + c0 + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = f2h(h2f(v[4 * j + e]) / sv[e]);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int n = 0; n < 4; ++n)
      out[4 * j + n] = as_h2((uint32_t)v[8 * j + n] | ((uint32_t)v[8 * j + n + 4] << 16));
}

// (c - z) for the 32 codes of one chunk as 16 fp16 pairs in code-word order.  nib is the
// nibble-pair mask 0x000F000F and one024 the fp16 pair (1024, 1024), 0x64006400; both come
// in as kernel arguments, so each pair costs one v_and_or_b32 (plus a shift) and one
// packed subtraction instead of separate and/or instructions with literal operands.
__device__ __forceinline__ void chunk_delta(const u32x4 cw, h2 zz, uint32_t nib,
                                            uint32_t one024, h2 d[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = cw[j];
#pragma unroll
    for (int n = 0; n < 4; ++n) d[4 * j + n] = as_h2(((w >> (4 * n)) & nib) | one024) - zz;
  }
}

// sum over the chunk of (c - z) * x~ for one token, fp32 accumulation.
__device__ __forceinline__ float chunk_dot(const h2 d[16], const h2 xt[16]) {
  float acc = 0.0f;
#pragma unroll
  for (int p = 0; p < 16; ++p) acc = __builtin_amdgcn_fdot2(d[p], xt[p], acc, false);
  return acc;
}

// Codes, step and zero (raw fp16) of RB consecutive rows for this thread's chunk.  Every
// lane loads: rows at or past m_end read row m_end - 1 and lanes without a chunk read
// chunk 0, values the multiply never uses.  The loads are one straight-line run and
// nothing here uses a loaded value (the step and zero are converted when the batch is
// multiplied), so no wait for a row's loads is needed before the next row's are issued.
template <int RB>
struct RowBatch {
  u32x4 cw[RB];
  uint16_t st[RB], zh[RB];
};

template <int RB>
__device__ __forceinline__ void load_rows(RowBatch<RB>& b, const uint8_t* __restrict__ codes,
                                          const uint16_t* __restrict__ scales,
                                          const uint16_t* __restrict__ zeros, int m0, int m_end,
                                          bool has, int tid, int K, int gpr, int gcol) {
  const int tc = has ? tid : 0;
  const int gc = has ? gcol : 0;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int m = min(m0 + r, m_end - 1);
    b.cw[r] = *(const u32x4*)(codes + (size_t)m * (K >> 1) + (size_t)tc * 16);
    const size_t gi = (size_t)m * gpr + gc;
    b.st[r] = scales[gi];
    b.zh[r] = zeros[gi];
  }
}

// Block: nthreads = 64 * nwaves threads (at most MAXT); thread tid owns code chunk tid
// (32 channels) of every row in [m_begin, m_end), RB rows at a time.  The loads of the
// next RB rows are issued before the current ones are multiplied, and the first batch's
// before x~ is formed, so HBM traffic overlaps the ALU work.
// Each thread writes one fp32 partial per (row, token) to LDS, red[chunk * rs + o] with
// o = row * T + token and an odd stride rs = rows_per_block * T + 1 (so neither the
// writes, one chunk per lane, nor the reads, one output per lane, hit a bank twice); after
// one barrier, output o is the sum over chunks in order.
template <int T, int MAXT, int RB>
__global__ __launch_bounds__(MAXT) void k_w4a16_gemv(const uint8_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint16_t* __restrict__ zeros,
                                                     const uint16_t* __restrict__ x,
                                                     const float* __restrict__ s, int M, int K,
                                                     int log2g, int rows_per_block,
                                                     uint32_t nib, uint32_t one024,
                                                     uint16_t* __restrict__ y) {
  extern __shared__ float red[];
  const int nthreads = blockDim.x;
  const int tid = threadIdx.x;
  const int nchunks = K >> 5;
  const int gpr = K >> log2g;
  const int m_begin = blockIdx.x * rows_per_block;
  const int m_end = min(M, m_begin + rows_per_block);
  const int rs = rows_per_block * T + 1;
  const bool has = tid < nchunks;
  const int gcol = (tid * 32) >> log2g;
  // one of the two decode constants must sit in a VGPR for v_and_or_b32 (a VOP3 can read
  // one scalar register); the copy is opaque so the compiler keeps it there.
  uint32_t one024_v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(one024_v) : "s"(one024));

  RowBatch<RB> ba = {}, bb = {};
  load_rows<RB>(ba, codes, scales, zeros, m_begin, m_end, has, tid, K, gpr, gcol);

  h2 xt[T][16];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (has) {
      load_xt(x + (size_t)t * K, s, tid * 32, xt[t]);
    } else {
#pragma unroll
      for (int p = 0; p < 16; ++p) xt[t][p] = as_h2(0u);
    }
  }

  // Row batches alternate between two register sets: while one batch is multiplied, the
  // next one's loads are in flight.
  auto process = [&](const RowBatch<RB>& b, int m0) {
    if (!has) return;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (m0 + r < m_end) {
        const uint16_t zh = f2h(h2f(b.zh[r]) + 1024.0f);
        const h2 zz = as_h2((uint32_t)zh | ((uint32_t)zh << 16));
        const float st = h2f(b.st[r]);
        h2 d[16];
        chunk_delta(b.cw[r], zz, nib, one024_v, d);
#pragma unroll
        for (int t = 0; t < T; ++t)
          red[tid * rs + ((m0 - m_begin) + r) * T + t] = chunk_dot(d, xt[t]) * st;
      }
    }
  };
  for (int m0 = m_begin; m0 < m_end; m0 += 2 * RB) {
    if (m0 + RB < m_end)
      load_rows<RB>(bb, codes, scales, zeros, m0 + RB, m_end, has, tid, K, gpr, gcol);
    process(ba, m0);
    if (m0 + RB >= m_end) break;
    if (m0 + 2 * RB < m_end)
      load_rows<RB>(ba, codes, scales, zeros, m0 + 2 * RB, m_end, has, tid, K, gpr, gcol);
    process(bb, m0 + RB);
  }
  __syncthreads();
  const int n_out = (m_end - m_begin) * T;
  for (int o = tid; o < n_out; o += nthreads) {
    float v = 0.0f;
    for (int c = 0; c < nchunks; ++c) v += red[c * rs + o];
    const int r = o / T, t = o - (o / T) * T;
    y[(size_t)t * M + m_begin + r] = f2h(v);
  }
}

// Rows per block for T tokens: the plan's count, cut so that the LDS partials
// (K/32 chunks x (rows*T + 1) floats) stay within kGemvLdsFloats; at least AWQ_GEMV_MIN_ROWS.
constexpr int kGemvLdsFloats = 24576;  // 96 KiB
int gemv_rows(const GemvPlan& p, int T, int K) {
  const int nchunks = K / 32 > 0 ? K / 32 : 1;
  int cap = (kGemvLdsFloats / nchunks - 1) / T;
  cap = (cap / AWQ_GEMV_MIN_ROWS) * AWQ_GEMV_MIN_ROWS;
  int rows = p.rows < cap ? p.rows : cap;
  return rows < AWQ_GEMV_MIN_ROWS ? AWQ_GEMV_MIN_ROWS : rows;
}

template <int T, int MAXT, int RB>
hipError_t launch_gemv_t(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                         const uint16_t* x, const float* s, int M, int K, int log2g,
                         const GemvPlan& p, uint16_t* y, hipStream_t stream) {
  const int rows = gemv_rows(p, T, K);
  const int blocks = (M + rows - 1) / rows;
  const int nchunks = K / 32 > 0 ? K / 32 : 1;
  const size_t lds = (size_t)nchunks * (rows * T + 1) * sizeof(float);
  hipLaunchKernelGGL((k_w4a16_gemv<T, MAXT, RB>), dim3(blocks), dim3(p.threads), lds, stream,
                     codes, scales, zeros, x, s, M, K, log2g, rows, 0x000F000Fu, 0x64006400u,
                     y);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                       const uint16_t* x, const float* s, int T, int M, int K, int log2g,
                       const GemvPlan& p, uint16_t* y, hipStream_t stream) {
#define AWQ_GEMV(TT, MT, RB) \
  launch_gemv_t<TT, MT, RB>(codes, scales, zeros, x, s, M, K, log2g, p, y, stream)
  if (p.threads <= 256) {
    switch (T) {
      case 1: return AWQ_GEMV(1, 256, AWQ_GEMV_RB);
      case 2: return AWQ_GEMV(2, 256, AWQ_GEMV_RB);
      case 3: return AWQ_GEMV(3, 256, AWQ_GEMV_RB);
      case 4: return AWQ_GEMV(4, 256, AWQ_GEMV_RB);
    }
  } else {
    switch (T) {
      case 1: return AWQ_GEMV(1, 1024, 4);
      case 2: return AWQ_GEMV(2, 1024, 4);
      case 3: return AWQ_GEMV(3, 1024, 4);
      case 4: return AWQ_GEMV(4, 1024, 2);
    }
  }
#undef AWQ_GEMV
  return hipErrorInvalidValue;
}

// ---- small batches on the matrix cores ---------------------------------------------
//
// For 2..16 tokens the VALU kernel's cost grows with T (16 dot2 per 32 channels per token);
// here one v_mfma_f32_16x16x32_f16 multiplies 16 rows x 32 channels by up to 16 tokens, so
// the per-weight work (the nibble decode) does not depend on T.  MFMA 16x16x32 f16 lane
// layout: A row (l mod 16) with k = 8 (l div 16) + e, B column (l mod 16) with the same k,
// C row 4 (l div 16) + e, column (l mod 16).
//   - A = (c - z) of 16 weight rows, exact in fp16 (decoded as in the VALU kernel, pairs
//     (n, n + 4) of each code word), B = x~ of the tokens (lane column = token; columns
//     >= T are zero), read from global memory and permuted into the same pair order.
//   - The 32 k-values of one MFMA are 32 channels of one quantisation group: lane group
//     q = l div 16 supplies channels q g/4 + 8 u + e of the group for MFMA u, u < g/32.
//     A group's MFMAs accumulate into their own fp32 tile, which is then multiplied by the
//     group's step for each row and added to the running fp32 result.
//   - A wave covers 2 or 4 row tiles (32 or 64 rows), so each B fragment feeds 2 or 4
//     MFMAs, and a range of groups; the (at most 8) waves of a block split the groups and
//     their results are added through LDS in a fixed order.  Code words and B fragments of
//     the next group are loaded while the current group is multiplied.
//   - Step and zero of the wave's rows are staged per 8 groups in a wave-private LDS slice
//     (two 2-byte loads per lane per group instead of one per row and MFMA).
constexpr int kMfmaMaxT = 16;         // tokens per pass
constexpr int kMfmaStageGroups = 8;   // groups of step/zero staged at once
constexpr int kMfmaMaxWaves = 8;      // two 8-wave blocks fit a CU at 128 VGPRs
constexpr int kMfmaTargetWaves = 4096;

// Tile geometry: TILES 16-row tiles per wave (4 when the layer has rows for one block per
// CU, else 2, for more blocks).  LDS per wave: the staged step and zero, then the
// wave's result tiles for the cross-wave sum.
template <int TILES>
struct MfmaGeo {
  static constexpr int ROWS = 16 * TILES;  // rows per block
  static constexpr int STAGE_BYTES = kMfmaStageGroups * ROWS * 4;
  static constexpr int LDS_PER_WAVE = 2 * STAGE_BYTES + TILES * 64 * 16;
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int GS, int kMfmaTiles>
__global__ __launch_bounds__(kMfmaMaxWaves * 64) void k_w4a16_mfma(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ zeros, const uint16_t* __restrict__ x, int M, int K, int T,
    uint32_t nib, uint32_t one024, uint16_t* __restrict__ y) {
  constexpr int WPL = GS / 32;  // code words (8 channels) per lane per group = MFMAs per group
  using Geo = MfmaGeo<kMfmaTiles>;
  constexpr int kMfmaRows = Geo::ROWS;
  constexpr int kMfmaStageBytes = Geo::STAGE_BYTES;
  constexpr int kMfmaLdsPerWave = Geo::LDS_PER_WAVE;
  // dynamic LDS, per wave: step (fp32) and (1024 + z) as an fp16 pair per staged group and
  // row, then the wave's result tiles for the cross-wave sum (kMfmaLdsPerWave bytes)
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  float (*st_sh)[kMfmaRows] = (float (*)[kMfmaRows])(lds + (size_t)w * kMfmaLdsPerWave);
  uint32_t (*zz_sh)[kMfmaRows] =
      (uint32_t (*)[kMfmaRows])(lds + (size_t)w * kMfmaLdsPerWave + kMfmaStageBytes);
  auto red = [&](int ww, int tl) -> floatx4* {
    return (floatx4*)(lds + (size_t)ww * kMfmaLdsPerWave + 2 * kMfmaStageBytes) + tl * 64;
  };
  const int ar = lane & 15, q = lane >> 4;
  const int m0 = blockIdx.x * kMfmaRows;
  const int G = K / GS;
  const int g0 = (int)(((long long)G * w) / nw), g1 = (int)(((long long)G * (w + 1)) / nw);
  uint32_t one024_v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(one024_v) : "s"(one024));

  floatx4 acc[kMfmaTiles];
#pragma unroll
  for (int i = 0; i < kMfmaTiles; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  const bool tok = ar < T;
  const uint16_t* xr = x + (size_t)(tok ? ar : 0) * K + q * (GS / 4);
  const size_t crow = (size_t)(K >> 1);

  // code words of the 4 row tiles and the B fragments of one group
  struct GroupBufs {
    uint32_t cw[kMfmaTiles][WPL];
    half8 bf[WPL];
  };
  // Every lane loads (lanes past the last token read token 0 and drop it; rows past
  // out_features read the last row and drop it), so the loads form one straight-line run
  // and the wait for the activations before their reordering leaves the code-word loads,
  // issued after them, in flight.
  auto load_group = [&](int j, GroupBufs& gb) {
#pragma unroll
    for (int u = 0; u < WPL; ++u) {
      const u32x4 r = *(const u32x4*)(xr + (size_t)j * GS + 8 * u);
      const uint32_t d0 = tok ? r[0] : 0u, d1 = tok ? r[1] : 0u, d2 = tok ? r[2] : 0u,
                     d3 = tok ? r[3] : 0u;
      // B in code-word pair order: (c0, c4), (c1, c5), (c2, c6), (c3, c7)
      const uint32_t p0 = (d0 & 0xffffu) | (d2 << 16), p1 = (d0 >> 16) | (d2 & 0xffff0000u);
      const uint32_t p2 = (d1 & 0xffffu) | (d3 << 16), p3 = (d1 >> 16) | (d3 & 0xffff0000u);
      const u32x4 pv = {p0, p1, p2, p3};
      gb.bf[u] = __builtin_bit_cast(half8, pv);
    }
#pragma unroll
    for (int tl = 0; tl < kMfmaTiles; ++tl) {
      const int row = min(m0 + 16 * tl + ar, M - 1);  // a row past the end: any codes, dropped
      const uint8_t* cp = codes + (size_t)row * crow + (size_t)j * (GS / 2) + q * (GS / 8);
      if constexpr (WPL == 4) {
        const u32x4 r = *(const u32x4*)cp;
        gb.cw[tl][0] = r[0]; gb.cw[tl][1] = r[1]; gb.cw[tl][2] = r[2]; gb.cw[tl][3] = r[3];
      } else if constexpr (WPL == 2) {
        const uint2 r = *(const uint2*)cp;
        gb.cw[tl][0] = r.x; gb.cw[tl][1] = r.y;
      } else {
        gb.cw[tl][0] = *(const uint32_t*)cp;
      }
    }
  };
  // step and zero of rows m0 .. m0 + 63 for groups js .. js + ng - 1, into the wave's LDS
  // slice.  Consecutive lanes take consecutive groups of one row, so a load instruction
  // touches a few rows' metadata (not 64 rows).  LDS operations of a wave complete in
  // order, so the slice's previous contents have been read by the time these writes land.
  auto stage = [&](int js) {
    const int ng = min(kMfmaStageGroups, g1 - js);
    for (int idx = lane; idx < kMfmaRows * ng; idx += 64) {
      const int r = idx / ng, jj = idx - (idx / ng) * ng;
      const int row = m0 + r;
      float stv = 0.0f;
      uint32_t zzv = 0x64006400u;
      if (row < M) {
        const size_t gi = (size_t)row * G + js + jj;
        stv = h2f(scales[gi]);
        const uint16_t zh = f2h(h2f(zeros[gi]) + 1024.0f);
        zzv = (uint32_t)zh | ((uint32_t)zh << 16);
      }
      st_sh[jj][r] = stv;
      zz_sh[jj][r] = zzv;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the slice is written
  };
  auto compute_group = [&](int j, const GroupBufs& gb) {
    const int jj = (j - g0) % kMfmaStageGroups;
#pragma unroll
    for (int tl = 0; tl < kMfmaTiles; ++tl) {
      const h2 zz = as_h2(zz_sh[jj][16 * tl + ar]);
      floatx4 cg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < WPL; ++u) {
        h2 dp[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) dp[n] = as_h2(((gb.cw[tl][u] >> (4 * n)) & nib) | one024_v) - zz;
        const u32x4 av = {__builtin_bit_cast(uint32_t, dp[0]), __builtin_bit_cast(uint32_t, dp[1]),
                          __builtin_bit_cast(uint32_t, dp[2]), __builtin_bit_cast(uint32_t, dp[3])};
        cg = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), gb.bf[u], cg,
                                                   0, 0, 0);
      }
      const floatx4 stv = *(const floatx4*)&st_sh[jj][16 * tl + 4 * q];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[tl][e] = fmaf(stv[e], cg[e], acc[tl][e]);
    }
  };
  // groups in pairs: while one group is multiplied, the next one's loads are in flight
  GroupBufs ga, gb2;
  if (g0 < g1) load_group(g0, ga);
  for (int j = g0; j < g1; j += 2) {
    if (j + 1 < g1) load_group(j + 1, gb2);
    if ((j - g0) % kMfmaStageGroups == 0) stage(j);
    compute_group(j, ga);
    if (j + 1 >= g1) break;
    if (j + 2 < g1) load_group(j + 2, ga);
    if ((j + 1 - g0) % kMfmaStageGroups == 0) stage(j + 1);
    compute_group(j + 1, gb2);
  }
#pragma unroll
  for (int tl = 0; tl < kMfmaTiles; ++tl) red(w, tl)[lane] = acc[tl];
  __syncthreads();
  // waves added in order; tile tl is summed by lanes of wave tl (or of wave 0 for every
  // tile when the block has fewer waves than tiles)
  for (int tl = w; tl < kMfmaTiles; tl += nw) {
    floatx4 v = red(0, tl)[lane];
    for (int ww = 1; ww < nw; ++ww) {
      const floatx4 o = red(ww, tl)[lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += o[e];
    }
    if (tok) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + 16 * tl + 4 * q + e;
        if (row < M) y[(size_t)ar * M + row] = f2h(v[e]);
      }
    }
  }
}

// x~[t][c] = fp16(fp32(x[t][c]) / s[c]): one correctly rounded fp32 division, then one
// rounding to fp16 -- the fold the product applies when s is given.  Eight channels a
// thread (in_features is a multiple of 32).
__global__ __launch_bounds__(256) void k_fold_inverse_scales(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ s,
                                                             int64_t n8, int K,
                                                             uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 8-channel chunk
  if (i >= n8) return;
  const int c0 = (int)((i * 8) % K);
  const u32x4 r = *(const u32x4*)(x + i * 8);
  const f32x4 s0 = *(const f32x4*)(s + c0), s1 = *(const f32x4*)(s + c0 + 4);
  const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint16_t lo = f2h(h2f((uint16_t)(r[j] & 0xffffu)) / sv[2 * j]);
    const uint16_t hi = f2h(h2f((uint16_t)(r[j] >> 16)) / sv[2 * j + 1]);
    o[j] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
  *(u32x4*)(out + i * 8) = o;
}

}  // namespace

GemvPlan w4a16_gemv_plan(int64_t M, int64_t K) {
  GemvPlan p{};
  const int64_t nchunks = K / 32;
  p.threads = (int)(((nchunks + 63) / 64) * 64);
  if (p.threads < 64) p.threads = 64;
  const int nwaves = p.threads / 64;
  // enough blocks to give every CU several waves; whole row batches; at most 64 rows
  int64_t rows = (M * nwaves) / AWQ_GEMV_TARGET_WAVES;
  rows = (rows / AWQ_GEMV_MIN_ROWS) * AWQ_GEMV_MIN_ROWS;
  if (rows < AWQ_GEMV_MIN_ROWS) rows = AWQ_GEMV_MIN_ROWS;
  if (rows > AWQ_GEMV_MAX_ROWS) rows = AWQ_GEMV_MAX_ROWS;
  p.rows = (int)rows;
  return p;
}

int w4a16_mfma_tiles(int64_t M) {
  return (M + 63) / 64 >= 256 ? 4 : 2;
}

int w4a16_mfma_waves(int64_t M, int64_t K, int group_size) {
  const int rows = 16 * w4a16_mfma_tiles(M);
  const int64_t blocks = (M + rows - 1) / rows;
  const int64_t G = K / group_size;
  int64_t nw = (kMfmaTargetWaves + blocks - 1) / blocks;  // waves in total
  if (nw > kMfmaMaxWaves) nw = kMfmaMaxWaves;
  if (nw > G) nw = G;
  if (nw < 1) nw = 1;
  return (int)nw;
}

hipError_t launch_w4a16_mfma(const uint8_t* codes, const uint16_t* scales,
                             const uint16_t* zeros, const uint16_t* x, int T, int M, int K,
                             int group_size, uint16_t* y, hipStream_t stream) {
  if (T <= 0 || M <= 0 || K <= 0) return hipSuccess;
  const int nw = w4a16_mfma_waves(M, K, group_size);
  const int tiles = w4a16_mfma_tiles(M);
  const int blocks = (M + 16 * tiles - 1) / (16 * tiles);
  for (int t0 = 0; t0 < T; t0 += kMfmaMaxT) {
    const int tc = T - t0 < kMfmaMaxT ? T - t0 : kMfmaMaxT;
    const uint16_t* xs = x + (size_t)t0 * K;
    uint16_t* ys = y + (size_t)t0 * M;
#define AWQ_MFMA(GS, TL)                                                                  \
  hipLaunchKernelGGL((k_w4a16_mfma<GS, TL>), dim3(blocks), dim3(nw * 64),                  \
                     (size_t)nw * MfmaGeo<TL>::LDS_PER_WAVE, stream, codes, scales, zeros, xs, \
                     M, K, tc, 0x000F000Fu, 0x64006400u, ys)
    switch (group_size * 8 + tiles) {
      case 32 * 8 + 2: AWQ_MFMA(32, 2); break;
      case 32 * 8 + 4: AWQ_MFMA(32, 4); break;
      case 64 * 8 + 2: AWQ_MFMA(64, 2); break;
      case 64 * 8 + 4: AWQ_MFMA(64, 4); break;
      case 128 * 8 + 2: AWQ_MFMA(128, 2); break;
      case 128 * 8 + 4: AWQ_MFMA(128, 4); break;
      default: return hipErrorInvalidValue;
    }
#undef AWQ_MFMA
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_w4a16_gemv(const uint8_t* codes, const uint16_t* scales,
                             const uint16_t* zeros, const uint16_t* x, const float* s, int T,
                             int M, int K, int group_size, uint16_t* y, hipStream_t stream) {
  if (T <= 0 || M <= 0 || K < 0) return hipSuccess;  // K = 0 still writes y = 0
  if (K % 32 != 0 || K > kGemvMaxK) return hipErrorInvalidValue;
  int log2g = 0;
  while ((1 << log2g) < group_size) ++log2g;
  if ((1 << log2g) != group_size || group_size < 32) return hipErrorInvalidValue;
  // S^-1 folded, several tokens: the matrix-core kernel
  if (s == nullptr && T >= kW4a16MfmaMinT && K > 0)
    return launch_w4a16_mfma(codes, scales, zeros, x, T, M, K, group_size, y, stream);
  const GemvPlan p = w4a16_gemv_plan(M, K);
  for (int t0 = 0; t0 < T; t0 += kGemvMaxT) {
    const int tc = T - t0 < kGemvMaxT ? T - t0 : kGemvMaxT;
    const hipError_t e = launch_gemv(codes, scales, zeros, x + (size_t)t0 * K, s, tc, M, K,
                                     log2g, p, y + (size_t)t0 * M, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace awq

namespace awq {

hipError_t launch_fold_inverse_scales(const uint16_t* x, const float* s, int T, int K,
                                      uint16_t* out, hipStream_t stream) {
  const int64_t n8 = (int64_t)T * K / 8;
  if (n8 <= 0) return hipSuccess;
  if (K % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fold_inverse_scales, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                     stream, x, s, n8, K, out);
  return hipGetLastError();
}

}  // namespace awq
