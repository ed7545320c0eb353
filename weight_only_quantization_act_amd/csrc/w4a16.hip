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
#define AWQ_GEMV_RB 4  // rows whose code loads are in flight together (256-thread blocks)
#endif
#ifndef AWQ_GEMV_TARGET_WAVES
#define AWQ_GEMV_TARGET_WAVES 4096  // waves the row split aims for
#endif
#ifndef AWQ_GEMV_MAX_ROWS
#define AWQ_GEMV_MAX_ROWS 64
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

// Codes, step and zero of RB consecutive rows for this thread's chunk.  Rows at or past
// m_end are not loaded (their registers keep stale values and are never read).
template <int RB>
struct RowBatch {
  u32x4 cw[RB];
  float st[RB];
  h2 zz[RB];
};

template <int RB>
__device__ __forceinline__ void load_rows(RowBatch<RB>& b, const uint8_t* __restrict__ codes,
                                          const uint16_t* __restrict__ scales,
                                          const uint16_t* __restrict__ zeros, int m0, int m_end,
                                          bool has, int tid, int K, int gpr, int gcol) {
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int m = m0 + r;
    if (has && m < m_end) {
      b.cw[r] = *(const u32x4*)(codes + (size_t)m * (K >> 1) + (size_t)tid * 16);
      const size_t gi = (size_t)m * gpr + gcol;
      b.st[r] = h2f(scales[gi]);
      const uint16_t zh = f2h(h2f(zeros[gi]) + 1024.0f);
      b.zz[r] = as_h2((uint32_t)zh | ((uint32_t)zh << 16));
    }
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
        h2 d[16];
        chunk_delta(b.cw[r], b.zz[r], nib, one024_v, d);
#pragma unroll
        for (int t = 0; t < T; ++t)
          red[tid * rs + ((m0 - m_begin) + r) * T + t] = chunk_dot(d, xt[t]) * b.st[r];
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
// (K/32 chunks x (rows*T + 1) floats) stay within kGemvLdsFloats; at least 8.
constexpr int kGemvLdsFloats = 24576;  // 96 KiB
int gemv_rows(const GemvPlan& p, int T, int K) {
  const int nchunks = K / 32 > 0 ? K / 32 : 1;
  int cap = (kGemvLdsFloats / nchunks - 1) / T;
  cap = (cap / 8) * 8;
  int rows = p.rows < cap ? p.rows : cap;
  return rows < 8 ? 8 : rows;
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

}  // namespace

GemvPlan w4a16_gemv_plan(int64_t M, int64_t K) {
  GemvPlan p{};
  const int64_t nchunks = K / 32;
  p.threads = (int)(((nchunks + 63) / 64) * 64);
  if (p.threads < 64) p.threads = 64;
  const int nwaves = p.threads / 64;
  // enough blocks to give every CU several waves; whole row batches; at most 64 rows
  int64_t rows = (M * nwaves) / AWQ_GEMV_TARGET_WAVES;
  rows = (rows / 8) * 8;
  if (rows < 8) rows = 8;
  if (rows > AWQ_GEMV_MAX_ROWS) rows = AWQ_GEMV_MAX_ROWS;
  p.rows = (int)rows;
  return p;
}

hipError_t launch_w4a16_gemv(const uint8_t* codes, const uint16_t* scales,
                             const uint16_t* zeros, const uint16_t* x, const float* s, int T,
                             int M, int K, int group_size, uint16_t* y, hipStream_t stream) {
  if (T <= 0 || M <= 0 || K < 0) return hipSuccess;  // K = 0 still writes y = 0
  if (K % 32 != 0 || K > kGemvMaxK) return hipErrorInvalidValue;
  int log2g = 0;
  while ((1 << log2g) < group_size) ++log2g;
  if ((1 << log2g) != group_size || group_size < 32) return hipErrorInvalidValue;
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
