// Variants around the scale search: percentile-threshold fixed-factor scales and a
// blockwise Hadamard rotation of weights or activations.
//
// Pages: "AWQ量化" tutorial, 显著识别 (an indicator of channels above a percentile
// threshold of the importance scores), 缩放保护 and Python 演示 (scale those channels by a
// fixed factor, 70th percentile and factor 2 in the demo); "AWQ" scholia-log notes §5.1
// (an orthogonal R keeps WX = (WR)(R^T X); a normalised Hadamard spreads an outlier
// channel over many) and §5.2 (structured rotations in O(d log d)).
#include <hip/hip_runtime.h>

#include <math.h>

#include "awq_internal.h"
#include "quantizer.h"

namespace awq {

namespace {

constexpr int kSortThreads = 1024;

// One block: the two order statistics around position p/100 * (K-1) by radix selection,
// the linear-interpolation percentile in fp64 between them, then s_i = factor if a_i >
// threshold else 1, decided in fp64 exactly as the reference does.  Keys are the scores'
// fp32 bit patterns mapped to unsigned integers in value order (negative values
// complemented, non-negative ones with the sign bit set; NaN taken as +inf, so non-finite
// values sort last); four passes of an 8-bit histogram over the candidates that share the
// prefix found so far give the key at rank lo exactly, and one more pass its successor
// (the same key when ties reach past lo, else the smallest larger key).  A single block
// reads every a_i before it writes any s_i, so s_out may be a itself.
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v != v) v = INFINITY;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__global__ __launch_bounds__(kSortThreads) void k_threshold_scales(const float* __restrict__ a,
                                                                   int K, double percentile,
                                                                   float factor,
                                                                   float* __restrict__ s_out) {
  __shared__ uint32_t key[kMaxThresholdK];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_prefix, sel_rank, cnt_le, min_gt;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < K; i += kSortThreads) key[i] = order_key(a[i]);
  const double pos = percentile / 100.0 * (double)(K - 1);
  int lo = (int)floor(pos);
  if (lo > K - 1) lo = K - 1;
  const int hi = lo + 1 < K ? lo + 1 : K - 1;
  uint32_t prefix = 0u, mask = 0u, rank = (uint32_t)lo;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();  // (the first one also publishes the keys)
    for (int i = tid; i < K; i += kSortThreads) {
      const uint32_t u = key[i];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {  // wave 0: lane l holds bins 4l .. 4l + 3; an inclusive scan over lanes
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t sum = c0 + c1 + c2 + c3;
      uint32_t incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const uint32_t excl = incl - sum;
      if (rank >= excl && rank < incl) {  // exactly one lane
        const uint32_t c[4] = {c0, c1, c2, c3};
        uint32_t run = excl;
        int j = 0;
        while (rank >= run + c[j]) run += c[j++];
        sel_prefix = prefix | ((uint32_t)(4 * lane + j) << shift);
        sel_rank = rank - run;
      }
    }
    __syncthreads();
    prefix = sel_prefix;
    rank = sel_rank;
    mask |= 0xffu << shift;
  }
  const uint32_t klo = prefix;
  uint32_t khi = klo;
  if (hi != lo) {
    if (tid == 0) {
      cnt_le = 0u;
      min_gt = 0xffffffffu;
    }
    __syncthreads();
    uint32_t n = 0u, m = 0xffffffffu;
    for (int i = tid; i < K; i += kSortThreads) {
      const uint32_t u = key[i];
      n += (u <= klo) ? 1u : 0u;
      if (u > klo && u < m) m = u;
    }
    atomicAdd(&cnt_le, n);
    atomicMin(&min_gt, m);
    __syncthreads();
    khi = cnt_le > (uint32_t)hi ? klo : min_gt;
  }
  const double frac = pos - (double)lo;
  const double vlo = (double)key_value(klo), vhi = (double)key_value(khi);
  const double tau = vlo + frac * (vhi - vlo);
  for (int i = tid; i < K; i += kSortThreads) s_out[i] = ((double)a[i] > tau) ? factor : 1.0f;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp64 -> fp16, correctly rounded (nearest, ties to even): round to odd into fp32
// (toward zero, then set the last bit if anything was cut off), then nearest-even into
// fp16.  fp32 carries 13 more bits than fp16, so the second rounding sees the exact
// value's position relative to every fp16 midpoint and the two steps round once.
// With f = fp32(d) to nearest: exact, it is kept; otherwise the round-to-odd value is f's
// own bits when they are odd, else the neighbour toward d, whose last bit is odd (one step
// down in magnitude if f rounded away from zero, one step up if it rounded toward it).
__device__ __forceinline__ uint16_t d2h_rn(double d) {
  const float f = (float)d;
  const double fd = (double)f;
  uint32_t u = __float_as_uint(f);
  if (fd != d) u = (u & 1u) ? u : (fabs(fd) > fabs(d) ? u - 1u : u + 1u);
  return f2h(__uint_as_float(u));
}

// Cross-lane partner of a butterfly at lane distance D (D < 16) by DPP moves inside a row
// of 16 lanes: distances 1 and 2 by quad permutations, 8 by a rotation of the row by 8,
// and 4 by two masked row shifts (lanes 0-3 and 8-11 of a row read lane + 4, lanes 4-7
// and 12-15 lane - 4; a move writes only the lanes of the enabled 4-lane banks).
// A move with all banks enabled writes every lane; the masked pair for distance 4 writes
// the lanes of banks 0 and 2 first and those of banks 1 and 3 over the same register.
template <int CTRL, int BANKS>
__device__ __forceinline__ double dpp64(double src) {
  const uint64_t v = __builtin_bit_cast(uint64_t, src);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, BANKS, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, BANKS, false);
  return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}
template <int CTRL, int BANKS>
__device__ __forceinline__ double dpp64_over(double old, double src) {
  const uint64_t o = __builtin_bit_cast(uint64_t, old), v = __builtin_bit_cast(uint64_t, src);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)o, (int)(uint32_t)v,
                                                            CTRL, 0xf, BANKS, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(
      (int)(uint32_t)(o >> 32), (int)(uint32_t)(v >> 32), CTRL, 0xf, BANKS, false);
  return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}
constexpr int kDppQuadXor1 = 0xb1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4e;  // quad_perm [2, 3, 0, 1]
constexpr int kDppRowShl4 = 0x104, kDppRowShr4 = 0x114, kDppRowRor8 = 0x128;
template <int D>
__device__ __forceinline__ double partner(double x) {
  if constexpr (D == 1) return dpp64<kDppQuadXor1, 0xf>(x);
  if constexpr (D == 2) return dpp64<kDppQuadXor2, 0xf>(x);
  if constexpr (D == 4) return dpp64_over<kDppRowShr4, 0xa>(dpp64<kDppRowShl4, 0x5>(x), x);
  if constexpr (D == 8) return dpp64<kDppRowRor8, 0xf>(x);
  if constexpr (D >= 16) return __shfl_xor(x, D);
}

// Butterflies at lane distances D, 2D, ... below END: the lower lane of a pair keeps
// x + p, the upper one p - x, as fma(x, -1 or +1, p) (the product is exact, so this is
// the one rounding of the sum, exact here in any case).
template <int D, int END>
__device__ __forceinline__ void cross_lane(double (&x)[8], int lane) {
  if constexpr (D < END) {
    const double sg = (lane & D) ? -1.0 : 1.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fma(x[i], sg, partner<D>(x[i]));
    cross_lane<2 * D, END>(x, lane);
  }
}

// Fast Walsh-Hadamard transform within aligned blocks of BLOCK channels (Sylvester order:
// butterflies (x_j + x_{j+h}, x_j - x_{j+h}) for h = 1, 2, 4, ...), scaled by 1/sqrt(BLOCK).
// A thread holds 8 consecutive channels (h < 8 in registers); a block of BLOCK channels
// spans BLOCK/8 consecutive lanes of one wave (h >= 8 across lanes: DPP moves inside a
// row of 16 lanes, xor shuffles beyond).  The butterflies
// run in fp64, where they are exact (fp16 values are multiples of 2^-24 below 2^16, so a
// sum of up to 512 of them needs at most 49 significant bits); the scaling is the one
// rounding, and the fp16 result is the correctly rounded value of that.  In-place use is
// safe: every thread reads its 16 bytes before any write and writes only those.
template <int BLOCK>
__global__ __launch_bounds__(256) void k_hadamard(const uint16_t* __restrict__ A, long long chunks,
                                                  double scale, uint16_t* __restrict__ out) {
  const long long chunk = (long long)blockIdx.x * 256 + threadIdx.x;
  const bool ok = chunk < chunks;
  const int lane = threadIdx.x & 63;
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (ok) raw = *(const u32x4*)(A + chunk * 8);
  double x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = (double)h2f((uint16_t)(raw[j] & 0xffffu));
    x[2 * j + 1] = (double)h2f((uint16_t)(raw[j] >> 16));
  }
  constexpr int IN = BLOCK < 8 ? BLOCK : 8;
#pragma unroll
  for (int h = 1; h < IN; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0) {
        const double p = x[i], q = x[i + h];
        x[i] = p + q;
        x[i + h] = p - q;
      }
  cross_lane<1, BLOCK / 8>(x, lane);
  if (ok) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = (uint32_t)d2h_rn(x[2 * j] * scale) | ((uint32_t)d2h_rn(x[2 * j + 1] * scale) << 16);
    *(u32x4*)(out + chunk * 8) = r;
  }
}

template <int BLOCK>
hipError_t launch_h(const uint16_t* A, long long chunks, double scale, uint16_t* out,
                    hipStream_t stream) {
  const long long blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(k_hadamard<BLOCK>, dim3((unsigned)blocks), dim3(256), 0, stream, A, chunks,
                     scale, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_threshold_scales(const float* a, int K, double percentile, float factor,
                                   float* s_out, hipStream_t stream) {
  if (K <= 0) return hipSuccess;
  if (K > kMaxThresholdK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_threshold_scales, dim3(1), dim3(kSortThreads), 0, stream, a, K,
                     percentile, factor, s_out);
  return hipGetLastError();
}

hipError_t launch_hadamard(const uint16_t* A, int rows, int K, int block, uint16_t* out,
                           hipStream_t stream) {
  if (rows <= 0 || K <= 0) return hipSuccess;
  const long long chunks = (long long)rows * K / 8;
  const double scale = 1.0 / sqrt((double)block);
  switch (block) {
    case 2: return launch_h<2>(A, chunks, scale, out, stream);
    case 4: return launch_h<4>(A, chunks, scale, out, stream);
    case 8: return launch_h<8>(A, chunks, scale, out, stream);
    case 16: return launch_h<16>(A, chunks, scale, out, stream);
    case 32: return launch_h<32>(A, chunks, scale, out, stream);
    case 64: return launch_h<64>(A, chunks, scale, out, stream);
    case 128: return launch_h<128>(A, chunks, scale, out, stream);
    case 256: return launch_h<256>(A, chunks, scale, out, stream);
    case 512: return launch_h<512>(A, chunks, scale, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace awq
