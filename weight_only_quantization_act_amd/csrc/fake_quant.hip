// Scale family, fused scale -> quantise -> dequantise -> weight error, and final packing.
//
// Pages: "AWQ" scholia-log notes §4.1 (s_i = a_i^alpha), §2.2-§2.3 (quantise the scaled
// weight, divide back); "AWQ量化" tutorial 缩放保护 (W_hat = Q(s W) / s); kwkr.cn AWQ
// 技术解析 §1.2, §2.1, §4.2 (int4 codes with fp16 scales, two codes per byte).
//
// Layout of work: a block of 256 threads owns a stripe of column chunks and a few output
// rows.  The fake quantisation gives each lane 16 input channels of 8 rows (weights kept
// in registers and reused for every grid point); the pack gives each lane 8 channels
// (quantize8).  Either way a lane keeps its scales in registers, the per-element traffic
// is the fp16 weight read and the fp16 (or 4-bit) write as 16-byte coalesced accesses,
// and a group of g channels is g/16 (g/8) consecutive lanes.
#include <hip/hip_runtime.h>

#include "awq_act.h"
#include "awq_internal.h"
#include "quantizer.h"

#pragma clang fp contract(off)

namespace awq {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsFQ = 8;    // rows per block, fake quantisation
constexpr long long kFqSliceBelow = 256;    // fewer blocks than this: slice the grid points
constexpr long long kFqSmallTarget = 1024;  // blocks to aim for when slicing
// rows per block, packing (same-device sweep at 4096 x 4096: 14.4 us for 2 rows against 15.8
// for 8, 18.7 for 16; 1 and 4 rows in between; the same bytes out)
constexpr int kRowsPack = 2;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack8(const u32x4& r, float (&w)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[2 * j] = h2f((uint16_t)(r[j] & 0xffffu));
    w[2 * j + 1] = h2f((uint16_t)(r[j] >> 16));
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&x)[8]) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = (uint32_t)f2h(x[2 * j]) | ((uint32_t)f2h(x[2 * j + 1]) << 16);
  return r;
}

__global__ __launch_bounds__(kThreads) void k_make_scales(const float* __restrict__ a, int K,
                                                          AlphaList alphas,
                                                          float* __restrict__ s_table) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  const int k = blockIdx.y;
  if (i >= K) return;
  const float ai = a[i];
  // s = a^alpha in fp64, rounded to fp32; a channel with a == 0 keeps s = 1.
  const float s = (ai == 0.0f) ? 1.0f : (float)pow((double)ai, (double)alphas.v[k]);
  s_table[(size_t)k * K + i] = s;
}

// Cross-lane max / min over aligned groups of L lanes (2, 4 or 8) with DPP moves: a
// half-row mirror (i <-> 7 - i) leaves every group member's value in each quad, then quad
// swaps finish the reduction.
template <int L>
__device__ __forceinline__ float gmax_lanes(float x) {
  static_assert(L == 2 || L == 4 || L == 8, "group of 2, 4 or 8 lanes");
  if constexpr (L == 8) x = fmaxf(x, dpp_mov<kDppRowHalfMirror>(x));
  if constexpr (L >= 4) x = fmaxf(x, dpp_mov<kDppQuadXor2>(x));
  return fmaxf(x, dpp_mov<kDppQuadXor1>(x));
}
template <int L>
__device__ __forceinline__ float gmin_lanes(float x) {
  static_assert(L == 2 || L == 4 || L == 8, "group of 2, 4 or 8 lanes");
  if constexpr (L == 8) x = fminf(x, dpp_mov<kDppRowHalfMirror>(x));
  if constexpr (L >= 4) x = fminf(x, dpp_mov<kDppQuadXor2>(x));
  return fminf(x, dpp_mov<kDppQuadXor1>(x));
}

// dW_k = (v - Q(v)) / s for every grid point k, v = w s_k.  A lane owns 16 consecutive
// input channels (a group is g / 16 lanes) of kRowsFQ rows, keeps the rows' weights as
// fp16 pairs in registers and reuses them for every k; the next grid point's scales load
// during the current one.  The quantiser is the pack's (quantize8) in a leaner form: the
// code relative to the zero, c - z = clamp(rint(v / step), -z, top - z) (or
// +-qmax), comes from one med3; v / step is v * rcp(step) unless a quotient of the row (or
// -lo / step) lies within 2^-17 of a half-integer or is not finite, in which case the
// lane redoes the row with the correctly rounded divisions -- the same integers either way.
// The error v - (c - z) step is one fused multiply-add, multiplied by rcp(s) (the error
// only enters the fp16 loss product) and rounded once to fp16.
template <int LANES, bool ZP>
__global__ __launch_bounds__(kThreads) void k_fake_quant_delta(
    const uint16_t* __restrict__ W, const float* __restrict__ s_table, int M, int K, int nb,
    int w_bit, uint16_t* __restrict__ dW) {
  const int chunk = blockIdx.x * kThreads + threadIdx.x;
  const int col0 = chunk * 16;
  const bool col_ok = col0 < K;
  const int row0 = blockIdx.y * kRowsFQ;
  const int nrows = min(kRowsFQ, M - row0);

  uint32_t w[kRowsFQ][8];  // fp16 pairs (channel 2 i low, 2 i + 1 high)
#pragma unroll
  for (int r = 0; r < kRowsFQ; ++r) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (col_ok && r < nrows) {
      const u32x4* src = (const u32x4*)(W + (size_t)(row0 + r) * K + col0);
      a = src[0];
      b = src[1];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[r][q] = a[q];
      w[r][4 + q] = b[q];
    }
  }
  const float top = (float)((1 << w_bit) - 1);
  const float qmax = (float)((1 << (w_bit - 1)) - 1);
  // grid points [k_begin, k_end) of this block: blockIdx.z slices the grid points when the
  // layer alone gives fewer blocks than the chip has CUs
  const int per_z = (nb + (int)gridDim.z - 1) / (int)gridDim.z;
  const int k_begin = (int)blockIdx.z * per_z;
  const int k_end = min(nb, k_begin + per_z);
  float4 sn[4];
  auto load_s = [&](int k) {
    const float4* sp = (const float4*)(s_table + (size_t)k * K + col0);
#pragma unroll
    for (int q = 0; q < 4; ++q) sn[q] = col_ok ? sp[q] : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
  };
  load_s(k_begin);  // every slice has at least one grid point (see the launcher)

  for (int k = k_begin; k < k_end; ++k) {
    float s[16], is[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[4 * q] = sn[q].x;
      s[4 * q + 1] = sn[q].y;
      s[4 * q + 2] = sn[q].z;
      s[4 * q + 3] = sn[q].w;
    }
    if (k + 1 < k_end) load_s(k + 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) is[i] = __builtin_amdgcn_rcpf(s[i]);

    uint16_t* out = dW + (size_t)k * M * K;
#pragma unroll
    for (int r = 0; r < kRowsFQ; ++r) {
      if (r >= nrows) break;  // uniform across the block
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const _Float16 wh =
            __builtin_bit_cast(_Float16, (uint16_t)(w[r][i >> 1] >> (16 * (i & 1))));
        v[i] = fmaf((float)wh, s[i], 0.0f);  // = w s (a zero's sign is immaterial)
      }
      float hi = v[0], lo = v[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        hi = fmaxf(hi, v[i]);
        lo = fminf(lo, v[i]);
      }
      hi = gmax_lanes<LANES>(hi);
      lo = gmin_lanes<LANES>(lo);
      float st, clo, chi, lr = 0.0f;
      bool need;
      if constexpr (ZP) {
        const float hr = fmaxf(hi, 0.0f);
        lr = fminf(lo, 0.0f);
        st = (hr - lr) / top;
        if (st == 0.0f) st = 1.0f;
        const float tz = -lr * __builtin_amdgcn_rcpf(st);
        const float z = rintf(tz);
        need = !(fabsf(tz - z) < 0.5f - kTieBand);
        const float zc = __builtin_amdgcn_fmed3f(z, 0.0f, top);
        clo = -zc;
        chi = top - zc;
      } else {
        st = fmaxf(fabsf(hi), fabsf(lo)) / qmax;
        if (st == 0.0f) st = 1.0f;
        clo = -qmax;
        chi = qmax;
        need = false;
      }
      // a step below the smallest normal fp32 (or NaN) takes the divisions: the NaN-dropping
      // maximum below would not see the non-finite quotients of an infinite reciprocal
      need |= !(st >= kMinNormal);
      const float inv = __builtin_amdgcn_rcpf(st);
      float cz[16];
      float dist = 0.0f;  // the largest |t - rint t| of the row
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float t0 = v[i] * inv, t1 = v[i + 1] * inv;
        const float q0 = rintf(t0), q1 = rintf(t1);
        dist = fmaxf(dist, fmaxf(fabsf(t0 - q0), fabsf(t1 - q1)));
        cz[i] = __builtin_amdgcn_fmed3f(q0, clo, chi);
        cz[i + 1] = __builtin_amdgcn_fmed3f(q1, clo, chi);
      }
      need |= !(dist < 0.5f - kTieBand);
      if (need) {  // rare: the correctly rounded divisions
        if constexpr (ZP) {
          const float zc = __builtin_amdgcn_fmed3f(rintf(-lr / st), 0.0f, top);
          clo = -zc;
          chi = top - zc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) cz[i] = __builtin_amdgcn_fmed3f(rintf(v[i] / st), clo, chi);
      }
      if (col_ok) {
        uint32_t e[8];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const half2_t ep = {(_Float16)(fmaf(-cz[i], st, v[i]) * is[i]),
                              (_Float16)(fmaf(-cz[i + 1], st, v[i + 1]) * is[i + 1])};
          e[i >> 1] = __builtin_bit_cast(uint32_t, ep);
        }
        u32x4* dst = (u32x4*)(out + (size_t)(row0 + r) * K + col0);
        dst[0] = u32x4{e[0], e[1], e[2], e[3]};
        dst[1] = u32x4{e[4], e[5], e[6], e[7]};
      }
    }
  }
}

template <int LANES>
__global__ __launch_bounds__(kThreads) void k_quant_pack(
    const uint16_t* __restrict__ W, const float* __restrict__ s_in,
    const float* __restrict__ clip, int M, int K, int w_bit, int zero_point,
    uint8_t* __restrict__ codes_out, uint16_t* __restrict__ scales,
    uint16_t* __restrict__ zeros, int32_t* __restrict__ status) {
  const int chunk = blockIdx.x * kThreads + threadIdx.x;
  const int col0 = chunk * 8;
  const bool col_ok = col0 < K;
  const int row0 = blockIdx.y * kRowsPack;
  const int nrows = min(kRowsPack, M - row0);
  const bool zp = zero_point != 0;
  const int G = K / (LANES * 8);
  const int group = col0 / (LANES * 8);
  const bool leader = (threadIdx.x % LANES) == 0;

  float s[8];
  if (col_ok) {
    const float4* sp = (const float4*)(s_in + col0);
    const float4 s0 = sp[0], s1 = sp[1];
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 1.0f;
  }

  for (int r = 0; r < kRowsPack; ++r) {
    if (r >= nrows) break;  // uniform across the block
    const int row = row0 + r;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (col_ok) raw = *(const u32x4*)(W + (size_t)row * K + col0);
    float w[8], v[8], code[8], st, z;
    unpack8(raw, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = w[i] * s[i];
    const float ratio = (clip != nullptr && col_ok) ? clip[(size_t)row * G + group] : 1.0f;
    quantize8<LANES>(v, w_bit, zp, code, st, z, ratio);
    if (col_ok) {
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) packed |= ((uint32_t)code[i] & 0xfu) << (4 * i);
      *(uint32_t*)(codes_out + (size_t)row * (K / 2) + col0 / 2) = packed;
      if (leader) {
        const uint16_t sh = f2h(st);
        scales[(size_t)row * G + group] = sh;
        zeros[(size_t)row * G + group] = f2h(z);
        // every writer stores the same value, after the one-thread initialisation that
        // precedes this launch on the stream
        if (status != nullptr && (sh & 0x7c00u) == 0x7c00u) status[0] = AWQ_W_SCALE_OVERFLOW;
      }
    }
  }
}

__global__ void k_status_init(int32_t* __restrict__ status) { status[0] = AWQ_OK; }

}  // namespace

hipError_t launch_make_scales(const float* a, int K, const AlphaList& alphas, int n_alpha,
                              float* s_table, hipStream_t stream) {
  if (K <= 0 || n_alpha <= 0) return hipSuccess;
  dim3 grid((K + kThreads - 1) / kThreads, n_alpha);
  hipLaunchKernelGGL(k_make_scales, grid, dim3(kThreads), 0, stream, a, K, alphas, s_table);
  return hipGetLastError();
}

hipError_t launch_fake_quant_delta(const uint16_t* W, const float* s_table, int M, int K,
                                   int nb, int w_bit, int group_size, int zero_point,
                                   uint16_t* dW, hipStream_t stream) {
  if (M <= 0 || K <= 0 || nb <= 0) return hipSuccess;
  const int chunks = K / 16;
  dim3 grid((chunks + kThreads - 1) / kThreads, (M + kRowsFQ - 1) / kRowsFQ);
  // a small layer: slice the grid points over blockIdx.z (each slice re-reads its rows of
  // W), about kFqSmallTarget blocks in all; every slice gets at least one grid point
  const long long xy = (long long)grid.x * grid.y;
  if (xy < kFqSliceBelow) {
    long long nz = (kFqSmallTarget + xy - 1) / xy;
    if (nz > nb) nz = nb;
    const long long per = (nb + nz - 1) / nz;
    grid.z = (unsigned)((nb + per - 1) / per);
  }
#define AWQ_FQ(L)                                                                         \
  if (zero_point)                                                                         \
    hipLaunchKernelGGL((k_fake_quant_delta<L, true>), grid, dim3(kThreads), 0, stream, W,  \
                       s_table, M, K, nb, w_bit, dW);                                     \
  else                                                                                    \
    hipLaunchKernelGGL((k_fake_quant_delta<L, false>), grid, dim3(kThreads), 0, stream, W, \
                       s_table, M, K, nb, w_bit, dW)
  switch (group_size) {
    case 32: AWQ_FQ(2); break;
    case 64: AWQ_FQ(4); break;
    case 128: AWQ_FQ(8); break;
    default: return hipErrorInvalidValue;
  }
#undef AWQ_FQ
  return hipGetLastError();
}

hipError_t launch_quant_pack(const uint16_t* W, const float* s, const float* clip, int M,
                             int K, int w_bit, int group_size, int zero_point, uint8_t* codes,
                             uint16_t* scales, uint16_t* zeros, int32_t* status,
                             hipStream_t stream) {
  if (status) {
    hipLaunchKernelGGL(k_status_init, dim3(1), dim3(1), 0, stream, status);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (M <= 0 || K <= 0) return hipSuccess;
  const int chunks = K / 8;
  dim3 grid((chunks + kThreads - 1) / kThreads, (M + kRowsPack - 1) / kRowsPack);
  switch (group_size) {
    case 32:
      hipLaunchKernelGGL(k_quant_pack<4>, grid, dim3(kThreads), 0, stream, W, s, clip, M, K, w_bit,
                         zero_point, codes, scales, zeros, status);
      break;
    case 64:
      hipLaunchKernelGGL(k_quant_pack<8>, grid, dim3(kThreads), 0, stream, W, s, clip, M, K, w_bit,
                         zero_point, codes, scales, zeros, status);
      break;
    case 128:
      hipLaunchKernelGGL(k_quant_pack<16>, grid, dim3(kThreads), 0, stream, W, s, clip, M, K, w_bit,
                         zero_point, codes, scales, zeros, status);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace awq
