// Scale family, fused scale -> quantise -> dequantise -> weight error, and final packing.
//
// Pages: "AWQ" scholia-log notes §4.1 (s_i = a_i^alpha), §2.2-§2.3 (quantise the scaled
// weight, divide back); "AWQ量化" tutorial 缩放保护 (W_hat = Q(s W) / s); kwkr.cn AWQ
// 技术解析 §1.2, §2.1, §4.2 (int4 codes with fp16 scales, two codes per byte).
//
// Layout of work: a block of 256 threads owns a stripe of 256 column chunks (8 input
// channels each, 2048 channels) and ROWS consecutive output rows.  Each thread keeps its
// 8 scales (and their reciprocals) in registers and reuses them for all ROWS rows, so
// the per-element traffic is the fp16 weight read and the fp16 result write, both as
// 16-byte coalesced accesses.  Groups of g channels are g/8 consecutive lanes.
#include <hip/hip_runtime.h>

#include "awq_internal.h"
#include "quantizer.h"

#pragma clang fp contract(off)

namespace awq {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsFQ = 8;    // rows per block, fake quantisation
constexpr int kRowsPack = 8;  // rows per block, packing

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

template <int LANES>
__global__ __launch_bounds__(kThreads) void k_fake_quant_delta(
    const uint16_t* __restrict__ W, const float* __restrict__ s_table, int M, int K, int nb,
    int w_bit, int zero_point, uint16_t* __restrict__ dW) {
  const int chunk = blockIdx.x * kThreads + threadIdx.x;
  const int col0 = chunk * 8;
  const bool col_ok = col0 < K;
  const int row0 = blockIdx.y * kRowsFQ;
  const int nrows = min(kRowsFQ, M - row0);
  const bool zp = zero_point != 0;

  float w[kRowsFQ][8];
#pragma unroll
  for (int r = 0; r < kRowsFQ; ++r) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (col_ok && r < nrows) raw = *(const u32x4*)(W + (size_t)(row0 + r) * K + col0);
    unpack8(raw, w[r]);
  }

  for (int k = 0; k < nb; ++k) {
    float s[8], inv[8];
    if (col_ok) {
      const float4* sp = (const float4*)(s_table + (size_t)k * K + col0);
      const float4 s0 = sp[0], s1 = sp[1];
      s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
      s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = 1.0f;
    }
    // 1/s only enters the weight error fed to the fp16 loss product (not the codes), so
    // the hardware reciprocal (1 ulp) is accurate enough.
#pragma unroll
    for (int i = 0; i < 8; ++i) inv[i] = __builtin_amdgcn_rcpf(s[i]);

    uint16_t* out = dW + (size_t)k * M * K;
#pragma unroll
    for (int r = 0; r < kRowsFQ; ++r) {
      if (r >= nrows) break;  // uniform across the block
      float v[8], code[8], st, z;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = w[r][i] * s[i];
      quantize8<LANES>(v, w_bit, zp, code, st, z);
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = (code[i] - z) * st;   // quantised scaled weight
        e[i] = (v[i] - d) * inv[i];           // weight error, W - Q(W s)/s = (v - d)/s
      }
      if (col_ok) *(u32x4*)(out + (size_t)(row0 + r) * K + col0) = pack8(e);
    }
  }
}

template <int LANES>
__global__ __launch_bounds__(kThreads) void k_quant_pack(
    const uint16_t* __restrict__ W, const float* __restrict__ s_in,
    const float* __restrict__ clip, int M, int K, int w_bit, int zero_point,
    uint8_t* __restrict__ codes_out, uint16_t* __restrict__ scales,
    uint16_t* __restrict__ zeros) {
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
        scales[(size_t)row * G + group] = f2h(st);
        zeros[(size_t)row * G + group] = f2h(z);
      }
    }
  }
}

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
  const int chunks = K / 8;
  dim3 grid((chunks + kThreads - 1) / kThreads, (M + kRowsFQ - 1) / kRowsFQ);
  switch (group_size) {
    case 32:
      hipLaunchKernelGGL(k_fake_quant_delta<4>, grid, dim3(kThreads), 0, stream, W, s_table,
                         M, K, nb, w_bit, zero_point, dW);
      break;
    case 64:
      hipLaunchKernelGGL(k_fake_quant_delta<8>, grid, dim3(kThreads), 0, stream, W, s_table,
                         M, K, nb, w_bit, zero_point, dW);
      break;
    case 128:
      hipLaunchKernelGGL(k_fake_quant_delta<16>, grid, dim3(kThreads), 0, stream, W, s_table,
                         M, K, nb, w_bit, zero_point, dW);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_pack(const uint16_t* W, const float* s, const float* clip, int M,
                             int K, int w_bit, int group_size, int zero_point, uint8_t* codes,
                             uint16_t* scales, uint16_t* zeros, hipStream_t stream) {
  if (M <= 0 || K <= 0) return hipSuccess;
  const int chunks = K / 8;
  dim3 grid((chunks + kThreads - 1) / kThreads, (M + kRowsPack - 1) / kRowsPack);
  switch (group_size) {
    case 32:
      hipLaunchKernelGGL(k_quant_pack<4>, grid, dim3(kThreads), 0, stream, W, s, clip, M, K, w_bit,
                         zero_point, codes, scales, zeros);
      break;
    case 64:
      hipLaunchKernelGGL(k_quant_pack<8>, grid, dim3(kThreads), 0, stream, W, s, clip, M, K, w_bit,
                         zero_point, codes, scales, zeros);
      break;
    case 128:
      hipLaunchKernelGGL(k_quant_pack<16>, grid, dim3(kThreads), 0, stream, W, s, clip, M, K, w_bit,
                         zero_point, codes, scales, zeros);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace awq
