// Group quantiser of AWQ's scaled weight, device side (gfx950, wave64).
//
// One lane holds 8 consecutive input channels of one output row; a quantisation group
// of g channels is LANES = g/8 consecutive lanes of the same wave (16 for g = 128, 8 for
// g = 64, 4 for g = 32), always aligned to a multiple of LANES.  The group range is
// reduced across those lanes with xor shuffles that never leave the group.
//
// Arithmetic (pages: "AWQ" scholia-log notes §2.3 and §3.2; "AWQ量化" tutorial,
// 量化基础 and 缩放保护; kwkr.cn AWQ 技术解析 §2.1):
//   v = w * s                                    one fp32 rounding
//   symmetric:  step = max|v| / (2^(b-1) - 1);   q = clamp(rint(v / step), -qmax, qmax)
//               code = q + 2^(b-1), zero = 2^(b-1)
//   zero-point: hi = max(max v, 0), lo = min(min v, 0), step = (hi - lo) / (2^b - 1)
//               zero = clamp(rint(-lo / step), 0, 2^b - 1)
//               code = clamp(rint(v / step) + zero, 0, 2^b - 1)
//   a step of exactly 0 is replaced by 1 (the group is all zeros and stays zero)
//   dequantised scaled value d = (code - zero) * step        one fp32 rounding
// Every operation is a single IEEE fp32 operation: no contraction into FMA (the build
// uses -ffp-contract=off and this header turns it off again), divisions correctly
// rounded, rint = round half to even (v_rndne_f32), fp32 denormals kept.  That makes
// the codes bit-identical to any implementation that performs the same operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace awq {

template <int LANES>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

template <int LANES>
__device__ __forceinline__ float group_min(float x) {
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) x = fminf(x, __shfl_xor(x, m));
  return x;
}

// Quantise the lane's 8 scaled values v[] of one group.  On return code[] holds the
// integer codes as floats (exact), and step/zero the group's parameters.
template <int LANES>
__device__ __forceinline__ void quantize8(const float (&v)[8], int w_bit, bool zero_point,
                                          float (&code)[8], float& step, float& zero) {
  if (zero_point) {
    float hi = v[0], lo = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      hi = fmaxf(hi, v[i]);
      lo = fminf(lo, v[i]);
    }
    hi = fmaxf(group_max<LANES>(hi), 0.0f);
    lo = fminf(group_min<LANES>(lo), 0.0f);
    const float top = (float)((1 << w_bit) - 1);
    float st = (hi - lo) / top;
    if (st == 0.0f) st = 1.0f;
    float z = rintf(-lo / st);
    z = fminf(fmaxf(z, 0.0f), top);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = rintf(v[i] / st) + z;
      code[i] = fminf(fmaxf(q, 0.0f), top);
    }
    step = st;
    zero = z;
  } else {
    float m = fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = group_max<LANES>(m);
    const float qmax = (float)((1 << (w_bit - 1)) - 1);
    const float off = (float)(1 << (w_bit - 1));
    float st = m / qmax;
    if (st == 0.0f) st = 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = rintf(v[i] / st);
      q = fminf(fmaxf(q, -qmax), qmax);
      code[i] = q + off;
    }
    step = st;
    zero = off;
  }
}

// fp16 <-> fp32 helpers on raw uint16 storage (conversions are exact / RNE).
__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

}  // namespace awq
