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
// rounded, rint = round half to even (v_rndne_f32), fp32 denormals kept.  The quotient
// v / step is evaluated through a reciprocal with an exact fallback near ties (see
// round_quotient), which provably yields the same integer.  That makes the codes
// bit-identical to any implementation that performs the same operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace awq {

// Cross-lane max/min inside aligned groups of LANES lanes (4, 8 or 16) with DPP moves.
// max and min are exact, so any pattern that lets every lane see every member of its
// group gives the same result: row_mirror (lane i <-> 15-i within 16), row_half_mirror
// (i <-> 7-i within 8), then quad swaps (i <-> i^1, i <-> i^2).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xf, 0xf, false));
}
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]

template <int LANES>
__device__ __forceinline__ float group_max(float x) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group of 4, 8 or 16 lanes");
  if constexpr (LANES == 16) x = fmaxf(x, dpp_mov<kDppRowMirror>(x));
  if constexpr (LANES >= 8) x = fmaxf(x, dpp_mov<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_mov<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_mov<kDppQuadXor2>(x));
  return x;
}

template <int LANES>
__device__ __forceinline__ float group_min(float x) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group of 4, 8 or 16 lanes");
  if constexpr (LANES == 16) x = fminf(x, dpp_mov<kDppRowMirror>(x));
  if constexpr (LANES >= 8) x = fminf(x, dpp_mov<kDppRowHalfMirror>(x));
  x = fminf(x, dpp_mov<kDppQuadXor1>(x));
  x = fminf(x, dpp_mov<kDppQuadXor2>(x));
  return x;
}

// rint(fl(v / st)) computed as rint(fl(v * inv)) with inv the hardware reciprocal of st
// (relative error <= 2^-23 for a normal st), except near a half-integer.  Only quotients
// with |v / st| <= 2^b can decide a code: every larger one (possible for a clipped group,
// whose range is shrunk before the step is taken) is clamped to the same end code
// whichever integer it rounds to, as is -min / st for the zero.  For |v / st| <= 16,
// fl(v * inv) is within 16 * 3 * 2^-24 and fl(v / st) within 16 * 2^-24 of the exact
// quotient, so the two are at most 2^-18 apart and round to the same integer unless the
// product lies within 2^-18 of a half-integer.  r = |t - rint(t)| and r - 0.5 are exact
// (Sterbenz), so the test is exact; lanes inside the band (about 1 in 10^5) and any
// non-finite case take the correctly rounded division.  A step below the smallest normal
// fp32 (where the reciprocal's error bound is not claimed) uses inv = +inf, which makes
// every quotient non-finite and so takes the division too.
constexpr float kTieBand = 7.62939453125e-06f;  // 2^-17, twice the bound above
constexpr float kMinNormal = 1.17549435e-38f;   // 2^-126

__device__ __forceinline__ float step_reciprocal(float st) {
  return st >= kMinNormal ? __builtin_amdgcn_rcpf(st) : __builtin_inff();
}

__device__ __forceinline__ bool near_half(float t, float q) {
  return !(fabsf(fabsf(t - q) - 0.5f) > kTieBand);
}

// The 8 quotients of a lane at once, so that the common case costs one branch per 8.
__device__ __forceinline__ void round_quotients(const float (&v)[8], float st, float inv,
                                                float (&q)[8]) {
  bool any_near = false;
  bool near[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = v[i] * inv;
    q[i] = rintf(t);
    near[i] = near_half(t, q[i]);
    any_near |= near[i];
  }
  if (any_near) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (near[i]) q[i] = rintf(v[i] / st);
  }
}

// Quantise the lane's 8 scaled values v[] of one group.  On return code[] holds the
// integer codes as floats (exact), and step/zero the group's parameters.  ratio (1 for no
// clipping) multiplies the group's range (hi and lo, or max|v|) before the step is taken;
// the clamps then clip the values beyond it.  Multiplying by 1 is exact, so ratio 1 is the
// plain quantiser bit for bit.
template <int LANES>
__device__ __forceinline__ void quantize8(const float (&v)[8], int w_bit, bool zero_point,
                                          float (&code)[8], float& step, float& zero,
                                          float ratio = 1.0f) {
  if (zero_point) {
    float hi = v[0], lo = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      hi = fmaxf(hi, v[i]);
      lo = fminf(lo, v[i]);
    }
    hi = fmaxf(group_max<LANES>(hi), 0.0f) * ratio;
    lo = fminf(group_min<LANES>(lo), 0.0f) * ratio;
    const float top = (float)((1 << w_bit) - 1);
    float st = (hi - lo) / top;
    if (st == 0.0f) st = 1.0f;
    const float inv = step_reciprocal(st);
    const float tz = -lo * inv;
    float z = rintf(tz);
    if (near_half(tz, z)) z = rintf(-lo / st);
    z = fminf(fmaxf(z, 0.0f), top);
    float q[8];
    round_quotients(v, st, inv, q);
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = fminf(fmaxf(q[i] + z, 0.0f), top);
    step = st;
    zero = z;
  } else {
    float m = fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = group_max<LANES>(m) * ratio;
    const float qmax = (float)((1 << (w_bit - 1)) - 1);
    const float off = (float)(1 << (w_bit - 1));
    float st = m / qmax;
    if (st == 0.0f) st = 1.0f;
    const float inv = step_reciprocal(st);
    float q[8];
    round_quotients(v, st, inv, q);
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = fminf(fmaxf(q[i], -qmax), qmax) + off;
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
