// Output-error loss of each grid point:  L_k = || dW_k X^T ||_F^2  (fp16 MFMA, fp32
// accumulation, squared-sum epilogue, fp64 per-tile partials), and the argmin.
//
// Pages: "AWQ" scholia-log notes §1.1 (output error Delta Y = Delta W X) and §4.1
// (argmin of the squared Frobenius norm over the scale family); ewbang.com GPTQ与AWQ
// §3 二 (objective ||WX - Q(W s)(X/s)|| with a grid search over alpha in [0, 1]).
//
// dW_k is fp16 [M][K] and X is fp16 [N][K]: both operands are K-contiguous, so C = dW X^T
// is a "TN" product whose tiles stream straight from HBM.  The product itself is never
// stored: each 256 x 256 tile is squared and summed in registers.
//
// Tiling for CDNA4 (gfx950, wave64, 160 KiB LDS per CU):
//   block 256 threads = 4 waves in a 2 x 2 arrangement, tile 256 (dW rows) x 256 (tokens)
//   wave sub-tile 128 x 128 = 4 x 4 MFMA 32x32x16 f16 blocks, 256 fp32 accumulators/lane
//   K staged 64 at a time through a double-buffered LDS ring (2 x 64 KiB); global loads of
//   stage k+1 are issued before the MFMAs of stage k.  Rows of a stage are 128 bytes; the
//   16-byte chunk index is XOR-swizzled with (row & 7) so that the 8 lanes served per LDS
//   cycle read 8 distinct bank groups.
//   MFMA operand layout (32x32x16 f16): lane l supplies row (l mod 32) and channels
//   8*(l div 32) .. +7 of the 16-channel slice for A, and the same for B with tokens
//   in place of rows.  The loss only needs the sum of squares of the output tile, so the
//   accumulator layout never has to be decoded.
//   Block-to-tile map: hardware hands block b to XCD (b mod 8); blocks are renumbered so
//   each XCD walks a contiguous range of tiles, ordered in bands of 4 tile-rows, which
//   keeps the panels its 32 CUs share resident in that XCD's L2.
#include <hip/hip_runtime.h>

#include "awq_act.h"
#include "awq_internal.h"

namespace awq {

namespace {

constexpr int BM = kLossBM, BN = kLossBN, BK = kLossBK;
constexpr int kThreads = 256;
constexpr int kStageHalves = (BM + BN) * BK;          // 32768 halves = 64 KiB
constexpr int kLoadsA = BM * BK / 8 / kThreads;       // 16-byte chunks per thread, A
constexpr int kLoadsB = BN * BK / 8 / kThreads;       // same for B
constexpr int kBandM = 4;                              // tile-rows per raster band

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads, 1) void k_loss_gemm(
    const uint16_t* __restrict__ dW, const uint16_t* __restrict__ X, int M, int N, int K,
    int tiles_m, int tiles_n, int nb, double* __restrict__ partials) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kStageHalves];
  __shared__ double red[kThreads / 64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // ---- block -> (grid point, tile row, tile column), XCD-contiguous ----------------
  const int per_alpha = tiles_m * tiles_n;
  const int total = nb * per_alpha;
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int local = b >> 3;
  const int q = total >> 3, r = total & 7;
  const int logical = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  const int kk_alpha = logical / per_alpha;
  const int rem = logical - kk_alpha * per_alpha;
  const int band = rem / (kBandM * tiles_n);
  const int first_m = band * kBandM;
  const int band_rows = min(kBandM, tiles_m - first_m);
  const int in_band = rem - band * kBandM * tiles_n;
  const int tm = first_m + in_band % band_rows;
  const int tn = in_band / band_rows;

  const uint16_t* A = dW + (size_t)kk_alpha * M * K + (size_t)tm * BM * K;
  const uint16_t* B = X + (size_t)tn * BN * K;
  const int rows_a = min(BM, M - tm * BM);
  const int rows_b = min(BN, N - tn * BN);

  // ---- global -> register staging ----------------------------------------------------
  const int ld_row = tid >> 3;  // 0..31
  const int ld_kc = tid & 7;    // 16-byte chunk within a 64-channel stage row
  u32x4 ra[kLoadsA], rb[kLoadsB];

  auto gload = [&](int k0) {
    const int kc = k0 + ld_kc * 8;
    const bool k_ok = kc < K;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
      const int row = ld_row + 32 * j;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k_ok && row < rows_a) v = *(const u32x4*)(A + (size_t)row * K + kc);
      ra[j] = v;
    }
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j) {
      const int row = ld_row + 32 * j;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (k_ok && row < rows_b) v = *(const u32x4*)(B + (size_t)row * K + kc);
      rb[j] = v;
    }
  };
  auto sstore = [&](int stage) {
    uint16_t* sa = smem + stage * kStageHalves;
    uint16_t* sb = sa + BM * BK;
#pragma unroll
    for (int j = 0; j < kLoadsA; ++j) {
      const int row = ld_row + 32 * j;
      *(u32x4*)(sa + row * BK + ((ld_kc ^ (row & 7)) << 3)) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < kLoadsB; ++j) {
      const int row = ld_row + 32 * j;
      *(u32x4*)(sb + row * BK + ((ld_kc ^ (row & 7)) << 3)) = rb[j];
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  const int swz = frag_row & 7;  // (row & 7) for every fragment row of this lane

  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const uint16_t* sa = smem + cur * kStageHalves + (wm * 128 + frag_row) * BK;
    const uint16_t* sb = smem + cur * kStageHalves + BM * BK + (wn * 128 + frag_row) * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = ((2 * ks + frag_half) ^ swz) << 3;
      half8 af[4], bf[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) af[mi] = *(const half8*)(sa + mi * 32 * BK + chunk);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) bf[ni] = *(const half8*)(sb + ni * 32 * BK + chunk);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mi], bf[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: sum of squares of the 256 x 256 output tile -------------------------
  double ssum = 0.0;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      float t = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) t += acc[mi][ni][e] * acc[mi][ni][e];
      ssum += (double)t;
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ssum += __shfl_xor(ssum, off);
  if (lane == 0) red[wave] = ssum;
  __syncthreads();
  if (tid == 0)
    partials[(size_t)kk_alpha * per_alpha + (size_t)tm * tiles_n + tn] =
        (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void k_reduce_select(const double* __restrict__ partials,
                                                       int n_alpha, int tiles,
                                                       const float* __restrict__ s_table,
                                                       int K, double* __restrict__ losses,
                                                       int32_t* __restrict__ best_out,
                                                       int32_t* __restrict__ status_out,
                                                       float* __restrict__ s_out) {
  __shared__ double red[256];
  __shared__ double lsh[kMaxAlpha];
  __shared__ int best_sh;
  const int tid = threadIdx.x;
  for (int k = 0; k < n_alpha; ++k) {
    double acc = 0.0;
    for (int i = tid; i < tiles; i += 256) acc += partials[(size_t)k * tiles + i];
    red[tid] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    if (tid == 0) {
      lsh[k] = red[0];
      losses[k] = red[0];
    }
    __syncthreads();
  }
  if (tid == 0) {
    int best = -1;
    double bl = 0.0;
    for (int k = 0; k < n_alpha; ++k) {
      const double l = lsh[k];
      if (isfinite(l) && (best < 0 || l < bl)) {
        best = k;
        bl = l;
      }
    }
    best_sh = best;
    best_out[0] = best;
    if (status_out) status_out[0] = best < 0 ? AWQ_W_NONFINITE : AWQ_OK;
  }
  __syncthreads();
  const int best = best_sh;
  for (int i = tid; i < K; i += 256) s_out[i] = best >= 0 ? s_table[(size_t)best * K + i] : 1.0f;
}

}  // namespace

hipError_t launch_loss_gemm(const uint16_t* dW, const uint16_t* X, int M, int N, int K, int nb,
                            double* partials, hipStream_t stream) {
  if (M <= 0 || N <= 0 || nb <= 0) return hipSuccess;
  const int tm = (int)loss_tiles_m(M), tn = (int)loss_tiles_n(N);
  const long long blocks = (long long)nb * tm * tn;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_loss_gemm, dim3((unsigned)blocks), dim3(kThreads), 0, stream, dW, X, M, N,
                     K, tm, tn, nb, partials);
  return hipGetLastError();
}

hipError_t launch_reduce_select(const double* partials, int n_alpha, int tiles,
                                const float* s_table, int K, double* losses, int32_t* best,
                                int32_t* status, float* s_out, hipStream_t stream) {
  hipLaunchKernelGGL(k_reduce_select, dim3(1), dim3(256), 0, stream, partials, n_alpha, tiles,
                     s_table, K, losses, best, status, s_out);
  return hipGetLastError();
}

}  // namespace awq
