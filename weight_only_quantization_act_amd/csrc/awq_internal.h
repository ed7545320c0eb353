// Internal launchers shared between the HIP kernel files and the C-ABI layer.
// Every launcher enqueues on `stream` and returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace awq {

// ---- loss product tiling (also used by the host to size workspaces) ----------------
constexpr int kLossBM = 256;  // rows of dW per tile
constexpr int kLossBN = 256;  // tokens per tile

inline int64_t loss_tiles_m(int64_t M) { return (M + kLossBM - 1) / kLossBM; }
inline int64_t loss_tiles_n(int64_t N) { return (N + kLossBN - 1) / kLossBN; }
// The loss through G = X^T X (launch_gram_full + launch_loss_gemm_gram) instead of the
// direct product when it is estimated to take less time, for in_features up to 32768.
// Matrix-core work in flops: N K^2 for G's upper triangle, and per grid point
// M K^2 (1 + BN/K) over the block upper triangle of G, against the direct 2 M K N.  The
// Gram pass runs at about a third of the loss product's rate (its fp64 flushes and its
// re-reads of X), hence the weight kGramPassWeight; the triangular product loses a little
// to its uneven tiles, hence the ratio.
#ifndef AWQ_LOSS_GRAM_RATIO
#define AWQ_LOSS_GRAM_RATIO 0.85
#endif
constexpr double kGramPassWeight = 3.0;
inline bool loss_use_gram(int64_t M, int64_t K, int64_t N, int64_t n_alpha) {
  if (M <= 0 || K <= 0 || N <= 0 || K > 32768) return false;
  // the G pass reads X^T [K][N rounded up to 8] through 32-bit buffer offsets
  if ((double)K * (double)(N + 8) * 2.0 > 2147483648.0) return false;
  const double k2 = (double)K * (double)K;
  const double gram = kGramPassWeight * (double)N * k2 +
                      (double)M * k2 * (double)n_alpha * (1.0 + (double)kLossBN / (double)K);
  const double direct = 2.0 * (double)M * (double)K * (double)N * (double)n_alpha;
  return gram < AWQ_LOSS_GRAM_RATIO * direct;
}

// ---- statistics ----------------------------------------------------------------------
constexpr int kStatMeanAbs = 0;   // mean |x|
constexpr int kStatMaxAbs = 1;    // max |x|
constexpr int kStatRmsRatio = 2;  // mean |x| / sqrt(mean x^2)
constexpr int kStatEmaMean = 3;   // EMA of per-batch mean |x|
// Token splits of the two-pass reduction: batches of B tokens (B = N except for the
// EMA statistic), each cut into `sub` pieces of tpb tokens; nq fp64 partials per split.
struct StatsPlan {
  int B, n_batches, sub, tpb, splits, nq;
};
StatsPlan stats_plan(int64_t N, int64_t K, int mode, int64_t batch_tokens);
// ev0 / ev1 (nullable) are recorded on the stream right before and after the streaming
// pass over X (the first of the two launches).
hipError_t launch_act_stats(const uint16_t* X, int N, int K, int mode, const StatsPlan& plan,
                            double momentum, float* a_out, double* partials, hipStream_t stream,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// ---- scales, fake quantisation, packing ------------------------------------------------
constexpr int kMaxAlpha = 64;
struct AlphaList {
  float v[kMaxAlpha];
};
hipError_t launch_make_scales(const float* a, int K, const AlphaList& alphas, int n_alpha,
                              float* s_table, hipStream_t stream);
// dW[k] = fp16(W - Q(W s_k) / s_k) for k in [0, nb); dW stride M*K per k.
hipError_t launch_fake_quant_delta(const uint16_t* W, const float* s_table, int M, int K,
                                   int nb, int w_bit, int group_size, int zero_point,
                                   uint16_t* dW, hipStream_t stream);
// s_i = factor where a_i exceeds the linear-interpolation percentile of a, else 1.
constexpr int kMaxThresholdK = 32768;
hipError_t launch_threshold_scales(const float* a, int K, double percentile, float factor,
                                   float* s_out, hipStream_t stream);
// Rotate each row of A [rows][K] by blockwise normalised Hadamard matrices along K.
hipError_t launch_hadamard(const uint16_t* A, int rows, int K, int block, uint16_t* out,
                           hipStream_t stream);
// clip (nullable, fp32 [M][K/group_size]) shrinks each group's range by its ratio.
// status (nullable, device int32 [1]): set to AWQ_OK by a one-thread launch first, then
// AWQ_W_SCALE_OVERFLOW by the pack wherever a stored fp16 step is not finite.
hipError_t launch_quant_pack(const uint16_t* W, const float* s, const float* clip, int M,
                             int K, int w_bit, int group_size, int zero_point, uint8_t* codes,
                             uint16_t* scales, uint16_t* zeros, int32_t* status,
                             hipStream_t stream);

// ---- clip search ------------------------------------------------------------------------
constexpr int kMaxClip = 64;
struct ClipList {
  float v[kMaxClip];
};
// Scaled Gram matrices of the activation groups: G~[j] = S_j^-1 X_j^T X_j S_j^-1 with
// S_j = diag(s) over the group's channels (X_j^T X_j as fp32 matrix-core sums over at most
// 256 tokens, added in fp64 within a token split; split partials fp32 [splits][K/g][g][g]
// added in fp64 into G64 [K/g][g][g]), stored as G~[j] 2^-gexp[j] = Ghi + Glo with Ghi, Glo
// fp16 [K/g][g][g] and gexp int32 [K/g].  cmax: fp64 [K/g][gram_chunks(g)] per-chunk maxima.
int gram_splits(int64_t N, int64_t K, int group_size);
int gram_chunks(int group_size);
hipError_t launch_group_gram(const uint16_t* X, const float* s, int N, int K, int group_size,
                             float* partials, double* G64, double* cmax, uint16_t* Ghi,
                             uint16_t* Glo, int32_t* gexp, hipStream_t stream);
// Per (row, group): the group's own output error d^T G_j d for every ratio, the first
// smallest, its ratio (1 when none is finite); errors (nullable) fp32 [n][M][K/g].
// n_ratio <= 64.
hipError_t launch_clip_search(const uint16_t* W, const float* s, const uint16_t* Ghi,
                              const uint16_t* Glo, const int32_t* gexp, int M, int K, int w_bit,
                              int group_size, int zero_point, const ClipList& ratios,
                              int n_ratio, float* clip_out, int32_t* best_out, float* errors,
                              hipStream_t stream);

// ---- W4A16 product of a packed layer ----------------------------------------------------
constexpr int kGemvMaxT = 4;      // tokens per GEMV pass (more tokens run in passes)
constexpr int kGemvMaxK = 32768;  // one 32-channel code chunk per thread, 1024 threads
struct GemvPlan {
  int threads, rows;  // threads per block (K / 32 rounded up to waves), rows per block
};
GemvPlan w4a16_gemv_plan(int64_t M, int64_t K);
// Folded activations (s == null) and at least this many tokens take the matrix-core kernel.
#ifndef AWQ_W4A16_MFMA_MIN_T
#define AWQ_W4A16_MFMA_MIN_T 2
#endif
constexpr int kW4a16MfmaMinT = AWQ_W4A16_MFMA_MIN_T;
int w4a16_mfma_tiles(int64_t M);  // 16-row tiles per wave of the matrix-core kernel
int w4a16_mfma_waves(int64_t M, int64_t K, int group_size);
// y [T][M] fp16 = x~ [T][K] times the dequantised packed weights; s may be null.
hipError_t launch_w4a16_gemv(const uint8_t* codes, const uint16_t* scales,
                             const uint16_t* zeros, const uint16_t* x, const float* s, int T,
                             int M, int K, int group_size, uint16_t* y, hipStream_t stream);
// x~ [T][K] fp16 = fp16(fp32(x) / s) per element (K a multiple of 8).
hipError_t launch_fold_inverse_scales(const uint16_t* x, const float* s, int T, int K,
                                      uint16_t* out, hipStream_t stream);

// ---- loss product and selection ------------------------------------------------------
// partials[k * tiles + tm * tiles_n + tn] = sum over the tile of (dW_k X^T)^2.
hipError_t launch_loss_gemm(const uint16_t* dW, const uint16_t* X, int M, int N, int K,
                            int nb, double* partials, hipStream_t stream);
// The G form's Gram pass (loss_gram.hip): Xt = X^T (fp16 [K][ld]) | split partials of G's
// upper block triangle (fp32 [splits][pairs][kLossBM][kLossBN]) | their tile maxima
// tmax [splits][pairs] are scratch; outputs Gh = G' 2^-gexp (fp16 [K][K]; G with the
// kLossBN blocks above its diagonal doubled, the diagonal zero, the blocks below it not
// written), gdiag = diag(G) 2^-gexp (fp32 [K]) and gexp.  Tokens are split in runs of
// kchunk <= kGramSplitTokens (gram_split_tokens), each summed in fp32 on the matrix cores;
// K a multiple of 8.
constexpr int kGramSplitTokens = 8192;
struct GramPlan {
  int64_t ld, kchunk, splits, pairs, tmax;
};
int64_t gram_split_tokens(int64_t N, int64_t pairs);
GramPlan gram_plan(int64_t N, int64_t K);
hipError_t launch_gram_full(const uint16_t* X, int N, int K, uint16_t* Xt, float* part,
                            float* tmax, uint16_t* Gh, float* gdiag, int32_t* gexp,
                            hipStream_t stream);
// G build mode of the loss kernel (loss_gemm.hip): tiles tm <= tn of G over splits of
// kchunk tokens from Xt [K][ld]; out = the split partials, tmax [splits][pairs].
hipError_t launch_gram_build(const uint16_t* Xt, int N, int ld, int K, int kchunk, int splits,
                             float* out, float* tmax, hipStream_t stream);
// partials as launch_loss_gemm (loss_tiles_m(M) x loss_tiles_n(K) tiles per grid point),
// each the tile's share of sum_r dW_r G dW_r^T.
hipError_t launch_loss_gemm_gram(const uint16_t* dW, const uint16_t* Gh, const float* gdiag,
                                 const int32_t* gexp, int M, int K, int nb, double* partials,
                                 hipStream_t stream);
hipError_t launch_reduce_select(const double* partials, int n_alpha, int tiles,
                                const float* s_table, int K, double* losses, int32_t* best,
                                int32_t* status, float* s_out, hipStream_t stream);


// ---- measurement probes (this device's ceilings; not part of the search) -------------
// clocks: device [blocks][2] (shader-clock ticks, 100 MHz real-time ticks of each block's
// loop).  The stream probes use kProbeStreamBlocks blocks of 256 threads.
constexpr int kProbeStreamBlocks = 4096;
hipError_t launch_probe_mfma(int blocks, int iters, unsigned long long* clocks,
                             hipStream_t stream);
hipError_t launch_probe_lds(int blocks, int iters, unsigned long long* clocks,
                            hipStream_t stream);
hipError_t launch_probe_read(const void* src, long long bytes, hipStream_t stream);
hipError_t launch_probe_write(void* dst, long long bytes, hipStream_t stream);
hipError_t launch_probe_copy(const void* src, void* dst, long long bytes, hipStream_t stream);

}  // namespace awq
