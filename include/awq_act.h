/*
 * awq_act.h -- C ABI of the MI355X (gfx950) library for AWQ's per-layer
 * activation-aware scale search and 4-bit packing.
 *
 * Pages this interface follows (title, site):
 *   [AWQ-notes]   "AWQ" -- lizn-zn.github.io scholia-log, inference-quantization notes
 *   [AWQ-tut]     "AWQ量化" tutorial -- aiqz.cc
 *   [AWQ-blog]    "AWQ量化技术解析：激活感知的权重量化革命" -- kwkr.cn
 *   [GPTQ-AWQ]    "大模型的开发应用（十八）：大模型量化：GPTQ与AWQ" -- ewbang.com
 *   [AutoAWQ-70B] "AWQ 量化全流程拆解：将 70B 大模型塞进单张消费级 GPU" -- lnrq.cn
 *
 * Layouts (all row-major, fp16 = IEEE binary16 stored as uint16):
 *   W   fp16 [out_features][in_features]      weight of one linear layer, M x K
 *   X   fp16 [n_tokens][in_features]          calibration activations, N x K (the
 *                                             pages' X, K x N, stored transposed)
 *   a   fp32 [in_features]                    per-channel mean |x|
 *   s   fp32 [in_features]                    per-channel scale
 *
 * Conventions shared by every entry point:
 *   - Array arguments are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or keeps them.  Scratch memory comes from a caller-provided
 *     workspace whose size the matching *_workspace_bytes query returns.
 *   - W, X, packed codes and dW pointers must be 16-byte aligned; other arrays 4-byte
 *     (8-byte for fp64).  in_features must be a multiple of group_size.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *     asynchronous: outputs are valid once the caller synchronises that stream.  No
 *     call synchronises the host.
 *   - Errors are return codes (awq_status); nothing throws across the ABI.  All
 *     argument checks run on the host before any launch; a failed check enqueues
 *     nothing.  AWQ_E_HIP reports a failed launch or HIP runtime call.  Before its first
 *     launch every entry point clears the calling thread's pending HIP error (as
 *     hipGetLastError does), so that an earlier, unrelated failed runtime call is not
 *     reported as its own.
 *   - Calls are thread-safe given distinct workspaces (no global mutable state other
 *     than the per-thread profiling hook below).
 *   - Sizes: M*K and N*K must stay below 2^31 elements.
 */
#ifndef AWQ_ACT_H
#define AWQ_ACT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantiser settings: AutoAWQ's quant_config keys w_bit, q_group_size, zero_point
 * [AutoAWQ-70B §三; GPTQ-AWQ §3 (key parameters)]. */
typedef struct awq_qconfig {
  int32_t w_bit;      /* 2, 3 or 4; codes always occupy a 4-bit slot              */
  int32_t group_size; /* 32, 64 or 128 consecutive input channels of one row      */
  int32_t zero_point; /* 0 = symmetric (offset-binary codes), 1 = zero-point      */
} awq_qconfig;

typedef enum awq_status {
  AWQ_OK = 0,
  AWQ_E_NULL = 1,       /* a required pointer is NULL                                */
  AWQ_E_SHAPE = 2,      /* negative/zero size where one is needed, K % g != 0, too big */
  AWQ_E_CONFIG = 3,     /* w_bit or group_size or zero_point out of range             */
  AWQ_E_ALPHA = 4,      /* n_alpha outside [1, AWQ_MAX_ALPHA] or an alpha outside [0,1] */
  AWQ_E_WORKSPACE = 5,  /* workspace NULL or smaller than required                    */
  AWQ_E_DEVICE = 6,     /* a pointer that must be device memory is not                */
  AWQ_E_HIP = 7,        /* a HIP runtime call or kernel launch failed                 */
  AWQ_W_NONFINITE = 8,  /* device status word only: no alpha gave a finite loss      */
  AWQ_E_ALIGN = 9,      /* a pointer is not aligned as required                       */
  AWQ_W_SCALE_OVERFLOW = 10 /* device status word only: a stored fp16 step is not finite */
} awq_status;

#define AWQ_MAX_ALPHA 64

/* Human-readable name of a status code (static storage; never NULL). */
const char* awq_status_str(int status);

/* ------------------------------------------------------------------------------------
 * A1  activation statistics: a_i = (1/N) * sum_t |X[t][i]|
 *     [AWQ-notes §1.2 (a_i = E|x_i|); AWQ-tut 激活感知 (mean absolute activation over
 *     the N calibration samples)].
 *   X          fp16 [n_tokens][in_features], device
 *   a_out      fp32 [in_features], device (written)
 *   workspace  device scratch of at least awq_act_stats_workspace_bytes(N, K) bytes
 * Sums are taken in fp64 in a fixed order (deterministic; exact for fp16 inputs while
 * partial sums stay below 2^29), divided by N in fp64, rounded to fp32.
 * n_tokens >= 1, in_features >= 0.
 * ---------------------------------------------------------------------------------- */
size_t awq_act_stats_workspace_bytes(int64_t n_tokens, int64_t in_features);
int awq_act_stats(const void* X, int64_t n_tokens, int64_t in_features, float* a_out,
                  void* workspace, size_t workspace_bytes, void* stream);

/* awq_act_stats for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and the
 * same result bit for bit, with the partial sums in a static device array of the library
 * (AWQ_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, held until the process
 * ends) instead of a workspace.  The array's address on the current device is looked up
 * on the first call there.  Shapes whose partials need more than the array holds
 * (awq_act_stats_workspace_bytes(N, K) > AWQ_NOALLOC_SCRATCH_BYTES; about 4 MiB suffices
 * for every in_features up to 10^6) return AWQ_E_WORKSPACE.  Every call on one GPU uses
 * that GPU's one array: calls that overlap on a GPU (other streams, other threads) race
 * and must be ordered by the caller.  Other arguments and errors as for awq_act_stats. */
#define AWQ_NOALLOC_SCRATCH_BYTES (8u << 20)
int awq_act_stats_noalloc(const void* X, int64_t n_tokens, int64_t in_features, float* a_out,
                          void* stream);

/* Other statistics (same workspace convention, sized by the _ex query):
 *   AWQ_STAT_MEAN_ABS   mean |x|                                     (as awq_act_stats)
 *   AWQ_STAT_MAX_ABS    max |x| over tokens [GPTQ-AWQ §3 二.2: s = (max|A|)^alpha]; exact
 *   AWQ_STAT_RMS_RATIO  mean|x| / sqrt(mean x^2) in fp64 [AWQ-blog §1.2 importance score];
 *                       0 for an all-zero channel; the fp64 sum of squares is not exact,
 *                       so results may differ from another summation order by 1 ulp
 *   AWQ_STAT_EMA_MEAN   e <- momentum*e + (1-momentum)*mean_batch|x| from e = 0 over
 *                       consecutive batches of batch_tokens tokens (the last may be short)
 *                       [AWQ-blog §2.1, momentum 0.9]; fp64, exact batch sums
 * batch_tokens and momentum (in [0,1)) are read only for AWQ_STAT_EMA_MEAN.  The page's
 * running max of max|x| over batches equals AWQ_STAT_MAX_ABS. */
enum { AWQ_STAT_MEAN_ABS = 0, AWQ_STAT_MAX_ABS = 1, AWQ_STAT_RMS_RATIO = 2, AWQ_STAT_EMA_MEAN = 3 };
size_t awq_act_stats_ex_workspace_bytes(int64_t n_tokens, int64_t in_features,
                                        int32_t statistic, int64_t batch_tokens);
int awq_act_stats_ex(const void* X, int64_t n_tokens, int64_t in_features, int32_t statistic,
                     int64_t batch_tokens, double momentum, float* a_out, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * A2-A5  scale search over an alpha grid
 *   For every alpha_k:  s_k = a^alpha_k (a_i == 0 -> 1)            [AWQ-notes §4.1]
 *                       dW_k = W - Q(W diag(s_k)) diag(s_k)^-1      [AWQ-tut 缩放保护]
 *                       losses[k] = || dW_k X^T ||_F^2               [AWQ-notes §1.1, §4.1]
 *   best = argmin over finite losses (first index on ties), s_out = s_best
 *   [AWQ-notes §4.1; GPTQ-AWQ §3 二 (objective and grid search of alpha in [0,1])].
 *   Q: per (row, group of group_size input channels), fp32 with one rounding per
 *   operation, round-half-to-even; symmetric step = max|v|/(2^(b-1)-1), zero-point
 *   step = (max(v,0) - min(v,0))/(2^b-1), z = rint(-min/step); a zero step becomes 1.
 *
 *   W           fp16 [out][in], device           X  fp16 [n_tokens][in], device
 *   a           fp32 [in], device (from awq_act_stats or the caller)
 *   alphas_host fp32 [n_alpha], HOST memory, each in [0,1]; copied during the call
 *   s_out       fp32 [in], device (written: s of the chosen alpha; all 1 if none)
 *   losses_out  fp64 [n_alpha], device (written)
 *   best_out    int32 [1], device (written: chosen index, or -1 if no finite loss)
 *   status_out  int32 [1], device (written: AWQ_OK or AWQ_W_NONFINITE); may be NULL
 *   workspace   device scratch; see awq_workspace_bytes.
 * Losses are computed with dW rounded to fp16 and an fp16 MFMA product with fp32
 * accumulation, reduced in fp64 in a fixed order (bitwise repeatable run to run).  When
 * the estimated cost favours it (roughly n_tokens >= in_features), the same quantity is
 * taken as sum_r dW_r G dW_r^T with G = X^T X [AWQ-notes §1.1]: G summed on the matrix
 * cores (fp32 over runs of at most 8192 tokens, the runs added in fp64 and rounded to
 * fp32); its off-diagonal entries, scaled by one power of two, enter an fp16 MFMA
 * product, its diagonal enters in fp32.
 * out_features >= 0, in_features >= 0 (multiple of group_size, at most 4194304),
 * n_tokens >= 1.
 * ---------------------------------------------------------------------------------- */

/* Workspace bytes for a search that processes `alpha_batch` grid points per pass
 * (alpha_batch > n_alpha means all n_alpha at once).  alpha_batch <= 0 lets the library
 * choose, for speed: all points at once, unless their fp16 dW (2 out_features
 * in_features bytes each) exceeds 192 MiB, the loss product has enough work per byte of
 * dW (in_features >= 2048 in the G form, n_tokens >= 2048 in the direct form) and at
 * least 4 points fit in 192 MiB.  Then a pass takes the largest
 * number b >= 4 of points that fit whose loss-product blocks fill at least 9/10 of
 * their last round on the 256 compute units (if no such b, all at once).  Each pass's
 * dW then stays in the device's 256 MB last-level cache between the fake quantisation
 * that writes it and the loss product that reads it (the 4096 x 4096 layer with 4096
 * tokens: 6 points a pass, 192 MiB instead of 640 MiB, 1.3% faster; results are
 * bit-identical whatever the batching).  Any workspace of at least
 * awq_workspace_bytes(..., 1) bytes is accepted; the search then runs as many grid points
 * per pass as fit.  Returns 0 for invalid arguments. */
size_t awq_workspace_bytes(int64_t out_features, int64_t in_features, int64_t n_tokens,
                           const awq_qconfig* cfg, int32_t n_alpha, int32_t alpha_batch);

/* Which form the search takes for these sizes: AWQ_LOSS_DIRECT (the product dW X^T) or
 * AWQ_LOSS_GRAM (sum_r dW_r G dW_r^T, G = X^T X formed once per call).  Both give the
 * losses defined above; the choice depends on the sizes only.  Returns -1 for sizes that
 * awq_workspace_bytes rejects (n_alpha outside 1 .. AWQ_MAX_ALPHA, negative sizes,
 * n_tokens < 1); group size and bit width do not enter. */
enum { AWQ_LOSS_DIRECT = 0, AWQ_LOSS_GRAM = 1 };
int awq_loss_form(int64_t out_features, int64_t in_features, int64_t n_tokens, int32_t n_alpha);

int awq_search_scales(const void* W, const void* X, const float* a,
                      int64_t out_features, int64_t in_features, int64_t n_tokens,
                      const awq_qconfig* cfg, const float* alphas_host, int32_t n_alpha,
                      float* s_out, double* losses_out, int32_t* best_out,
                      int32_t* status_out, void* workspace, size_t workspace_bytes,
                      void* stream);

/* The same search over an explicit table of candidate scale vectors instead of a^alpha
 * (e.g. fixed-factor protection scales, or scales built from another statistic).
 *   s_table     fp32 [n_cand][in], device, 16-byte aligned, every entry > 0 (not checked)
 *   n_cand      1 .. AWQ_MAX_ALPHA; other arguments as for awq_search_scales, and the
 *               workspace is sized by awq_workspace_bytes(..., n_cand, batch). */
int awq_search_scale_table(const void* W, const void* X, const float* s_table, int32_t n_cand,
                           int64_t out_features, int64_t in_features, int64_t n_tokens,
                           const awq_qconfig* cfg, float* s_out, double* losses_out,
                           int32_t* best_out, int32_t* status_out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Fixed-factor protection scales: s_i = factor if a_i is above the percentile threshold of
 * a, else 1 [AWQ-tut 显著识别 (indicator of channels above a high percentile, 70-90),
 * 缩放保护 (protect by a factor > 1), Python 演示 (70th percentile, factor 2)].  The
 * threshold interpolates linearly between order statistics at position
 * (percentile/100)(K-1), in fp64; the comparison is made in fp64.  NaN sorts last (as
 * +inf); +-inf sort at the ends.  s_out may be a itself.
 *   a fp32 [in], s_out fp32 [in] (device); 1 <= in <= 32768; percentile in [0, 100];
 *   factor finite and > 0. */
int awq_threshold_scales(const float* a, int64_t in_features, double percentile, float factor,
                         float* s_out, void* stream);

/* Blockwise Hadamard rotation along the input dimension: every row of A is multiplied by
 * the block-diagonal orthogonal matrix with blocks H_block / sqrt(block) (Sylvester order),
 * so (W R)(X R)^T = W X^T when W and X are both rotated [AWQ-notes §5.1 (rotation keeps the
 * product and spreads an outlier channel), §5.2 (fast structured rotation)].
 *   A, out fp16 [rows][in] (device, 16-byte aligned; out may equal A); block a power of
 *   two in [2, 512] dividing in; in a multiple of 8.  The butterflies run in fp64, where
 *   the +-1 sums of fp16 values are exact; the 1/sqrt(block) scaling is the one rounding,
 *   and each result is the nearest-even fp16 of that. */
int awq_hadamard_rotate(const void* A, int64_t rows, int64_t in_features, int32_t block,
                        void* out, void* stream);

/* ------------------------------------------------------------------------------------
 * Clip search after the scale search
 *   For every row m, group j and ratio rho_k of the grid: shrink the group's range of
 *   v = W diag(s) by rho_k (hi and lo, or max|v|, multiplied in fp32), quantise as
 *   awq_quantize_pack does (values beyond the range clamp), and score the group's own
 *   output error e = sum_t (sum_{i in j} d_i x_{t,i})^2 with d = W - Q(v) / s.  The
 *   chosen ratio is the first smallest finite e (ratio 1 when none is finite)
 *   [AWQ-notes closing note (the practical algorithm may add clipping), §2.3 (Q rounds
 *   and clips), §1.1 (output error = weight error times activations)].
 *   The GPU evaluates e = d^T (X_j^T X_j) d through the group Gram matrices: fp16
 *   products summed on the matrix cores in fp32 over runs of at most 256 tokens, the runs
 *   added in fp64; each group's matrix (divided by s_a s_b in fp64) is scaled by a power
 *   of two and stored as fp16 hi + lo.  d is split into fp16 hi + lo the same way, and
 *   the quadratic form takes three fp16 matrix-core passes (hi.hi, hi.lo, lo.hi) with
 *   fp32 accumulation.
 *   W fp16 [out][in], X fp16 [n_tokens][in] (16-byte aligned), s fp32 [in] (the chosen
 *   scales, e.g. awq_search_scales' s_out), all device
 *   ratios_host  fp32 [n_ratio], HOST memory, each in (0, 1]; n_ratio in [1, 64]
 *   clip_out     fp32 [out][in/group_size], device (written: chosen ratios)
 *   best_out     int32 [out][in/group_size] chosen indices (-1: none finite), or NULL
 *   errors_out   fp32 [n_ratio][out][in/group_size] every group error, or NULL
 *   workspace    device scratch of awq_clip_workspace_bytes(...) bytes, 256-byte aligned
 * ---------------------------------------------------------------------------------- */
size_t awq_clip_workspace_bytes(int64_t out_features, int64_t in_features, int64_t n_tokens,
                                const awq_qconfig* cfg);
int awq_clip_search(const void* W, const void* X, const float* s, int64_t out_features,
                    int64_t in_features, int64_t n_tokens, const awq_qconfig* cfg,
                    const float* ratios_host, int32_t n_ratio, float* clip_out,
                    int32_t* best_out, float* errors_out, void* workspace,
                    size_t workspace_bytes, void* stream);
/* awq_quantize_pack with every group's range shrunk by its ratio clip[row][group]
 * (fp32 [out][in/group_size], device, each in (0, 1]); ratio 1 everywhere gives
 * awq_quantize_pack's output bit for bit. */
int awq_quantize_pack_clipped(const void* W, const float* s, const float* clip,
                              int64_t out_features, int64_t in_features, const awq_qconfig* cfg,
                              uint8_t* codes_out, void* scales_out, void* zeros_out,
                              void* stream);

/* ------------------------------------------------------------------------------------
 * W4A16 product of a packed layer (the consumer of awq_quantize_pack's output)
 *   y[t][m] = sum_i (c[m][i] - z[m][g]) * step[m][g] * xt[t][i],   g = i / group_size,
 *   xt = x when s is NULL (S^-1 already folded into the preceding operation
 *   [AWQ-notes §4.3]), otherwise xt = fp16(fp32(x / s)) per element
 *   [AWQ-blog §1.2 (dequantised weight = int4 code x fp16 scale), §4.2 (dequantisation
 *   fused into the product); AutoAWQ-70B §四 (GEMV kernel for single requests)].
 *   x        fp16 [n_tokens][in], device, 16-byte aligned
 *   s        fp32 [in], device, 16-byte aligned, or NULL
 *   codes    u8 [out][in/2], scales and zeros fp16 [out][in/group_size], as written by
 *            awq_quantize_pack (zeros must hold integers in [0, 15]); codes 16-byte aligned
 *   cfg      only group_size is read (codes occupy 4-bit slots for every w_bit)
 *   y        fp16 [n_tokens][out], device (written)
 *   workspace  device, 16-byte aligned, or NULL; with s given and n_tokens >= 2, a
 *            workspace of at least awq_w4a16_workspace_bytes(n_tokens, in) bytes makes the
 *            call write xt there first (one elementwise pass) and multiply with the
 *            matrix-core kernel; NULL or 0 bytes keeps the vector kernel, which forms xt in
 *            registers.  Both give the same xt; the sums may differ in rounding order.
 *            Nonzero but smaller than needed: AWQ_E_WORKSPACE.  Owned by the caller; its
 *            contents after the call are unspecified.
 * fp32 accumulation in a fixed order (bitwise repeatable), rounded to fp16 once.
 * in_features <= 32768; n_tokens >= 0 (0 enqueues nothing); in_features = 0 gives y = 0.
 * ---------------------------------------------------------------------------------- */
int awq_w4a16_matmul(const void* x, const float* s, int64_t n_tokens, const void* codes,
                     const void* scales, const void* zeros, int64_t out_features,
                     int64_t in_features, const awq_qconfig* cfg, void* y, void* workspace,
                     size_t workspace_bytes, void* stream);
/* Bytes of workspace for awq_w4a16_matmul's fold of x / s: 2 n_tokens in_features rounded
 * up to 256, or 0 when the fold is never taken (n_tokens < 2, or shapes out of range). */
size_t awq_w4a16_workspace_bytes(int64_t n_tokens, int64_t in_features);

/* ------------------------------------------------------------------------------------
 * A3 alone: dW = W - Q(W diag(s)) diag(s)^-1 rounded to fp16, the operand the search's
 * loss product consumes [AWQ-tut 缩放保护 (W_hat = Q(s W)/s)].
 *   W fp16 [out][in], s fp32 [in], dW_out fp16 [out][in]; all device.
 * ---------------------------------------------------------------------------------- */
int awq_fake_quant_delta(const void* W, const float* s, int64_t out_features,
                         int64_t in_features, const awq_qconfig* cfg, void* dW_out,
                         void* stream);

/* ------------------------------------------------------------------------------------
 * A6  quantise W diag(s) and pack
 *   codes_out   uint8 [out][in/2]: two codes per byte, input channel 2j in the low
 *               nibble [AWQ-blog §4.2]; codes in [0, 2^w_bit - 1] (symmetric codes are
 *               offset by 2^(w_bit-1))
 *   scales_out  fp16 [out][in/group_size]: the fp32 step rounded to nearest-even fp16
 *               [AWQ-blog §1.2, §2.1 (int4 codes with an fp16 scale)]
 *   zeros_out   fp16 [out][in/group_size]: the integer zero point z (2^(w_bit-1) when
 *               symmetric) [AutoAWQ-70B §三 zero_point, §四 per-group metadata]
 * Dequantisation of the scaled weight is (code - z) * scale; the unscaled weight is
 * that divided by s, which the caller folds into the preceding operation
 * [AWQ-notes §4.3].  Codes are bit-identical to the oracle's for the same s.
 * ---------------------------------------------------------------------------------- */
int awq_quantize_pack(const void* W, const float* s, int64_t out_features,
                      int64_t in_features, const awq_qconfig* cfg, uint8_t* codes_out,
                      void* scales_out, void* zeros_out, void* stream);

/* awq_quantize_pack (clip == NULL) or awq_quantize_pack_clipped (clip given) with a device
 * status word: status_out (int32 [1], device) is written AWQ_W_SCALE_OVERFLOW when any
 * stored fp16 step is not finite, AWQ_OK otherwise.  The pages store the step as FP16
 * [AWQ-blog §2.1]; a group whose fp32 step is 65520 or more (the nearest-even fp16 of
 * which is infinity), or not finite, cannot be dequantised from that format.  Codes,
 * steps and zeros are written exactly as by the unchecked calls (such a step as fp16
 * infinity).  One extra one-thread launch initialises the word before the pack. */
int awq_quantize_pack_checked(const void* W, const float* s, const float* clip,
                              int64_t out_features, int64_t in_features,
                              const awq_qconfig* cfg, uint8_t* codes_out, void* scales_out,
                              void* zeros_out, int32_t* status_out, void* stream);

/* ------------------------------------------------------------------------------------
 * Profiling hook (per calling thread, one-shot): the next awq_search_scales (or
 * awq_search_scale_table) call on this thread records `gemm_start`/`gemm_stop`
 * (hipEvent_t) on its stream immediately before its first and after its last
 * loss-product launch, `fq_start`/`fq_stop` around its first fake-quantisation launch,
 * and `gram_start`/`gram_stop` around the two launches that form G = X^T X (only when
 * the search takes the G form).  Any of them may be NULL.  With the whole alpha grid in
 * one pass (a workspace of awq_workspace_bytes(..., n_alpha, n_alpha)), the loss and
 * fake-quantisation pairs each bracket exactly one kernel launch; with several passes
 * the loss pair also spans the later passes' fake quantisation (use the per-pass hook
 * below).  Returns AWQ_OK.
 * ---------------------------------------------------------------------------------- */
int awq_set_profile_events(void* gemm_start, void* gemm_stop, void* fq_start,
                           void* fq_stop, void* gram_start, void* gram_stop);

/* Per-pass profiling hook (per calling thread, one-shot, independent of the one above):
 * `events` holds 4 n_pass hipEvent_t handles (copied; the array need not outlive the
 * call).  The next search on this thread records, for each pass p < n_pass, events[4p]
 * and events[4p + 1] on its stream right before and after that pass's fake-quantisation
 * launch, and events[4p + 2] and events[4p + 3] right before and after its loss-product
 * launch; passes at or past n_pass record nothing.  NULL handles are skipped.  The
 * number of passes is ceil(n_alpha / b) for the b grid points a pass that the workspace
 * holds (see awq_workspace_bytes).  n_pass = 0 clears the hook.  Returns AWQ_OK,
 * AWQ_E_SHAPE for n_pass outside [0, AWQ_MAX_ALPHA], AWQ_E_NULL for a NULL array with
 * n_pass > 0. */
int awq_set_profile_pass_events(void* const* events, int32_t n_pass);

/* The same kind of one-shot per-thread hook for the statistics: the next awq_act_stats or
 * awq_act_stats_ex call on this thread (one that enqueues work) records `pass_start` and
 * `pass_stop` (hipEvent_t, either may be NULL) on its stream right before and after its
 * streaming pass over X, the first of its two launches.  Returns AWQ_OK. */
int awq_set_stats_profile_events(void* pass_start, void* pass_stop);

/* ------------------------------------------------------------------------------------
 * Measurement probes: this device's practical ceilings, for reporting the kernels above
 * beside the published peaks.  They are not part of the search, compute nothing useful,
 * and are enqueued on `stream` like every other call.
 *
 * awq_probe_mfma: `blocks` blocks of eight waves (two a SIMD), each wave issuing
 *   iters x 8 back-to-back v_mfma_f32_32x32x16_f16 (32768 flop each) on register operands.
 *   clocks_out, device uint64 [blocks][2] (written): per block, the shader-clock ticks and
 *   the 100 MHz real-time ticks of its loop, so clock = ticks[0] / ticks[1] x 100 MHz.
 * awq_probe_lds: the same geometry, each wave issuing iters x 16 conflict-free 16-byte LDS
 *   reads per lane (1 KiB a wave-read); same clocks_out.
 * awq_probe_read: one streaming read of `bytes` (a multiple of 16) at src (16-byte
 *   aligned device memory), 16-byte loads, each block over its own contiguous range.
 * awq_probe_write: one streaming write of `bytes` (a multiple of 16) to dst, 16-byte stores
 *   (the contents become fp16 ones).
 * awq_probe_copy: one streaming copy of `bytes` from src to dst (distinct buffers).
 * awq_probe_wall_clock_khz: host-side query of the frequency of the real-time counter
 *   (hipDeviceAttributeWallClockRate of `device`) into *khz_out (host int32).
 * blocks and iters in [1, 2^16] and [1, 2^20] with blocks x iters at most 2^28 (about a quarter
 * of a second of matrix-core work at the device's clock).  Errors: AWQ_E_NULL, AWQ_E_SHAPE,
 * AWQ_E_ALIGN, AWQ_E_DEVICE, AWQ_E_HIP, as for the other calls.
 * ---------------------------------------------------------------------------------- */
int awq_probe_mfma(int32_t blocks, int32_t iters, uint64_t* clocks_out, void* stream);
int awq_probe_lds(int32_t blocks, int32_t iters, uint64_t* clocks_out, void* stream);
int awq_probe_read(const void* src, int64_t bytes, void* stream);
int awq_probe_write(void* dst, int64_t bytes, void* stream);
int awq_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);
int awq_probe_wall_clock_khz(int32_t device, int32_t* khz_out);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_ACT_H */
