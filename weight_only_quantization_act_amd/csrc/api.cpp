// C ABI of the AWQ scale-search library: argument checks, workspace carving, launches.
// Every check that can fail runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "awq_act.h"
#include "awq_internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxElems = (int64_t)1 << 31;  // M*K and N*K stay below 2^31

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool cfg_valid(const awq_qconfig* c) {
  if (!c) return false;
  if (c->w_bit < 2 || c->w_bit > 4) return false;
  if (c->group_size != 32 && c->group_size != 64 && c->group_size != 128) return false;
  if (c->zero_point != 0 && c->zero_point != 1) return false;
  return true;
}

// Shape check common to the weight-side calls.
int weight_shape(int64_t M, int64_t K, const awq_qconfig* cfg) {
  if (M < 0 || K < 0) return AWQ_E_SHAPE;
  if (K % cfg->group_size != 0) return AWQ_E_SHAPE;
  if (M >= kMaxElems || K >= kMaxElems || (K > 0 && M >= kMaxElems / K)) return AWQ_E_SHAPE;
  return AWQ_OK;
}

// The loss product addresses a 256-row panel of dW or X through 32-bit buffer offsets
// (at most 2^31 bytes), which bounds in_features for the search.
constexpr int64_t kMaxSearchK = (int64_t)1 << 22;

int token_shape(int64_t N, int64_t K) {
  if (N < 1 || K < 0) return AWQ_E_SHAPE;
  if (N >= kMaxElems || (K > 0 && N >= kMaxElems / K)) return AWQ_E_SHAPE;
  return AWQ_OK;
}

// A pointer the kernels dereference must be device (or managed) memory of HIP.
int device_ptr(const void* p) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return AWQ_E_DEVICE;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) return AWQ_OK;
  return AWQ_E_DEVICE;
}

// Workspace of the search: s table | loss partials | (Gram form: X^T, split partials of
// G's upper block triangle, fp16 G', fp32 diagonal, tile maxima, exponent) | dW batch.
struct SearchLayout {
  size_t s_off, p_off, dw_off;
  size_t xt_off, gpart_off, gh_off, gdiag_off, tmax_off, gexp_off;
  size_t dw_bytes_per_alpha;
  int64_t tiles;
  bool gram;
};

SearchLayout search_layout(int64_t M, int64_t K, int64_t N, int32_t n_alpha) {
  SearchLayout L;
  const bool work = (M > 0 && K > 0);
  L.gram = work && awq::loss_use_gram(M, K, N, n_alpha);
  L.tiles = work ? awq::loss_tiles_m(M) * awq::loss_tiles_n(L.gram ? K : N) : 0;
  L.s_off = 0;
  L.p_off = round_up((size_t)n_alpha * (size_t)K * sizeof(float), kAlign);
  size_t off = L.p_off + round_up((size_t)n_alpha * (size_t)L.tiles * sizeof(double), kAlign);
  L.xt_off = L.gpart_off = L.gh_off = L.gdiag_off = L.tmax_off = L.gexp_off = off;
  if (L.gram) {
    const size_t kk = (size_t)K * (size_t)K;
    const awq::GramPlan g = awq::gram_plan(N, K);
    L.xt_off = off;
    off += round_up((size_t)K * (size_t)g.ld * sizeof(uint16_t), kAlign);
    L.gpart_off = off;
    off += round_up((size_t)g.splits * (size_t)g.pairs * awq::kLossBM * awq::kLossBN * sizeof(float),
                    kAlign);
    L.gh_off = off;
    off += round_up(kk * sizeof(uint16_t), kAlign);
    L.gdiag_off = off;
    off += round_up((size_t)K * sizeof(float), kAlign);
    L.tmax_off = off;
    off += round_up((size_t)g.tmax * sizeof(float), kAlign);
    L.gexp_off = off;
    off += kAlign;
  }
  L.dw_off = off;
  L.dw_bytes_per_alpha = work ? (size_t)M * (size_t)K * 2 : 0;
  return L;
}

// Grid points per pass when the caller leaves the choice to the library (alpha_batch <= 0
// in awq_workspace_bytes).  A pass's dW is written by the fake quantisation and read back
// by the loss product; when it fits in three quarters of the device's 256 MB last-level
// cache, the loss product reads it from there (2-6% faster on the 4096^2 layer), but every
// extra pass re-reads W in its fake quantisation (10-14 us a pass on that layer).  Batching
// pays only when the loss product has enough work per byte of dW (in_features >= 2048 in
// the G form, n_tokens >= 2048 in the direct form), when at least 4 points fit, and when a
// pass's loss blocks fill at least 9/10 of their last generation on the compute units;
// otherwise the whole grid goes in one pass, as it does when all of dW fits the budget.
constexpr size_t kBatchDwBudget = (size_t)192 << 20;
constexpr int kMinBatch = 4;
constexpr int64_t kMinBatchWork = 2048;
constexpr int64_t kComputeUnits = 256;  // MI355X

int default_batch(int64_t M, int64_t K, int64_t N, int32_t n_alpha) {
  if (M <= 0 || K <= 0) return n_alpha;
  const size_t dw = (size_t)M * (size_t)K * 2;
  if ((size_t)n_alpha * dw <= kBatchDwBudget) return n_alpha;
  const int64_t fit = (int64_t)(kBatchDwBudget / dw);
  if (fit < kMinBatch) return n_alpha;
  const bool gram = awq::loss_use_gram(M, K, N, n_alpha);
  if ((gram ? K : N) < kMinBatchWork) return n_alpha;
  // loss-product blocks per grid point (the launchers' grids)
  const int64_t per_point = gram ? (awq::loss_tiles_m(K) + 1) / 2 * awq::loss_tiles_n(M)
                                 : awq::loss_tiles_m(M) * awq::loss_tiles_n(N);
  for (int64_t b = fit < n_alpha - 1 ? fit : n_alpha - 1; b >= kMinBatch; --b) {
    const int64_t blocks = b * per_point;
    const int64_t gens = (blocks + kComputeUnits - 1) / kComputeUnits;
    if (blocks * 10 >= gens * kComputeUnits * 9) return (int)b;
  }
  return n_alpha;
}

struct ProfileHook {
  void* gemm_start = nullptr;
  void* gemm_stop = nullptr;
  void* fq_start = nullptr;
  void* fq_stop = nullptr;
  void* gram_start = nullptr;
  void* gram_stop = nullptr;
};
thread_local ProfileHook g_hook;
// one-shot events around each pass of the next search (awq_set_profile_pass_events): for
// pass p, [4p] and [4p + 1] around its fake quantisation, [4p + 2] and [4p + 3] around its
// loss product
thread_local void* g_pass_ev[4 * AWQ_MAX_ALPHA];
thread_local int g_pass_n = 0;
// one-shot events around the statistics' streaming pass (awq_set_stats_profile_events)
thread_local void* g_stats_ev[2] = {nullptr, nullptr};

inline int hip_status(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_E_HIP; }

// The launchers report a failed launch through hipGetLastError, which would also return an
// error left pending by an earlier, unrelated runtime call of the calling thread (an event
// query that failed, say).  Every entry point clears that pending error before its first
// launch, so AWQ_E_HIP reports its own launches only.
inline void clear_pending_error() { (void)hipGetLastError(); }

inline int record(void* ev, hipStream_t st) {
  if (!ev) return AWQ_OK;
  return hip_status(hipEventRecord((hipEvent_t)ev, st));
}

// The search over nc candidate scale vectors s_table [nc][K] (device): fake quantisation,
// loss product and selection, in batches of as many candidates as the workspace holds.
// Arguments are already validated.  The workspace layout is the one awq_workspace_bytes
// describes (its s-table slot is unused when the caller supplies the table).
int run_search(const void* W, const void* X, const float* s_table, int64_t M, int64_t K,
               int64_t N, const awq_qconfig* cfg, int nc, float* s_out, double* losses_out,
               int32_t* best_out, int32_t* status_out, void* workspace, size_t workspace_bytes,
               void* stream) {
  ProfileHook hook = g_hook;
  g_hook = ProfileHook();
  const int n_pass_ev = g_pass_n;
  g_pass_n = 0;
  hipStream_t sm = (hipStream_t)stream;
  SearchLayout L = search_layout(M, K, N, nc);
  char* ws = (char*)workspace;
  double* partials = (double*)(ws + L.p_off);
  uint16_t* dW = (uint16_t*)(ws + L.dw_off);
  int batch = nc;
  if (L.dw_bytes_per_alpha > 0) {
    const size_t fit = (workspace_bytes - L.dw_off) / L.dw_bytes_per_alpha;
    if (fit < (size_t)batch) batch = (int)fit;
  }
  int st;
  if (L.tiles > 0) {
    uint16_t* Gh = (uint16_t*)(ws + L.gh_off);
    float* gdiag = (float*)(ws + L.gdiag_off);
    int32_t* gexp = (int32_t*)(ws + L.gexp_off);
    if (L.gram) {  // G = X^T X once, for every grid point
      if ((st = record(hook.gram_start, sm))) return st;
      st = hip_status(awq::launch_gram_full((const uint16_t*)X, (int)N, (int)K,
                                            (uint16_t*)(ws + L.xt_off),
                                            (float*)(ws + L.gpart_off),
                                            (float*)(ws + L.tmax_off), Gh, gdiag, gexp, sm));
      if (st) return st;
      if ((st = record(hook.gram_stop, sm))) return st;
    }
    for (int k0 = 0, pass = 0; k0 < nc; k0 += batch, ++pass) {
      const int nb = nc - k0 < batch ? nc - k0 : batch;
      const bool first = (k0 == 0);
      void* const* pev = pass < n_pass_ev ? g_pass_ev + 4 * pass : nullptr;
      if (first && (st = record(hook.fq_start, sm))) return st;
      if (pev && (st = record(pev[0], sm))) return st;
      st = hip_status(awq::launch_fake_quant_delta((const uint16_t*)W, s_table + (size_t)k0 * K,
                                                   (int)M, (int)K, nb, cfg->w_bit,
                                                   cfg->group_size, cfg->zero_point, dW, sm));
      if (st) return st;
      if (pev && (st = record(pev[1], sm))) return st;
      if (first && (st = record(hook.fq_stop, sm))) return st;
      if (first && (st = record(hook.gemm_start, sm))) return st;
      if (pev && (st = record(pev[2], sm))) return st;
      if (L.gram)
        st = hip_status(awq::launch_loss_gemm_gram(dW, Gh, gdiag, gexp, (int)M, (int)K, nb,
                                                   partials + (size_t)k0 * L.tiles, sm));
      else
        st = hip_status(awq::launch_loss_gemm(dW, (const uint16_t*)X, (int)M, (int)N, (int)K,
                                              nb, partials + (size_t)k0 * L.tiles, sm));
      if (st) return st;
      if (pev && (st = record(pev[3], sm))) return st;
    }
    if ((st = record(hook.gemm_stop, sm))) return st;
  }
  return hip_status(awq::launch_reduce_select(partials, nc, (int)L.tiles, s_table, (int)K,
                                              losses_out, best_out, status_out, s_out, sm));
}

}  // namespace

extern "C" {

const char* awq_status_str(int status) {
  switch (status) {
    case AWQ_OK: return "AWQ_OK";
    case AWQ_E_NULL: return "AWQ_E_NULL: a required pointer is NULL";
    case AWQ_E_SHAPE: return "AWQ_E_SHAPE: invalid or unsupported sizes";
    case AWQ_E_CONFIG: return "AWQ_E_CONFIG: w_bit, group_size or zero_point out of range";
    case AWQ_E_ALPHA: return "AWQ_E_ALPHA: n_alpha or an alpha value out of range";
    case AWQ_E_WORKSPACE: return "AWQ_E_WORKSPACE: workspace missing or too small";
    case AWQ_E_DEVICE: return "AWQ_E_DEVICE: pointer is not HIP device memory";
    case AWQ_E_HIP: return "AWQ_E_HIP: HIP runtime call or kernel launch failed";
    case AWQ_W_NONFINITE: return "AWQ_W_NONFINITE: no grid point gave a finite loss";
    case AWQ_E_ALIGN: return "AWQ_E_ALIGN: pointer not aligned as required";
    case AWQ_W_SCALE_OVERFLOW:
      return "AWQ_W_SCALE_OVERFLOW: a stored fp16 step is not finite (fp32 step >= 65520)";
    default: return "AWQ: unknown status";
  }
}

size_t awq_act_stats_ex_workspace_bytes(int64_t n_tokens, int64_t in_features,
                                        int32_t statistic, int64_t batch_tokens) {
  if (token_shape(n_tokens, in_features) != AWQ_OK) return 0;
  if (statistic < AWQ_STAT_MEAN_ABS || statistic > AWQ_STAT_EMA_MEAN) return 0;
  if (statistic == AWQ_STAT_EMA_MEAN && batch_tokens < 1) return 0;
  const awq::StatsPlan p = awq::stats_plan(n_tokens, in_features, statistic, batch_tokens);
  return round_up((size_t)p.nq * (size_t)p.splits * (size_t)in_features * sizeof(double),
                  kAlign) + kAlign;
}

size_t awq_act_stats_workspace_bytes(int64_t n_tokens, int64_t in_features) {
  return awq_act_stats_ex_workspace_bytes(n_tokens, in_features, AWQ_STAT_MEAN_ABS, 0);
}

int awq_act_stats_ex(const void* X, int64_t n_tokens, int64_t in_features, int32_t statistic,
                     int64_t batch_tokens, double momentum, float* a_out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!X || !a_out) return AWQ_E_NULL;
  if (!workspace) return AWQ_E_WORKSPACE;
  int st = token_shape(n_tokens, in_features);
  if (st != AWQ_OK) return st;
  if (statistic < AWQ_STAT_MEAN_ABS || statistic > AWQ_STAT_EMA_MEAN) return AWQ_E_CONFIG;
  if (statistic == AWQ_STAT_EMA_MEAN) {
    if (batch_tokens < 1 || batch_tokens >= kMaxElems) return AWQ_E_SHAPE;
    if (!(momentum >= 0.0 && momentum < 1.0)) return AWQ_E_CONFIG;
  }
  if (workspace_bytes <
      awq_act_stats_ex_workspace_bytes(n_tokens, in_features, statistic, batch_tokens))
    return AWQ_E_WORKSPACE;
  if (!aligned(X, in_features % 8 == 0 ? 16 : 2) || !aligned(a_out, 4) || !aligned(workspace, 8))
    return AWQ_E_ALIGN;
  if (in_features == 0) return AWQ_OK;
  if ((st = device_ptr(X)) || (st = device_ptr(a_out)) || (st = device_ptr(workspace))) return st;
  clear_pending_error();
  const awq::StatsPlan p = awq::stats_plan(n_tokens, in_features, statistic, batch_tokens);
  hipEvent_t ev0 = (hipEvent_t)g_stats_ev[0], ev1 = (hipEvent_t)g_stats_ev[1];
  g_stats_ev[0] = g_stats_ev[1] = nullptr;
  return hip_status(awq::launch_act_stats((const uint16_t*)X, (int)n_tokens, (int)in_features,
                                          statistic, p, momentum, a_out, (double*)workspace,
                                          (hipStream_t)stream, ev0, ev1));
}

int awq_act_stats(const void* X, int64_t n_tokens, int64_t in_features, float* a_out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return awq_act_stats_ex(X, n_tokens, in_features, AWQ_STAT_MEAN_ABS, 0, 0.0, a_out, workspace,
                          workspace_bytes, stream);
}

size_t awq_workspace_bytes(int64_t out_features, int64_t in_features, int64_t n_tokens,
                           const awq_qconfig* cfg, int32_t n_alpha, int32_t alpha_batch) {
  if (!cfg_valid(cfg)) return 0;
  if (weight_shape(out_features, in_features, cfg) != AWQ_OK) return 0;
  if (token_shape(n_tokens, in_features) != AWQ_OK) return 0;
  if (in_features > kMaxSearchK) return 0;
  if (n_alpha < 1 || n_alpha > AWQ_MAX_ALPHA) return 0;
  if (alpha_batch <= 0) alpha_batch = default_batch(out_features, in_features, n_tokens, n_alpha);
  if (alpha_batch > n_alpha) alpha_batch = n_alpha;
  SearchLayout L = search_layout(out_features, in_features, n_tokens, n_alpha);
  return L.dw_off + (size_t)alpha_batch * L.dw_bytes_per_alpha;
}

int awq_loss_form(int64_t out_features, int64_t in_features, int64_t n_tokens, int32_t n_alpha) {
  if (out_features < 0 || in_features < 0 || in_features > kMaxSearchK ||
      token_shape(n_tokens, in_features) != AWQ_OK)
    return -1;
  if (n_alpha < 1 || n_alpha > AWQ_MAX_ALPHA) return -1;
  return search_layout(out_features, in_features, n_tokens, n_alpha).gram ? AWQ_LOSS_GRAM
                                                                           : AWQ_LOSS_DIRECT;
}

int awq_search_scales(const void* W, const void* X, const float* a, int64_t out_features,
                      int64_t in_features, int64_t n_tokens, const awq_qconfig* cfg,
                      const float* alphas_host, int32_t n_alpha, float* s_out,
                      double* losses_out, int32_t* best_out, int32_t* status_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t M = out_features, K = in_features, N = n_tokens;
  if (!W || !X || !a || !cfg || !alphas_host || !s_out || !losses_out || !best_out)
    return AWQ_E_NULL;
  if (!workspace) return AWQ_E_WORKSPACE;
  if (!cfg_valid(cfg)) return AWQ_E_CONFIG;
  int st = weight_shape(M, K, cfg);
  if (st != AWQ_OK) return st;
  if ((st = token_shape(N, K)) != AWQ_OK) return st;
  if (K > kMaxSearchK) return AWQ_E_SHAPE;
  if (n_alpha < 1 || n_alpha > AWQ_MAX_ALPHA) return AWQ_E_ALPHA;
  awq::AlphaList al;
  memset(&al, 0, sizeof(al));
  for (int k = 0; k < n_alpha; ++k) {
    const float v = alphas_host[k];
    if (!(v >= 0.0f && v <= 1.0f)) return AWQ_E_ALPHA;  // also rejects NaN
    al.v[k] = v;
  }
  const size_t need_min = awq_workspace_bytes(M, K, N, cfg, n_alpha, 1);
  if (workspace_bytes < need_min) return AWQ_E_WORKSPACE;
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(a, 4) || !aligned(s_out, 4) ||
      !aligned(losses_out, 8) || !aligned(best_out, 4) || !aligned(status_out, 4) ||
      !aligned(workspace, kAlign))
    return AWQ_E_ALIGN;
  if ((st = device_ptr(W)) || (st = device_ptr(X)) || (st = device_ptr(a)) ||
      (st = device_ptr(s_out)) || (st = device_ptr(losses_out)) || (st = device_ptr(best_out)) ||
      (st = device_ptr(workspace)))
    return st;
  if (status_out && (st = device_ptr(status_out))) return st;

  clear_pending_error();
  if ((st = hip_status(awq::launch_make_scales(a, (int)K, al, n_alpha,
                                               (float*)workspace, (hipStream_t)stream))))
    return st;
  return run_search(W, X, (const float*)workspace, M, K, N, cfg, n_alpha, s_out, losses_out,
                    best_out, status_out, workspace, workspace_bytes, stream);
}

int awq_search_scale_table(const void* W, const void* X, const float* s_table, int32_t n_cand,
                           int64_t out_features, int64_t in_features, int64_t n_tokens,
                           const awq_qconfig* cfg, float* s_out, double* losses_out,
                           int32_t* best_out, int32_t* status_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const int64_t M = out_features, K = in_features, N = n_tokens;
  if (!W || !X || !s_table || !cfg || !s_out || !losses_out || !best_out) return AWQ_E_NULL;
  if (!workspace) return AWQ_E_WORKSPACE;
  if (!cfg_valid(cfg)) return AWQ_E_CONFIG;
  int st = weight_shape(M, K, cfg);
  if (st != AWQ_OK) return st;
  if ((st = token_shape(N, K)) != AWQ_OK) return st;
  if (K > kMaxSearchK) return AWQ_E_SHAPE;
  if (n_cand < 1 || n_cand > AWQ_MAX_ALPHA) return AWQ_E_ALPHA;
  if (K > 0 && (int64_t)n_cand * K >= kMaxElems) return AWQ_E_SHAPE;
  if (workspace_bytes < awq_workspace_bytes(M, K, N, cfg, n_cand, 1)) return AWQ_E_WORKSPACE;
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(s_table, 16) || !aligned(s_out, 4) ||
      !aligned(losses_out, 8) || !aligned(best_out, 4) || !aligned(status_out, 4) ||
      !aligned(workspace, kAlign))
    return AWQ_E_ALIGN;
  if ((st = device_ptr(W)) || (st = device_ptr(X)) || (st = device_ptr(s_table)) ||
      (st = device_ptr(s_out)) || (st = device_ptr(losses_out)) || (st = device_ptr(best_out)) ||
      (st = device_ptr(workspace)))
    return st;
  if (status_out && (st = device_ptr(status_out))) return st;
  clear_pending_error();
  return run_search(W, X, s_table, M, K, N, cfg, n_cand, s_out, losses_out, best_out, status_out,
                    workspace, workspace_bytes, stream);
}

int awq_threshold_scales(const float* a, int64_t in_features, double percentile, float factor,
                         float* s_out, void* stream) {
  if (!a || !s_out) return AWQ_E_NULL;
  if (in_features < 1 || in_features > awq::kMaxThresholdK) return AWQ_E_SHAPE;
  if (!(percentile >= 0.0 && percentile <= 100.0)) return AWQ_E_CONFIG;
  if (!(factor > 0.0f) || !isfinite(factor)) return AWQ_E_CONFIG;
  if (!aligned(a, 4) || !aligned(s_out, 4)) return AWQ_E_ALIGN;
  int st;
  if ((st = device_ptr(a)) || (st = device_ptr(s_out))) return st;
  clear_pending_error();
  return hip_status(awq::launch_threshold_scales(a, (int)in_features, percentile, factor, s_out,
                                                 (hipStream_t)stream));
}

int awq_hadamard_rotate(const void* A, int64_t rows, int64_t in_features, int32_t block,
                        void* out, void* stream) {
  if (!A || !out) return AWQ_E_NULL;
  if (block < 2 || block > 512 || (block & (block - 1))) return AWQ_E_CONFIG;
  if (rows < 0 || in_features < 0 || in_features % block || in_features % 8) return AWQ_E_SHAPE;
  if (rows >= kMaxElems || (in_features > 0 && rows >= kMaxElems / in_features))
    return AWQ_E_SHAPE;
  if (!aligned(A, 16) || !aligned(out, 16)) return AWQ_E_ALIGN;
  if (rows == 0 || in_features == 0) return AWQ_OK;
  int st;
  if ((st = device_ptr(A)) || (st = device_ptr(out))) return st;
  clear_pending_error();
  return hip_status(awq::launch_hadamard((const uint16_t*)A, (int)rows, (int)in_features, block,
                                         (uint16_t*)out, (hipStream_t)stream));
}

size_t awq_w4a16_workspace_bytes(int64_t n_tokens, int64_t in_features) {
  if (n_tokens < awq::kW4a16MfmaMinT || in_features <= 0 || in_features > awq::kGemvMaxK ||
      n_tokens >= kMaxElems / in_features)
    return 0;
  return round_up((size_t)n_tokens * (size_t)in_features * sizeof(uint16_t), kAlign);
}

int awq_w4a16_matmul(const void* x, const float* s, int64_t n_tokens, const void* codes,
                     const void* scales, const void* zeros, int64_t out_features,
                     int64_t in_features, const awq_qconfig* cfg, void* y, void* workspace,
                     size_t workspace_bytes, void* stream) {
  const int64_t T = n_tokens, M = out_features, K = in_features;
  if (!x || !codes || !scales || !zeros || !cfg || !y) return AWQ_E_NULL;
  if (!cfg_valid(cfg)) return AWQ_E_CONFIG;
  int st = weight_shape(M, K, cfg);
  if (st != AWQ_OK) return st;
  if (T < 0 || T >= kMaxElems || (K > 0 && T >= kMaxElems / K) ||
      (M > 0 && T >= kMaxElems / M))
    return AWQ_E_SHAPE;
  if (K > awq::kGemvMaxK) return AWQ_E_SHAPE;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 2) ||
      !aligned(y, 2) || (s && !aligned(s, 16)) || !aligned(workspace, 16))
    return AWQ_E_ALIGN;
  // the fold into the workspace is taken only when it helps: s given, several tokens
  const bool fold = s && workspace && workspace_bytes > 0 && T >= awq::kW4a16MfmaMinT && K > 0;
  if (fold && workspace_bytes < awq_w4a16_workspace_bytes(T, K)) return AWQ_E_WORKSPACE;
  if (T == 0 || M == 0) return AWQ_OK;
  if ((st = device_ptr(x)) || (st = device_ptr(codes)) || (st = device_ptr(scales)) ||
      (st = device_ptr(zeros)) || (st = device_ptr(y)))
    return st;
  if (s && (st = device_ptr(s))) return st;
  clear_pending_error();
  if (fold) {
    if ((st = device_ptr(workspace))) return st;
    uint16_t* xt = (uint16_t*)workspace;
    if ((st = hip_status(awq::launch_fold_inverse_scales((const uint16_t*)x, s, (int)T, (int)K,
                                                         xt, (hipStream_t)stream))))
      return st;
    return hip_status(awq::launch_w4a16_gemv((const uint8_t*)codes, (const uint16_t*)scales,
                                             (const uint16_t*)zeros, xt, nullptr, (int)T,
                                             (int)M, (int)K, cfg->group_size, (uint16_t*)y,
                                             (hipStream_t)stream));
  }
  return hip_status(awq::launch_w4a16_gemv((const uint8_t*)codes, (const uint16_t*)scales,
                                           (const uint16_t*)zeros, (const uint16_t*)x, s,
                                           (int)T, (int)M, (int)K, cfg->group_size,
                                           (uint16_t*)y, (hipStream_t)stream));
}

int awq_fake_quant_delta(const void* W, const float* s, int64_t out_features,
                         int64_t in_features, const awq_qconfig* cfg, void* dW_out,
                         void* stream) {
  if (!W || !s || !cfg || !dW_out) return AWQ_E_NULL;
  if (!cfg_valid(cfg)) return AWQ_E_CONFIG;
  int st = weight_shape(out_features, in_features, cfg);
  if (st != AWQ_OK) return st;
  if (!aligned(W, 16) || !aligned(s, 16) || !aligned(dW_out, 16)) return AWQ_E_ALIGN;
  if (out_features == 0 || in_features == 0) return AWQ_OK;
  if ((st = device_ptr(W)) || (st = device_ptr(s)) || (st = device_ptr(dW_out))) return st;
  clear_pending_error();
  return hip_status(awq::launch_fake_quant_delta(
      (const uint16_t*)W, s, (int)out_features, (int)in_features, 1, cfg->w_bit,
      cfg->group_size, cfg->zero_point, (uint16_t*)dW_out, (hipStream_t)stream));
}

namespace {
int pack_impl(const void* W, const float* s, const float* clip, int64_t out_features,
              int64_t in_features, const awq_qconfig* cfg, uint8_t* codes_out,
              void* scales_out, void* zeros_out, int32_t* status_out, void* stream) {
  if (!W || !s || !cfg || !codes_out || !scales_out || !zeros_out) return AWQ_E_NULL;
  if (!cfg_valid(cfg)) return AWQ_E_CONFIG;
  int st = weight_shape(out_features, in_features, cfg);
  if (st != AWQ_OK) return st;
  if (!aligned(W, 16) || !aligned(s, 16) || !aligned(codes_out, 4) || !aligned(scales_out, 2) ||
      !aligned(zeros_out, 2) || (clip && !aligned(clip, 4)) ||
      (status_out && !aligned(status_out, 4)))
    return AWQ_E_ALIGN;
  if (status_out && (st = device_ptr(status_out))) return st;
  clear_pending_error();
  if (out_features == 0 || in_features == 0) {
    // an empty layer stores no step: the status word still reports AWQ_OK
    if (status_out)
      return hip_status(awq::launch_quant_pack(nullptr, nullptr, nullptr, 0, 0, cfg->w_bit,
                                               cfg->group_size, cfg->zero_point, nullptr,
                                               nullptr, nullptr, status_out,
                                               (hipStream_t)stream));
    return AWQ_OK;
  }
  if ((st = device_ptr(W)) || (st = device_ptr(s)) || (st = device_ptr(codes_out)) ||
      (st = device_ptr(scales_out)) || (st = device_ptr(zeros_out)))
    return st;
  if (clip && (st = device_ptr(clip))) return st;
  return hip_status(awq::launch_quant_pack((const uint16_t*)W, s, clip, (int)out_features,
                                           (int)in_features, cfg->w_bit, cfg->group_size,
                                           cfg->zero_point, codes_out, (uint16_t*)scales_out,
                                           (uint16_t*)zeros_out, status_out,
                                           (hipStream_t)stream));
}
}  // namespace

int awq_quantize_pack(const void* W, const float* s, int64_t out_features, int64_t in_features,
                      const awq_qconfig* cfg, uint8_t* codes_out, void* scales_out,
                      void* zeros_out, void* stream) {
  return pack_impl(W, s, nullptr, out_features, in_features, cfg, codes_out, scales_out,
                   zeros_out, nullptr, stream);
}

int awq_quantize_pack_checked(const void* W, const float* s, const float* clip,
                              int64_t out_features, int64_t in_features,
                              const awq_qconfig* cfg, uint8_t* codes_out, void* scales_out,
                              void* zeros_out, int32_t* status_out, void* stream) {
  if (!status_out) return AWQ_E_NULL;
  return pack_impl(W, s, clip, out_features, in_features, cfg, codes_out, scales_out,
                   zeros_out, status_out, stream);
}

int awq_quantize_pack_clipped(const void* W, const float* s, const float* clip,
                              int64_t out_features, int64_t in_features, const awq_qconfig* cfg,
                              uint8_t* codes_out, void* scales_out, void* zeros_out,
                              void* stream) {
  if (!clip) return AWQ_E_NULL;
  return pack_impl(W, s, clip, out_features, in_features, cfg, codes_out, scales_out, zeros_out,
                   nullptr, stream);
}

size_t awq_clip_workspace_bytes(int64_t out_features, int64_t in_features, int64_t n_tokens,
                                const awq_qconfig* cfg) {
  if (!cfg_valid(cfg)) return 0;
  if (weight_shape(out_features, in_features, cfg) != AWQ_OK) return 0;
  if (token_shape(n_tokens, in_features) != AWQ_OK) return 0;
  const size_t kg = (size_t)in_features * cfg->group_size;
  const int splits = awq::gram_splits(n_tokens, in_features, cfg->group_size);
  const size_t ng = (size_t)(in_features / cfg->group_size);
  return 2 * round_up(kg * sizeof(uint16_t), kAlign) + round_up(ng * sizeof(int32_t), kAlign) +
         round_up(ng * awq::gram_chunks(cfg->group_size) * sizeof(double), kAlign) +
         round_up(kg * sizeof(double), kAlign) + round_up((size_t)splits * kg * sizeof(float), kAlign);
}

int awq_clip_search(const void* W, const void* X, const float* s, int64_t out_features,
                    int64_t in_features, int64_t n_tokens, const awq_qconfig* cfg,
                    const float* ratios_host, int32_t n_ratio, float* clip_out,
                    int32_t* best_out, float* errors_out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const int64_t M = out_features, K = in_features, N = n_tokens;
  if (!W || !X || !s || !cfg || !ratios_host || !clip_out) return AWQ_E_NULL;
  if (!workspace) return AWQ_E_WORKSPACE;
  if (!cfg_valid(cfg)) return AWQ_E_CONFIG;
  int st = weight_shape(M, K, cfg);
  if (st != AWQ_OK) return st;
  if ((st = token_shape(N, K)) != AWQ_OK) return st;
  if (n_ratio < 1 || n_ratio > awq::kMaxClip) return AWQ_E_ALPHA;
  awq::ClipList rl;
  memset(&rl, 0, sizeof(rl));
  for (int k = 0; k < n_ratio; ++k) {
    const float v = ratios_host[k];
    if (!(v > 0.0f && v <= 1.0f)) return AWQ_E_ALPHA;  // also rejects NaN
    rl.v[k] = v;
  }
  if (errors_out && K > 0 && (int64_t)n_ratio * M >= kMaxElems / (K / cfg->group_size))
    return AWQ_E_SHAPE;
  if (workspace_bytes < awq_clip_workspace_bytes(M, K, N, cfg)) return AWQ_E_WORKSPACE;
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(s, 4) || !aligned(clip_out, 4) ||
      !aligned(best_out, 4) || !aligned(errors_out, 4) || !aligned(workspace, kAlign))
    return AWQ_E_ALIGN;
  if (M == 0 || K == 0) return AWQ_OK;
  if ((st = device_ptr(W)) || (st = device_ptr(X)) || (st = device_ptr(s)) ||
      (st = device_ptr(clip_out)) || (st = device_ptr(workspace)))
    return st;
  if (best_out && (st = device_ptr(best_out))) return st;
  if (errors_out && (st = device_ptr(errors_out))) return st;
  const size_t kg = (size_t)K * cfg->group_size;
  char* ws = (char*)workspace;
  uint16_t* Ghi = (uint16_t*)ws;
  uint16_t* Glo = (uint16_t*)(ws + round_up(kg * sizeof(uint16_t), kAlign));
  const size_t ng = (size_t)(K / cfg->group_size);
  size_t off = 2 * round_up(kg * sizeof(uint16_t), kAlign);
  int32_t* gexp = (int32_t*)(ws + off);
  off += round_up(ng * sizeof(int32_t), kAlign);
  double* cmax = (double*)(ws + off);
  off += round_up(ng * awq::gram_chunks(cfg->group_size) * sizeof(double), kAlign);
  double* G64 = (double*)(ws + off);
  off += round_up(kg * sizeof(double), kAlign);
  float* partials = (float*)(ws + off);
  clear_pending_error();
  if ((st = hip_status(awq::launch_group_gram((const uint16_t*)X, s, (int)N, (int)K,
                                              cfg->group_size, partials, G64, cmax, Ghi, Glo,
                                              gexp, (hipStream_t)stream))))
    return st;
  return hip_status(awq::launch_clip_search((const uint16_t*)W, s, Ghi, Glo, gexp, (int)M,
                                            (int)K, cfg->w_bit, cfg->group_size,
                                            cfg->zero_point, rl, n_ratio, clip_out, best_out,
                                            errors_out, (hipStream_t)stream));
}

int awq_probe_mfma(int32_t blocks, int32_t iters, uint64_t* clocks_out, void* stream) {
  if (!clocks_out) return AWQ_E_NULL;
  if (blocks < 1 || blocks > (1 << 16) || iters < 1 || iters > (1 << 20) ||
      (int64_t)blocks * iters > ((int64_t)1 << 28))
    return AWQ_E_SHAPE;
  if (!aligned(clocks_out, 8)) return AWQ_E_ALIGN;
  int st;
  if ((st = device_ptr(clocks_out))) return st;
  clear_pending_error();
  return hip_status(awq::launch_probe_mfma(blocks, iters, (unsigned long long*)clocks_out,
                                           (hipStream_t)stream));
}

int awq_probe_lds(int32_t blocks, int32_t iters, uint64_t* clocks_out, void* stream) {
  if (!clocks_out) return AWQ_E_NULL;
  if (blocks < 1 || blocks > (1 << 16) || iters < 1 || iters > (1 << 20) ||
      (int64_t)blocks * iters > ((int64_t)1 << 28))
    return AWQ_E_SHAPE;
  if (!aligned(clocks_out, 8)) return AWQ_E_ALIGN;
  int st;
  if ((st = device_ptr(clocks_out))) return st;
  clear_pending_error();
  return hip_status(awq::launch_probe_lds(blocks, iters, (unsigned long long*)clocks_out,
                                          (hipStream_t)stream));
}

int awq_probe_read(const void* src, int64_t bytes, void* stream) {
  if (!src) return AWQ_E_NULL;
  if (bytes < 16 || bytes % 16 != 0) return AWQ_E_SHAPE;
  if (!aligned(src, 16)) return AWQ_E_ALIGN;
  int st;
  if ((st = device_ptr(src))) return st;
  clear_pending_error();
  return hip_status(awq::launch_probe_read(src, (long long)bytes, (hipStream_t)stream));
}

int awq_probe_write(void* dst, int64_t bytes, void* stream) {
  if (!dst) return AWQ_E_NULL;
  if (bytes < 16 || bytes % 16 != 0) return AWQ_E_SHAPE;
  if (!aligned(dst, 16)) return AWQ_E_ALIGN;
  int st;
  if ((st = device_ptr(dst))) return st;
  clear_pending_error();
  return hip_status(awq::launch_probe_write(dst, (long long)bytes, (hipStream_t)stream));
}

int awq_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst) return AWQ_E_NULL;
  if (bytes < 16 || bytes % 16 != 0) return AWQ_E_SHAPE;
  if (!aligned(src, 16) || !aligned(dst, 16)) return AWQ_E_ALIGN;
  int st;
  if ((st = device_ptr(src)) || (st = device_ptr(dst))) return st;
  clear_pending_error();
  return hip_status(awq::launch_probe_copy(src, dst, (long long)bytes, (hipStream_t)stream));
}

int awq_probe_wall_clock_khz(int32_t device, int32_t* khz_out) {
  if (!khz_out) return AWQ_E_NULL;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, device) != hipSuccess) {
    (void)hipGetLastError();
    return AWQ_E_HIP;
  }
  *khz_out = v;
  return AWQ_OK;
}

int awq_set_stats_profile_events(void* pass_start, void* pass_stop) {
  g_stats_ev[0] = pass_start;
  g_stats_ev[1] = pass_stop;
  return AWQ_OK;
}

int awq_set_profile_pass_events(void* const* events, int32_t n_pass) {
  if (n_pass < 0 || n_pass > AWQ_MAX_ALPHA) return AWQ_E_SHAPE;
  if (n_pass > 0 && !events) return AWQ_E_NULL;
  for (int i = 0; i < 4 * n_pass; ++i) g_pass_ev[i] = events[i];
  g_pass_n = n_pass;
  return AWQ_OK;
}

int awq_set_profile_events(void* gemm_start, void* gemm_stop, void* fq_start, void* fq_stop,
                           void* gram_start, void* gram_stop) {
  g_hook.gemm_start = gemm_start;
  g_hook.gemm_stop = gemm_stop;
  g_hook.fq_start = fq_start;
  g_hook.fq_stop = fq_stop;
  g_hook.gram_start = gram_start;
  g_hook.gram_stop = gram_stop;
  return AWQ_OK;
}

}  // extern "C"
