// Activation statistics for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels
// as awq_act_stats, with their fp64 partials in a static device array of this library
// instead of a caller workspace.
//
// The array lives in this code object; every GPU the library runs on holds its own copy
// from module load until the process ends.  Host code never passes the array's name to a
// kernel (in host code that name is a host-side stand-in, not a device address): on the
// first call on a device, with that device current, hipGetSymbolAddress gives the
// device's address, which is kept per device and used from then on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "awq_act.h"
#include "awq_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)AWQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return AWQ_E_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return AWQ_E_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AWQ_OK;
}

}  // namespace

extern "C" int awq_act_stats_noalloc(const void* X, int64_t n_tokens, int64_t in_features,
                                     float* a_out, void* stream) {
  if (!X || !a_out) return AWQ_E_NULL;
  // the size checks of awq_act_stats, and the partials must fit the static array
  const size_t need = awq_act_stats_workspace_bytes(n_tokens, in_features);
  if (need == 0) return AWQ_E_SHAPE;
  if (need > kScratchBytes) return AWQ_E_WORKSPACE;
  if (((uintptr_t)X % (in_features % 8 == 0 ? 16 : 2)) != 0 || ((uintptr_t)a_out % 4) != 0)
    return AWQ_E_ALIGN;
  if (in_features == 0) return AWQ_OK;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != AWQ_OK) return st;
  return awq_act_stats(X, n_tokens, in_features, a_out, ws, kScratchBytes, stream);
}
