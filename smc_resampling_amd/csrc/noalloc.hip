// noalloc.hip -- smc_reweight_resample for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation): the same kernels, with their workspace in a static
// device array instead of a caller's buffer.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "smcsd.h"

// The scratch: what smc_reweight_resample keeps in its workspace (reweighted
// log-weights, segment partials, bonus-row tile partials), one copy per GPU,
// held until the process ends.  Every byte a call reads, that call wrote
// first, so nothing has to start at zero.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SMCSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_lookup;

// The device address of the current device's scratch, looked up once per
// device with that device current.
hipError_t device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" int32_t smc_reweight_resample_noalloc(int32_t dtype, int32_t P, int32_t N, int32_t K, int32_t V,
                                                 float temperature, float ess_frac, const void* target_logits,
                                                 const void* draft_logits, const int32_t* draft_tokens,
                                                 const float* bonus_uniforms, const float* resample_uniforms,
                                                 float* log_weights, const int32_t* page_table_in,
                                                 int32_t* page_table_out, int32_t pages_per_particle,
                                                 int32_t* bonus_token, int32_t* ancestors, float* ess,
                                                 int32_t* resampled, uint32_t* status_flags, void* stream) {
  // Argument checks first, by the entry point itself: with no workspace it
  // returns before planning or launching anything, SMCSD_ERR_WORKSPACE
  // meaning every other argument is valid.
  const int32_t pre = smc_reweight_resample(dtype, P, N, K, V, temperature, ess_frac, target_logits, draft_logits,
                                            draft_tokens, bonus_uniforms, resample_uniforms, log_weights,
                                            page_table_in, page_table_out, pages_per_particle, bonus_token,
                                            ancestors, ess, resampled, status_flags, nullptr, 0, stream);
  if (pre != SMCSD_ERR_WORKSPACE) return pre;
  if (smc_workspace_bytes(dtype, P, N, K, V) > SMCSD_NOALLOC_SCRATCH_BYTES) return SMCSD_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (device_scratch(&ws) != hipSuccess) return SMCSD_ERR_HIP;
  return smc_reweight_resample(dtype, P, N, K, V, temperature, ess_frac, target_logits, draft_logits, draft_tokens,
                               bonus_uniforms, resample_uniforms, log_weights, page_table_in, page_table_out,
                               pages_per_particle, bonus_token, ancestors, ess, resampled, status_flags, ws,
                               SMCSD_NOALLOC_SCRATCH_BYTES, stream);
}
