// launch.h -- internal interface between the C-ABI entry points (api.hip) and
// the kernel launchers (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smcsd.h"

namespace smcsd {

// k_stream: softmax partials of every tile and the logit of each row's
// draft token, for groups (SD sequences / SMC particles) laid out group-major.
struct StreamArgs {
  const void* target;
  const void* draft;
  const int32_t* offsets;  // CSR over draft rows, or null (fixed K)
  const int32_t* tokens;   // draft token of each draft row
  int64_t ngroups, rows_t, rows_d, V, total_tiles;
  int K, ntiles;
  float c;         // log2(e) / T
  float2* part;    // [total_tiles] partial (mc, s) of each tile, group-major
  float* tokz;     // [rows] logit of each row's draft token, group-major rows
  uint32_t* flags;
};

struct SdTailArgs {
  StreamArgs s;
  const float* uniforms;
  uint32_t* rcount;  // [B] tiles of residual mass stored (zero between calls)
  float* rmass;      // [B * ntiles] residual mass per tile
  int32_t* num_accepted;
  int32_t* final_token;
};

struct SmcTailArgs {
  StreamArgs s;
  int N, L;
  float ess_frac;
  const float* bonus_u;
  const float* resample_u;
  const float* logw_in;
  float* logw_out;   // same buffer as logw_in (each entry is read before it is written)
  float* ws_logw;    // [P*N] reweighted log-weights
  uint32_t* pcount;  // [P] particles finished per prompt (zero between calls)
  const int32_t* pt_in;
  int32_t* pt_out;
  int32_t* bonus_token;
  int32_t* ancestors;
  float* ess;
  int32_t* resampled;
};

hipError_t launch_sd(const SdTailArgs& a, bool bf16, bool vec, hipStream_t s);
hipError_t launch_smc(const SmcTailArgs& a, bool bf16, bool vec, hipStream_t s);

}  // namespace smcsd
