// launch.h -- internal interface between the C-ABI entry points (api.hip) and
// the kernel launchers (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "smcsd.h"

#define SMCSD_MAX_K_DEV SMCSD_MAX_K
#define SMCSD_MAX_N_DEV SMCSD_MAX_N

namespace smcsd {

// cap on the grid of the streaming kernels (grid-stride loops beyond it)
constexpr int64_t kMaxStreamBlocks = 8192;

struct SdArgs {
  bool bf16, vec;
  int B, K;
  int64_t V, rows_t, rows_d;
  int ntiles;
  float c;  // log2(e) / T
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* uniforms;
  const int32_t* offsets;
  int32_t* num_accepted;
  int32_t* final_token;
  uint32_t* flags;
  float2* part;   // [(rows_t + rows_d) * ntiles]
  float* rmass;   // [B * ntiles]
  int32_t* ws_n;  // [B]
};

struct SmcArgs {
  bool bf16, vec;
  int P, N, K, L;
  int64_t V;
  int ntiles;
  float c, ess_frac;
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* bonus_u;
  const float* resample_u;
  float* logw;
  const int32_t* pt_in;
  int32_t* pt_out;
  int32_t* bonus_token;
  int32_t* ancestors;
  float* ess;
  int32_t* resampled;
  uint32_t* flags;
  float2* part;     // [P*N*(2K+1) * ntiles]
  float* ws_logw;   // [P*N]
};

hipError_t launch_sd(const SdArgs& a, hipStream_t s);
hipError_t launch_smc(const SmcArgs& a, hipStream_t s);

}  // namespace smcsd
