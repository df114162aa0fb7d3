// launch.h -- internal interface between the C-ABI entry points (api.hip) and
// the kernel launchers (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smcsd.h"

namespace smcsd {

// Phase A (tile streaming) of both kernels.
struct StreamArgs {
  const void* target;
  const void* draft;
  const int32_t* offsets;  // CSR over draft rows, or null (fixed K)
  int64_t ngroups, rows_t, rows_d, V, total_tiles;
  int K, ntiles;
  float c;           // log2(e) / T
  float2* part;      // [total_tiles] softmax partial of each tile, group-major
  uint32_t* gcount;  // [ngroups] tiles finished per group (zero between calls)
  uint32_t* flags;
};

struct SdFusedArgs {
  StreamArgs s;
  const int32_t* tokens;
  const float* uniforms;
  uint32_t* dec;     // [B] decision of each sequence (zero between calls)
  uint32_t* rcount;  // [B] residual slots arrived (zero between calls)
  void* rec;         // [B] statistics of the rejected pair
  float* rmass;      // [B * ntiles] residual mass per tile
  int32_t* num_accepted;
  int32_t* final_token;
};

struct SmcFusedArgs {
  StreamArgs s;
  int N, L;
  float ess_frac;
  const int32_t* tokens;
  const float* bonus_u;
  const float* resample_u;
  const float* logw_in;
  float* logw_out;    // same buffer as logw_in (each entry is read before it is written)
  float* ws_logw;     // [P*N] reweighted log-weights
  uint32_t* pcount;   // [P] particles finished per prompt (zero between calls)
  const int32_t* pt_in;
  int32_t* pt_out;
  int32_t* bonus_token;
  int32_t* ancestors;
  float* ess;
  int32_t* resampled;
};

hipError_t launch_sd(const SdFusedArgs& a, bool bf16, bool vec, hipStream_t s);
hipError_t launch_smc(const SmcFusedArgs& a, bool bf16, bool vec, hipStream_t s);

}  // namespace smcsd
