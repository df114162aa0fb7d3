// draft.hip -- PACER draft lengths ("PACER: Blockwise Pre-verification for
// Speculative Decoding with Adaptive Length", Methodik 1-3): drafting goes in
// blocks; after each block the pre-verifier's mean estimated acceptance of its
// tokens is compared with a threshold t; below it the sequence stops,
// otherwise t grows by a factor rho and another block is drafted.
//
// One workgroup, a thread per sequence (chunks of 1024 sequences): the rule is
// a handful of scores per sequence, and the CSR offsets the ragged verify
// needs are one workgroup scan.  The decision is taken in double exactly as
// stated (scores summed in index order, divided by the block size, compared
// strictly; t multiplied by rho), so any implementation of the same
// arithmetic reaches the same lengths.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device.h"
#include "smcsd.h"

namespace smcsd {
namespace {

constexpr int PC_BLOCK = 1024;
constexpr int PC_WAVES = PC_BLOCK / WAVE;

struct PacerArgs {
  int32_t B, block, max_blocks;
  double t0, rho;
  const float* scores;
  int32_t* lengths;
  int32_t* offsets;
};

// Draft length of sequence b.
__device__ __forceinline__ int32_t pacer_length(const PacerArgs& a, int64_t b) {
  const float* s = a.scores + b * a.max_blocks * a.block;
  double t = a.t0;
  int m = 1;
  for (;; m++) {
    double sum = 0.0;
    for (int k = 0; k < a.block; k++) sum += (double)s[(int64_t)(m - 1) * a.block + k];
    const double mean = sum / a.block;
    if (mean < t || m == a.max_blocks) break;
    t = t * a.rho;
  }
  return a.block * m;
}

__global__ __launch_bounds__(PC_BLOCK) void k_pacer_lengths(PacerArgs a) {
  __shared__ int32_t wsum[PC_WAVES];
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  int32_t carry = 0;
  if (threadIdx.x == 0) a.offsets[0] = 0;
  for (int64_t b0 = 0; b0 < a.B; b0 += PC_BLOCK) {
    const int64_t b = b0 + threadIdx.x;
    const int32_t k = b < a.B ? pacer_length(a, b) : 0;
    // inclusive scan of the lengths over the workgroup
    int32_t x = k;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
      const int32_t y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == WAVE - 1) wsum[wave] = x;
    __syncthreads();
    int32_t before = 0, total = 0;
    for (int w = 0; w < PC_WAVES; w++) {
      const int32_t t = wsum[w];
      before += w < wave ? t : 0;
      total += t;
    }
    if (b < a.B) {
      a.lengths[b] = k;
      a.offsets[b + 1] = carry + before + x;
    }
    carry += total;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
}

}  // namespace
}  // namespace smcsd

extern "C" {

int32_t pacer_lengths(int32_t B, int32_t block, int32_t max_blocks, double t0, double rho, const float* scores,
                      int32_t* lengths, int32_t* offsets, void* stream) {
  using namespace smcsd;
  if (B < 0 || block < 1 || max_blocks < 1 || !isfinite(t0) || !isfinite(rho)) return SMCSD_ERR_INVALID_ARG;
  if ((int64_t)B * max_blocks * block > INT32_MAX) return SMCSD_ERR_INVALID_ARG;
  if (!offsets || (B > 0 && (!scores || !lengths))) return SMCSD_ERR_INVALID_ARG;
  PacerArgs a;
  a.B = B;
  a.block = block;
  a.max_blocks = max_blocks;
  a.t0 = t0;
  a.rho = rho;
  a.scores = scores;
  a.lengths = lengths;
  a.offsets = offsets;
  hipLaunchKernelGGL(k_pacer_lengths, dim3(1), dim3(PC_BLOCK), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? SMCSD_OK : SMCSD_ERR_HIP;
}

}  // extern "C"
