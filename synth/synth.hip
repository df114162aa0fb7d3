// synth.hip -- seeded synthetic inputs for the verify-and-sample step.
//
// Test and benchmark infrastructure: it produces the logits, draft tokens,
// uniforms, ragged lengths and page tables that both the GPU library and the
// CPU oracle consume.  It holds none of the verify / resample arithmetic.
//
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11), key = (seed, stream id), counter =
// (step, row, column block, 0).  A 32-bit draw x maps to the uniform
// (x >> 8) * 2^-24 in [0, 1).
//
// Streams: 0 rank permutation, 1 target noise, 2 draft noise, 3 draft-token
// sampling, 4 verify / bonus uniforms, 5 resample uniforms, 6 PACER scores.
//
// Logits (the distribution the workload descriptions give): target
// z_t[i] = 3 g + base_i with g ~ N(0, 1) and base_i = -0.5 ln(1 + rank_i) for a
// seeded permutation rank; draft z_d = z_t + delta g' at the same position.
// Both are rounded once (round to nearest even) to the stored dtype, the draft
// from the unrounded target.  Draft tokens are drawn from softmax(z_d / T) of
// the stored draft row by the Gumbel-max method.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace {

struct U4 {
  uint32_t x, y, z, w;
};

__host__ __device__ inline void mulhilo(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  const uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

// Philox4x32 with 10 rounds.
__host__ __device__ inline U4 philox(U4 ctr, uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; r++) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo(0xD2511F53u, ctr.x, &hi0, &lo0);
    mulhilo(0xCD9E8D57u, ctr.z, &hi1, &lo1);
    ctr = U4{hi1 ^ ctr.y ^ k0, lo1, hi0 ^ ctr.w ^ k1, lo0};
  }
  return ctr;
}

__host__ __device__ inline float u01(uint32_t x) { return (float)(x >> 8) * (1.0f / 16777216.0f); }
// open interval (0, 1), for logarithms
__host__ __device__ inline float u01_open(uint32_t x) {
  return ((float)(x >> 8) + 0.5f) * (1.0f / 16777216.0f);
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)(b >> 16) | ((b & 0xFFFFu) ? 0x40 : 0);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Four standard normals from one Philox block (Box-Muller on two pairs).
__device__ inline void normals4(U4 r, float (&g)[4]) {
  const float two_pi = 6.283185307179586f;
  const float a = sqrtf(-2.0f * logf(u01_open(r.x)));
  const float b = sqrtf(-2.0f * logf(u01_open(r.z)));
  float s0, c0, s1, c1;
  sincosf(two_pi * u01(r.y), &s0, &c0);
  sincosf(two_pi * u01(r.w), &s1, &c1);
  g[0] = a * c0;
  g[1] = a * s0;
  g[2] = b * c1;
  g[3] = b * s1;
}

// One thread per 4 consecutive logits of a target row (and its draft row).
__global__ void k_logits(int bf16, int64_t rows_t, int64_t V, const float* __restrict__ base,
                         const int32_t* __restrict__ draft_row, const float* __restrict__ delta_row,
                         uint32_t seed, uint32_t step, void* target, void* draft) {
  const int64_t nblk = (V + 3) / 4;
  const int64_t total = rows_t * nblk;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = g / nblk;
    const int64_t cb = g - t * nblk;
    const U4 ctr{step, (uint32_t)t, (uint32_t)cb, 0u};
    float gt[4], gd[4];
    normals4(philox(ctr, seed, 1u), gt);
    const int32_t d = draft_row[t];
    if (d >= 0) normals4(philox(ctr, seed, 2u), gd);
    const float dl = delta_row[t];
    for (int k = 0; k < 4; k++) {
      const int64_t i = cb * 4 + k;
      if (i >= V) break;
      const float zt = 3.0f * gt[k] + base[i];
      if (bf16) {
        static_cast<uint16_t*>(target)[t * V + i] = f32_to_bf16_rne(zt);
        if (d >= 0) static_cast<uint16_t*>(draft)[(int64_t)d * V + i] = f32_to_bf16_rne(zt + dl * gd[k]);
      } else {
        static_cast<float*>(target)[t * V + i] = zt;
        if (d >= 0) static_cast<float*>(draft)[(int64_t)d * V + i] = zt + dl * gd[k];
      }
    }
  }
}

// Gumbel-max draw d from softmax(z / T) of draft row rowmap[d] (row d without
// a map); one block per draw.
__global__ void k_draft_tokens(int bf16, int64_t rows_d, int64_t V, float inv_t, const void* draft,
                               const int32_t* __restrict__ rowmap, uint32_t seed, uint32_t step,
                               int32_t* __restrict__ tokens) {
  __shared__ float sv[1024];
  __shared__ int si[1024];
  for (int64_t d = blockIdx.x; d < rows_d; d += gridDim.x) {
    const int64_t src = rowmap ? (int64_t)rowmap[d] : d;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    const int64_t nblk = (V + 3) / 4;
    for (int64_t cb = threadIdx.x; cb < nblk; cb += blockDim.x) {
      const U4 r = philox(U4{step, (uint32_t)d, (uint32_t)cb, 0u}, seed, 3u);
      const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
      for (int k = 0; k < 4; k++) {
        const int64_t i = cb * 4 + k;
        if (i >= V) break;
        float z;
        if (bf16)
          z = __uint_as_float((uint32_t) static_cast<const uint16_t*>(draft)[src * V + i] << 16);
        else
          z = static_cast<const float*>(draft)[src * V + i];
        const float s = z * inv_t - logf(-logf(u01_open(rr[k])));
        if (s > best) {  // ascending i within a thread: strict keeps the smallest
          best = s;
          bi = (int)i;
        }
      }
    }
    sv[threadIdx.x] = best;
    si[threadIdx.x] = bi;
    __syncthreads();
    for (int off = blockDim.x / 2; off > 0; off >>= 1) {
      if ((int)threadIdx.x < off) {
        const float o = sv[threadIdx.x + off];
        const int oi = si[threadIdx.x + off];
        if (o > sv[threadIdx.x] || (o == sv[threadIdx.x] && oi < si[threadIdx.x])) {
          sv[threadIdx.x] = o;
          si[threadIdx.x] = oi;
        }
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) tokens[d] = si[0] == 0x7FFFFFFF ? 0 : si[0];
    __syncthreads();
  }
}

__global__ void k_uniforms(int64_t n, uint32_t seed, uint32_t stream_id, uint32_t step,
                           float* __restrict__ out) {
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g * 4 < n;
       g += (int64_t)gridDim.x * blockDim.x) {
    const U4 r = philox(U4{step, (uint32_t)g, 0u, 0u}, seed, stream_id);
    const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
    for (int k = 0; k < 4; k++)
      if (g * 4 + k < n) out[g * 4 + k] = u01(rr[k]);
  }
}

unsigned grid_for(int64_t work, int threads) {
  int64_t b = (work + threads - 1) / threads;
  if (b > 65536) b = 65536;
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

extern "C" {

// Philox4x32-10 of one counter block (host), for tests.
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const U4 r = philox(U4{ctr[0], ctr[1], ctr[2], ctr[3]}, key[0], key[1]);
  out[0] = r.x;
  out[1] = r.y;
  out[2] = r.z;
  out[3] = r.w;
}

// Rank prior (host): Fisher-Yates permutation from stream 0, then
// base[i] = -0.5 * ln(1 + rank[i]) computed in double and stored as fp32.
void synth_rank_base(int64_t V, uint32_t seed, int32_t* rank, float* base) {
  for (int64_t i = 0; i < V; i++) rank[i] = (int32_t)i;
  for (int64_t i = V - 1; i >= 1; i--) {
    const U4 r = philox(U4{(uint32_t)i, 0u, 0u, 0u}, seed, 0u);
    const int64_t j = (int64_t)(((uint64_t)r.x * (uint64_t)(i + 1)) >> 32);
    const int32_t tmp = rank[i];
    rank[i] = rank[j];
    rank[j] = tmp;
  }
  for (int64_t i = 0; i < V; i++) base[i] = (float)(-0.5 * log(1.0 + (double)rank[i]));
}

// PACER pre-verifier stand-in scores (host): scores[b, (m-1) * block + k] ~
// U(0,1) from stream 6 at counter (step, b, m-1, k / 4), element k % 4, for
// blocks m = 1..max_blocks.  The draft lengths follow from them by the PACER
// rule, which the library and the oracle each implement.
void synth_pacer_scores(int32_t B, int32_t block, int32_t max_blocks, uint32_t seed, uint32_t step,
                        float* scores) {
  for (int32_t b = 0; b < B; b++) {
    for (int32_t m = 1; m <= max_blocks; m++) {
      float* out = scores + ((int64_t)b * max_blocks + (m - 1)) * block;
      for (int32_t k = 0; k < block; k += 4) {
        const U4 r = philox(U4{step, (uint32_t)b, (uint32_t)(m - 1), (uint32_t)(k / 4)}, seed, 6u);
        const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
        for (int32_t e = 0; e < 4 && k + e < block; e++) out[k + e] = u01(rr[e]);
      }
    }
  }
}

int32_t synth_logits(int32_t bf16, int64_t rows_t, int64_t V, const float* base,
                     const int32_t* draft_row, const float* delta_row, uint32_t seed, uint32_t step,
                     void* target, void* draft, void* stream) {
  const int64_t work = rows_t * ((V + 3) / 4);
  if (work > 0)
    hipLaunchKernelGGL(k_logits, dim3(grid_for(work, 256)), dim3(256), 0, (hipStream_t)stream, bf16,
                       rows_t, V, base, draft_row, delta_row, seed, step, target, draft);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t synth_draft_tokens(int32_t bf16, int64_t rows_d, int64_t V, float temperature,
                           const void* draft, uint32_t seed, uint32_t step, int32_t* tokens,
                           void* stream) {
  if (rows_d > 0)
    hipLaunchKernelGGL(k_draft_tokens, dim3(grid_for(rows_d, 1)), dim3(1024), 0, (hipStream_t)stream,
                       bf16, rows_d, V, 1.0f / temperature, draft, nullptr, seed, step, tokens);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// n draws, draw d from draft row rowmap[d] (several draws may share a row:
// the children of one tree node), counter (step, d, ...) as above.
int32_t synth_draft_tokens_rows(int32_t bf16, int64_t n, int64_t V, float temperature, const void* draft,
                                const int32_t* rowmap, uint32_t seed, uint32_t step, int32_t* tokens,
                                void* stream) {
  if (n > 0)
    hipLaunchKernelGGL(k_draft_tokens, dim3(grid_for(n, 1)), dim3(1024), 0, (hipStream_t)stream, bf16, n, V,
                       1.0f / temperature, draft, rowmap, seed, step, tokens);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t synth_uniforms(int64_t n, uint32_t seed, uint32_t stream_id, uint32_t step, float* out,
                       void* stream) {
  if (n > 0)
    hipLaunchKernelGGL(k_uniforms, dim3(grid_for((n + 3) / 4, 256)), dim3(256), 0,
                       (hipStream_t)stream, n, seed, stream_id, step, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
