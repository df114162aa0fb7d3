// kernels.hip -- HIP kernels (gfx950) of the verify-and-sample step.
//
// Pipeline of sd_verify (standard speculative decoding; "Faster LLM Inference
// via Sequential Monte Carlo", sec. 1):
//   1. row_partials  every target and draft row, tile by tile: softmax partial
//                    (max, sum of exponentials) of each 2048-logit tile.
//   2. sd_decide     per sequence: merge the partials into row statistics,
//                    test u_j < p_j(x_j) / q_j(x_j) up to the first rejection,
//                    and, when a draft was rejected, the residual mass
//                    sum max(0, p_n - q_n) of every tile of the rejected pair.
//   3. sd_final      per sequence: locate the tile holding u * (total mass) and
//                    finish the inverse-CDF draw inside it (residual, or the
//                    bonus draw from p_{K_b} when every draft was accepted).
// Pipeline of smc_reweight_resample (same page, sec. 2 steps 3-4, sec. 3):
//   1. row_partials  as above.
//   2. smc_particle  per particle: log-weight increment sum_j log p - log q,
//                    and the (K+1)-th token drawn from p_K.
//   3. smc_resample  per prompt: ESS, threshold, systematic resampling.
//   4. pt_gather     page-table rows gathered by ancestor.
#include "device.h"
#include "launch.h"

namespace smcsd {

// ---------------------------------------------------------------------------
// 1. softmax partials of every tile of every row
// ---------------------------------------------------------------------------
template <typename DT, bool VL>
__global__ __launch_bounds__(BLOCK) void k_row_partials(const typename DT::raw* __restrict__ target,
                                                        const typename DT::raw* __restrict__ draft,
                                                        int64_t rows_t, int64_t rows_d, int64_t V,
                                                        int ntiles, float c, float2* __restrict__ part) {
  const int lane = threadIdx.x % WAVE;
  const int64_t wave0 = (int64_t)blockIdx.x * WAVES_PER_BLOCK + threadIdx.x / WAVE;
  const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_BLOCK;
  const int64_t total = (rows_t + rows_d) * ntiles;
  for (int64_t id = wave0; id < total; id += nwaves) {
    const int64_t vrow = id / ntiles;
    const int64_t tile = id - vrow * ntiles;
    const typename DT::raw* row =
        vrow < rows_t ? target + vrow * V : draft + (vrow - rows_t) * V;
    float v[PER_LANE];
    load_tile<DT, VL>(row, V, tile, lane, v);
    const float2 pt = tile_partial(v, c);
    if (lane == 0) part[id] = pt;
  }
}

// ---------------------------------------------------------------------------
// shared pieces of the per-sequence / per-particle kernels
// ---------------------------------------------------------------------------
__device__ inline void raise_flags(uint32_t* flags, uint32_t bits) {
  if (flags && bits) atomicOr(flags, bits);
}

// Residual weights max(0, p - q) of one tile of a (target, draft) row pair.
__device__ inline void residual_weights(const float (&vt)[PER_LANE], const float (&vd)[PER_LANE],
                                        float Mt, float Md, float c, float st, float sd,
                                        float (&r)[PER_LANE]) {
#pragma unroll
  for (int e = 0; e < PER_LANE; e++) {
    const float p = __builtin_amdgcn_exp2f((vt[e] - Mt) * c) * st;
    const float q = __builtin_amdgcn_exp2f((vd[e] - Md) * c) * sd;
    r[e] = fmaxf(p - q, 0.0f);
  }
}

// Wave-level search over per-tile weights W_t (t < ntiles) in ascending tile
// order.  Returns the first tile whose inclusive prefix exceeds u * total and
// the prefix before it, or -1 (with the last tile of positive weight in
// *last_tile) when rounding leaves no such tile.
template <typename WFN>
__device__ inline int locate_tile(int ntiles, WFN weight, double u, int lane, double* before,
                                  double* scale_total, int* last_tile) {
  double total = 0.0;
  int lastt = -1;
  for (int t0 = 0; t0 < ntiles; t0 += WAVE) {
    const int t = t0 + lane;
    const double W = t < ntiles ? weight(t) : 0.0;
    const double incl = wave_incl_scan_f64(W, lane);
    total += __shfl(incl, WAVE - 1, WAVE);
    int lt = W > 0.0 ? t : -1;
    for (int off = 32; off >= 1; off >>= 1) lt = max(lt, __shfl_xor(lt, off, WAVE));
    if (lt >= 0) lastt = lt;
  }
  *scale_total = total;
  *last_tile = lastt;
  const double target = u * total;
  double run = 0.0;
  for (int t0 = 0; t0 < ntiles; t0 += WAVE) {
    const int t = t0 + lane;
    const double W = t < ntiles ? weight(t) : 0.0;
    const double incl = wave_incl_scan_f64(W, lane);
    const uint64_t bal = __ballot(run + incl > target);
    if (bal) {
      const int src = __builtin_ctzll(bal);
      *before = run + __shfl(incl - W, src, WAVE);
      return t0 + src;
    }
    run += __shfl(incl, WAVE - 1, WAVE);
  }
  return -1;
}

// Inverse-CDF draw from p (the row's softmax) with uniform u: locate the tile
// from the per-tile partials, then search inside it.  One wavefront.
template <typename DT, bool VL>
__device__ int draw_from_row(const typename DT::raw* __restrict__ row, int64_t V,
                             const float2* __restrict__ part, int ntiles, const RowStat& rs, float c,
                             float u, int lane, uint32_t* fl) {
  auto weight = [&](int t) -> double {
    const float2 pt = part[t];
    return pt.x == -INFINITY ? 0.0
                             : (double)pt.y * exp2(((double)pt.x - (double)rs.M) * (double)c);
  };
  double before = 0.0, total = 0.0;
  int last_tile = -1;
  const int t = locate_tile(ntiles, weight, (double)u, lane, &before, &total, &last_tile);
  const int tt = t >= 0 ? t : (last_tile >= 0 ? last_tile : ntiles - 1);
  const float mt = part[tt].x;
  float v[PER_LANE];
  load_tile<DT, VL>(row, V, tt, lane, v);
#pragma unroll
  for (int e = 0; e < PER_LANE; e++) v[e] = __builtin_amdgcn_exp2f((v[e] - mt) * c);
  int last_pos = -1;
  int idx = -1;
  if (t >= 0) {
    const double tscale = exp2(((double)mt - (double)rs.M) * (double)c);
    const float local = (float)(((double)u * total - before) / tscale);
    idx = tile_search<DT>(v, local, lane, &last_pos);
  } else {
    tile_search<DT>(v, INFINITY, lane, &last_pos);
  }
  if (idx < 0) {
    *fl |= FLAG_CDF_CLAMP;
    idx = last_pos >= 0 ? last_pos : 0;
  }
  return tt * TILE + idx;
}

// Row statistics of `nrows` rows, spread over the block's wavefronts, into LDS.
struct RowRef {
  int64_t vrow;  // row index into the partials
};

template <typename ROWFN>
__device__ inline void merge_rows(const float2* __restrict__ part, int ntiles, float c, int nrows,
                                  ROWFN vrow_of, float* sM, double* sS, int* sOk) {
  const int lane = threadIdx.x % WAVE;
  const int wave = threadIdx.x / WAVE;
  for (int r = wave; r < nrows; r += WAVES_PER_BLOCK) {
    const RowStat rs = merge_row(part + vrow_of(r) * ntiles, ntiles, c, lane);
    if (lane == 0) {
      sM[r] = rs.M;
      sS[r] = rs.S;
      sOk[r] = rs.ok;
    }
  }
}

__device__ inline RowStat lds_stat(const float* sM, const double* sS, const int* sOk, int r) {
  RowStat rs;
  rs.M = sM[r];
  rs.S = sS[r];
  rs.ok = sOk[r];
  return rs;
}

// CSR / fixed layout of sequence b; returns false (and flags) if malformed.
__device__ inline bool seq_layout(int b, int K, const int32_t* __restrict__ offsets, int64_t rows_d,
                                  int64_t* d0, int* Kb) {
  if (!offsets) {
    *d0 = (int64_t)b * K;
    *Kb = K;
    return true;
  }
  const int64_t a = offsets[b], e = offsets[b + 1];
  *d0 = a;
  *Kb = (int)(e - a);
  return a >= 0 && e >= a && e - a <= K && e <= rows_d;
}

// ---------------------------------------------------------------------------
// 2. SD decision + residual tile masses.  grid = (ceil(ntiles / 4), B)
// ---------------------------------------------------------------------------
template <typename DT, bool VL>
__global__ __launch_bounds__(BLOCK) void k_sd_decide(
    const typename DT::raw* __restrict__ target, const typename DT::raw* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms,
    const int32_t* __restrict__ offsets, int K, int64_t V, int64_t rows_t, int64_t rows_d,
    int ntiles, float c, const float2* __restrict__ part, float* __restrict__ rmass,
    int32_t* __restrict__ ws_n, int32_t* __restrict__ num_accepted, uint32_t* flags) {
  __shared__ float sM[2 * SMCSD_MAX_K_DEV];
  __shared__ double sS[2 * SMCSD_MAX_K_DEV];
  __shared__ int sOk[2 * SMCSD_MAX_K_DEV];
  __shared__ int sN;
  __shared__ uint32_t sFlags;
  const int b = blockIdx.y;
  const int lane = threadIdx.x % WAVE;
  const int wave = threadIdx.x / WAVE;
  int64_t d0;
  int Kb;
  const bool good = seq_layout(b, K, offsets, rows_d, &d0, &Kb);
  if (!good) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      raise_flags(flags, FLAG_BAD_INPUT);
      num_accepted[b] = 0;
      ws_n[b] = -1;
    }
    return;
  }
  const int64_t t0 = d0 + b;
  if (threadIdx.x == 0) sFlags = 0;
  // rows 0..Kb-1: target rows t0+j; rows Kb..2Kb-1: draft rows d0+j
  merge_rows(part, ntiles, c, 2 * Kb,
             [&](int r) -> int64_t { return r < Kb ? t0 + r : rows_t + d0 + (r - Kb); }, sM, sS, sOk);
  __syncthreads();
  if (wave == 0) {
    int first_reject = Kb;
    uint32_t fl = 0;
    for (int j0 = 0; j0 < Kb; j0 += WAVE) {
      const int j = j0 + lane;
      bool reject = false;
      if (j < Kb) {
        const int32_t x = tokens[d0 + j];
        const RowStat st = lds_stat(sM, sS, sOk, j);
        const RowStat sd = lds_stat(sM, sS, sOk, Kb + j);
        if (!st.ok || !sd.ok) fl |= FLAG_NONFINITE;
        if (x < 0 || x >= V) {
          fl |= FLAG_BAD_INPUT;
          reject = true;
        } else {
          const float zt = DT::to_f32(target[(t0 + j) * V + x]);
          const float zd = DT::to_f32(draft[(d0 + j) * V + x]);
          const double rho = exp(log_prob(zt, st, c) - log_prob(zd, sd, c));
          reject = !((double)uniforms[t0 + j] < rho);
        }
      }
      const uint64_t bal = __ballot(reject);
      if (bal && first_reject == Kb) first_reject = j0 + __builtin_ctzll(bal);
    }
    for (int off = 32; off >= 1; off >>= 1) fl |= __shfl_xor(fl, off, WAVE);
    if (lane == 0) {
      sN = first_reject;
      sFlags = fl;
    }
  }
  __syncthreads();
  const int n = sN;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    num_accepted[b] = n;
    ws_n[b] = n;
    raise_flags(flags, sFlags);
  }
  if (n >= Kb) return;
  // residual masses of this block's tiles of the rejected pair (target n, draft n)
  const int tile = blockIdx.x * WAVES_PER_BLOCK + wave;
  if (tile >= ntiles) return;
  const RowStat st = lds_stat(sM, sS, sOk, n);
  const RowStat sd = lds_stat(sM, sS, sOk, Kb + n);
  float vt[PER_LANE], vd[PER_LANE], r[PER_LANE];
  load_tile<DT, VL>(target + (t0 + n) * V, V, tile, lane, vt);
  load_tile<DT, VL>(draft + (d0 + n) * V, V, tile, lane, vd);
  residual_weights(vt, vd, st.M, sd.M, c, (float)(1.0 / st.S), (float)(1.0 / sd.S), r);
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < PER_LANE; e++) s += r[e];
  s = wave_sum(s);
  if (lane == 0) rmass[(int64_t)b * ntiles + tile] = s;
}

// ---------------------------------------------------------------------------
// 3. SD final token.  grid = B, block = one wavefront
// ---------------------------------------------------------------------------
template <typename DT, bool VL>
__global__ __launch_bounds__(WAVE) void k_sd_final(
    const typename DT::raw* __restrict__ target, const typename DT::raw* __restrict__ draft,
    const float* __restrict__ uniforms, const int32_t* __restrict__ offsets, int K, int64_t V,
    int64_t rows_t, int64_t rows_d, int ntiles, float c, const float2* __restrict__ part,
    const float* __restrict__ rmass, const int32_t* __restrict__ ws_n,
    int32_t* __restrict__ final_token, uint32_t* flags) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int64_t d0;
  int Kb;
  if (!seq_layout(b, K, offsets, rows_d, &d0, &Kb)) {
    if (lane == 0) final_token[b] = 0;
    return;
  }
  const int64_t t0 = d0 + b;
  const int n = ws_n[b];
  const float u = uniforms[t0 + Kb];
  uint32_t fl = 0;
  const RowStat st = merge_row(part + (t0 + n) * ntiles, ntiles, c, lane);
  if (!st.ok) fl |= FLAG_NONFINITE;
  int y;
  if (n >= Kb) {
    y = draw_from_row<DT, VL>(target + (t0 + n) * V, V, part + (t0 + n) * ntiles, ntiles, st, c, u,
                              lane, &fl);
  } else {
    const RowStat sd = merge_row(part + (rows_t + d0 + n) * ntiles, ntiles, c, lane);
    const float* rm = rmass + (int64_t)b * ntiles;
    auto weight = [&](int t) -> double { return (double)rm[t]; };
    double before = 0.0, total = 0.0;
    int last_tile = -1;
    const int t = locate_tile(ntiles, weight, (double)u, lane, &before, &total, &last_tile);
    if (!(total > 0.0)) {
      // p_n and q_n agree to rounding: draw from p_n with the same uniform
      fl |= FLAG_ZERO_RESIDUAL;
      y = draw_from_row<DT, VL>(target + (t0 + n) * V, V, part + (t0 + n) * ntiles, ntiles, st, c, u,
                                lane, &fl);
    } else {
      const int tt = t >= 0 ? t : last_tile;
      float vt[PER_LANE], vd[PER_LANE], r[PER_LANE];
      load_tile<DT, VL>(target + (t0 + n) * V, V, tt, lane, vt);
      load_tile<DT, VL>(draft + (d0 + n) * V, V, tt, lane, vd);
      residual_weights(vt, vd, st.M, sd.M, c, (float)(1.0 / st.S), (float)(1.0 / sd.S), r);
      int last_pos = -1;
      int idx = -1;
      if (t >= 0) idx = tile_search<DT>(r, (float)((double)u * total - before), lane, &last_pos);
      else tile_search<DT>(r, INFINITY, lane, &last_pos);
      if (idx < 0) {
        fl |= FLAG_CDF_CLAMP;
        idx = last_pos >= 0 ? last_pos : 0;
      }
      y = tt * TILE + idx;
    }
  }
  if (lane == 0) {
    final_token[b] = y;
    raise_flags(flags, fl);
  }
}

// ---------------------------------------------------------------------------
// SMC 2. per particle: log-weight increment and the (K+1)-th token
// grid = P*N
// ---------------------------------------------------------------------------
template <typename DT, bool VL>
__global__ __launch_bounds__(BLOCK) void k_smc_particle(
    const typename DT::raw* __restrict__ target, const typename DT::raw* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ bonus_u,
    const float* __restrict__ logw_in, int K, int64_t V, int64_t rows_t, int ntiles, float c,
    const float2* __restrict__ part, float* __restrict__ ws_logw, int32_t* __restrict__ bonus_token,
    uint32_t* flags) {
  __shared__ float sM[2 * SMCSD_MAX_K_DEV + 1];
  __shared__ double sS[2 * SMCSD_MAX_K_DEV + 1];
  __shared__ int sOk[2 * SMCSD_MAX_K_DEV + 1];
  const int64_t i = blockIdx.x;
  const int lane = threadIdx.x % WAVE;
  const int wave = threadIdx.x / WAVE;
  const int64_t t0 = i * (K + 1), d0 = i * K;
  // rows 0..K: target rows t0+j; rows K+1..2K: draft rows d0+j
  merge_rows(part, ntiles, c, 2 * K + 1,
             [&](int r) -> int64_t { return r <= K ? t0 + r : rows_t + d0 + (r - K - 1); }, sM, sS,
             sOk);
  __syncthreads();
  if (wave != 0) return;
  uint32_t fl = 0;
  double delta = 0.0;
  for (int j0 = 0; j0 < K; j0 += WAVE) {
    const int j = j0 + lane;
    double dj = 0.0;
    if (j < K) {
      const int32_t x = tokens[d0 + j];
      const RowStat st = lds_stat(sM, sS, sOk, j);
      const RowStat sd = lds_stat(sM, sS, sOk, K + 1 + j);
      if (!st.ok || !sd.ok) fl |= FLAG_NONFINITE;
      if (x < 0 || x >= V) {
        fl |= FLAG_BAD_INPUT;
      } else {
        const float zt = DT::to_f32(target[(t0 + j) * V + x]);
        const float zd = DT::to_f32(draft[(d0 + j) * V + x]);
        dj = log_prob(zt, st, c) - log_prob(zd, sd, c);
      }
    }
    delta += wave_sum_f64(dj);
  }
  const RowStat sK = lds_stat(sM, sS, sOk, K);
  if (!sK.ok) fl |= FLAG_NONFINITE;
  const float lw = (float)((double)logw_in[i] + delta);
  if (lw != lw || lw == INFINITY) fl |= FLAG_NONFINITE;
  const int y = draw_from_row<DT, VL>(target + (t0 + K) * V, V, part + (t0 + K) * ntiles, ntiles, sK,
                                      c, bonus_u[i], lane, &fl);
  for (int off = 32; off >= 1; off >>= 1) fl |= __shfl_xor(fl, off, WAVE);
  if (lane == 0) {
    ws_logw[i] = lw;
    bonus_token[i] = y;
    raise_flags(flags, fl);
  }
}

// ---------------------------------------------------------------------------
// SMC 3. per prompt: ESS, threshold, systematic resampling.
// grid = P, block = 64 * ceil(N / 64) threads
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_smc_resample(const float* __restrict__ ws_logw,
                                                      const float* __restrict__ resample_u, int N,
                                                      float ess_frac, float* __restrict__ logw_out,
                                                      int32_t* __restrict__ ancestors,
                                                      float* __restrict__ ess,
                                                      int32_t* __restrict__ resampled,
                                                      uint32_t* flags) {
  __shared__ double sC[SMCSD_MAX_N_DEV];
  __shared__ double sRed[3][SMCSD_MAX_N_DEV / WAVE];
  const int p = blockIdx.x;
  const int k = threadIdx.x;
  const int lane = k % WAVE, wave = k / WAVE, nw = blockDim.x / WAVE;
  const float lw = k < N ? ws_logw[(int64_t)p * N + k] : -INFINITY;
  // max
  double m = wave_max_f64((double)lw);
  if (lane == 0) sRed[0][wave] = m;
  __syncthreads();
  double M = -INFINITY;
  for (int w = 0; w < nw; w++) M = fmax(M, sRed[0][w]);
  __syncthreads();
  const bool zero = !(M > -INFINITY);
  const double w = (!zero && k < N) ? exp((double)lw - M) : 0.0;
  // sums of w and w^2, and the inclusive scan of w
  const double incl = wave_incl_scan_f64(w, lane);
  const double w2 = wave_sum_f64(w * w);
  if (lane == WAVE - 1) sRed[1][wave] = incl;
  if (lane == 0) sRed[2][wave] = w2;
  __syncthreads();
  double before = 0.0, Sw = 0.0, Sw2 = 0.0;
  for (int v = 0; v < nw; v++) {
    if (v < wave) before += sRed[1][v];
    Sw += sRed[1][v];
    Sw2 += sRed[2][v];
  }
  const double E = zero ? 0.0 : Sw * Sw / Sw2;
  const bool do_res = !zero && E < (double)ess_frac * (double)N;
  if (k < N) sC[k] = (before + incl) / Sw;
  __syncthreads();
  uint32_t fl = 0;
  if (k == 0) {
    if (zero) fl |= FLAG_ZERO_WEIGHTS;
    if (M == INFINITY || M != M) fl |= FLAG_NONFINITE;
    ess[p] = (float)E;
    resampled[p] = do_res ? 1 : 0;
  }
  if (k < N) {
    int a = k;
    if (do_res) {
      const double U = ((double)resample_u[p] + (double)k) / (double)N;
      int lo = 0, hi = N;  // first index with C > U
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sC[mid] > U) hi = mid;
        else lo = mid + 1;
      }
      if (lo >= N) {
        fl |= FLAG_CDF_CLAMP;
        lo = N - 1;
        while (lo > 0 && !(exp((double)ws_logw[(int64_t)p * N + lo] - M) > 0.0)) lo--;
      }
      a = lo;
    }
    ancestors[(int64_t)p * N + k] = a;
    logw_out[(int64_t)p * N + k] = do_res ? 0.0f : lw;
  }
  raise_flags(flags, fl);
}

// ---------------------------------------------------------------------------
// SMC 4. page-table rows gathered by ancestor (a pointer permutation)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BLOCK) void k_pt_gather(const int32_t* __restrict__ pt_in,
                                                    int32_t* __restrict__ pt_out,
                                                    const int32_t* __restrict__ ancestors, int N,
                                                    int64_t rows, int L) {
  const int64_t total = rows * L;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = g / L;
    const int64_t l = g - i * L;
    const int64_t src = (i / N) * N + ancestors[i];
    pt_out[g] = pt_in[src * L + l];
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <typename DT, bool VL>
static hipError_t launch_sd_t(const SdArgs& a, hipStream_t s) {
  using raw = typename DT::raw;
  const raw* tg = static_cast<const raw*>(a.target);
  const raw* dr = static_cast<const raw*>(a.draft);
  const int64_t total_tiles = (a.rows_t + a.rows_d) * a.ntiles;
  const int64_t blocks = std::min<int64_t>((total_tiles + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK,
                                           kMaxStreamBlocks);
  hipLaunchKernelGGL((k_row_partials<DT, VL>), dim3((unsigned)blocks), dim3(BLOCK), 0, s, tg, dr,
                     a.rows_t, a.rows_d, a.V, a.ntiles, a.c, a.part);
  hipLaunchKernelGGL((k_sd_decide<DT, VL>),
                     dim3((unsigned)((a.ntiles + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK), a.B),
                     dim3(BLOCK), 0, s, tg, dr, a.tokens, a.uniforms, a.offsets, a.K, a.V, a.rows_t,
                     a.rows_d, a.ntiles, a.c, a.part, a.rmass, a.ws_n, a.num_accepted, a.flags);
  hipLaunchKernelGGL((k_sd_final<DT, VL>), dim3(a.B), dim3(WAVE), 0, s, tg, dr, a.uniforms,
                     a.offsets, a.K, a.V, a.rows_t, a.rows_d, a.ntiles, a.c, a.part, a.rmass, a.ws_n,
                     a.final_token, a.flags);
  return hipGetLastError();
}

hipError_t launch_sd(const SdArgs& a, hipStream_t s) {
  if (a.bf16) return a.vec ? launch_sd_t<Bf16, true>(a, s) : launch_sd_t<Bf16, false>(a, s);
  return a.vec ? launch_sd_t<F32, true>(a, s) : launch_sd_t<F32, false>(a, s);
}

template <typename DT, bool VL>
static hipError_t launch_smc_t(const SmcArgs& a, hipStream_t s) {
  using raw = typename DT::raw;
  const raw* tg = static_cast<const raw*>(a.target);
  const raw* dr = static_cast<const raw*>(a.draft);
  const int64_t PN = (int64_t)a.P * a.N;
  const int64_t rows_t = PN * (a.K + 1), rows_d = PN * a.K;
  const int64_t total_tiles = (rows_t + rows_d) * a.ntiles;
  const int64_t blocks = std::min<int64_t>((total_tiles + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK,
                                           kMaxStreamBlocks);
  hipLaunchKernelGGL((k_row_partials<DT, VL>), dim3((unsigned)blocks), dim3(BLOCK), 0, s, tg, dr,
                     rows_t, rows_d, a.V, a.ntiles, a.c, a.part);
  hipLaunchKernelGGL((k_smc_particle<DT, VL>), dim3((unsigned)PN), dim3(BLOCK), 0, s, tg, dr,
                     a.tokens, a.bonus_u, a.logw, a.K, a.V, rows_t, a.ntiles, a.c, a.part,
                     a.ws_logw, a.bonus_token, a.flags);
  const int threads = ((a.N + WAVE - 1) / WAVE) * WAVE;
  hipLaunchKernelGGL(k_smc_resample, dim3(a.P), dim3(threads), 0, s, a.ws_logw, a.resample_u, a.N,
                     a.ess_frac, a.logw, a.ancestors, a.ess, a.resampled, a.flags);
  if (a.pt_in && a.L > 0) {
    const int64_t total = PN * a.L;
    const int64_t blocks2 = std::min<int64_t>((total + BLOCK - 1) / BLOCK, kMaxStreamBlocks);
    hipLaunchKernelGGL(k_pt_gather, dim3((unsigned)blocks2), dim3(BLOCK), 0, s, a.pt_in, a.pt_out,
                       a.ancestors, a.N, PN, a.L);
  }
  return hipGetLastError();
}

hipError_t launch_smc(const SmcArgs& a, hipStream_t s) {
  if (a.bf16) return a.vec ? launch_smc_t<Bf16, true>(a, s) : launch_smc_t<Bf16, false>(a, s);
  return a.vec ? launch_smc_t<F32, true>(a, s) : launch_smc_t<F32, false>(a, s);
}

}  // namespace smcsd
