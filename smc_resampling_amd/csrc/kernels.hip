// kernels.hip -- the fused HIP kernels (gfx950) of the verify-and-sample step.
//
// One launch per library call.  The grid is persistent and no larger than the
// device holds at once, so every workgroup is resident for the whole launch.
//
// Phase A (both kernels): the logit rows are laid out group by group (a group
// is an SD sequence or an SMC particle; its rows are target rows 0..K_b, then
// draft rows 0..K_b-1) and cut into 2048-logit tiles.  Each wavefront streams a
// contiguous range of tiles, stores the softmax partial (max, sum of
// exponentials) of each, and adds the number of tiles it finished to its
// group's counter.  The wavefront that completes a group's count handles that
// group next.
//
// sd_verify ("Faster LLM Inference via Sequential Monte Carlo", sec. 1;
// variable lengths as in "PACER", Methodik):
//   decider   (last phase-A wavefront of a sequence): merges the partials into
//             row statistics, tests u_j < p_j(x_j) / q_j(x_j) up to the first
//             rejection n.  n = K_b: draws the bonus token from p_{K_b} (tile
//             located from the partials, then searched) and is done.
//             n < K_b: publishes n and the statistics of the rejected pair.
//   residual  one slot per tile of every sequence: waits (bounded) for the
//             decision; if a draft was rejected, stores the tile's mass of
//             max(0, p_n - q_n).  The last slot of a sequence to arrive
//             locates u * (total mass) among the tile masses and finishes the
//             inverse-CDF draw inside that tile.
// smc_reweight_resample (same page, sec. 2 steps 3-4; sec. 3):
//   particle  (last phase-A wavefront of a particle): log-weight increment
//             sum_j log p_j(x_j) - log q_j(x_j), and the (K+1)-th token drawn
//             from p_K.
//   prompt    (last particle of a prompt): Kish ESS, threshold, systematic
//             resampling, page-table rows gathered by ancestor.
// No wavefront waits on anything in the SMC kernel.
//
// Counters and flags live in the caller's workspace; each call returns them to
// zero, so the workspace must be zero-filled once before its first use.
#include <map>
#include <mutex>

#include "device.h"
#include "launch.h"

namespace smcsd {

constexpr int MAXR = 2 * SMCSD_MAX_K + 1;     // rows per group
constexpr uint32_t DEC_BONUS = 0xFFFFFFFFu;   // decision: every draft accepted
// bounded waits: give up after this many ticks of the 100 MHz wall clock
constexpr uint64_t kSpinTicks = 50000000ull;  // 0.5 s

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void raise_flags(uint32_t* flags, uint32_t bits) {
  if (flags && bits) atomicOr(flags, bits);
}

__device__ __forceinline__ uint32_t atomic_add_acq_rel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

// one acq_rel add per wavefront (lane 0), old value broadcast to every lane
__device__ __forceinline__ uint32_t wave_add(uint32_t* p, uint32_t v, int lane) {
  uint32_t old = 0;
  if (lane == 0) old = atomic_add_acq_rel(p, v);
  return __shfl(old, 0, WAVE);
}

__device__ __forceinline__ uint32_t load_acquire(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_release(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// reductions inside each 16-lane row; every lane receives its row's result
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f32<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f32<DPP_ROR4>(v));
  return fmaxf(v, dpp_f32<DPP_ROR8>(v));
}
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<DPP_QUAD_1032>(v);
  v += dpp_f64<DPP_QUAD_2301>(v);
  v += dpp_f64<DPP_ROR4>(v);
  return v + dpp_f64<DPP_ROR8>(v);
}

// Row statistics of `nrows` consecutive rows of partials (one wavefront; 16
// lanes per row, 4 rows at a time) into the wavefront's LDS slice.
__device__ __forceinline__ void merge_group_rows(const float2* __restrict__ part, int nrows, int ntiles, float c,
                                        float* sM, double* sS, int lane) {
  const int sub = lane & 15;
  for (int r0 = 0; r0 < nrows; r0 += 4) {
    const int r = r0 + (lane >> 4);
    const bool live = r < nrows;
    const float2* pr = part + (int64_t)(live ? r : 0) * ntiles;
    float m = -INFINITY;
    if (live)
      for (int t = sub; t < ntiles; t += 16) m = fmaxf(m, pr[t].x);
    const float M = row16_max(m);
    double s = 0.0;
    if (live && M != -INFINITY) {
      for (int t = sub; t < ntiles; t += 16) {
        const float2 pt = pr[t];
        if (pt.x != -INFINITY) s += (double)pt.y * exp2(((double)pt.x - (double)M) * (double)c);
      }
    }
    const double S = row16_sum(s);
    if (live && sub == 0) {
      sM[r] = M;
      sS[r] = S;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");  // LDS writes done before other lanes read
}

__device__ __forceinline__ RowStat stat_of(const float* sM, const double* sS, int r) {
  RowStat rs;
  rs.M = sM[r];
  rs.S = sS[r];
  rs.ok = (rs.M > -INFINITY) && (rs.M < INFINITY) && (rs.S >= 1.0) && (rs.S < INFINITY);
  return rs;
}

// Residual weights max(0, p - q) of one tile of a (target, draft) row pair.
__device__ __forceinline__ void residual_weights(const float (&vt)[PER_LANE], const float (&vd)[PER_LANE],
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
// order: the first tile whose inclusive prefix exceeds u * total, and the
// prefix before it; -1 (with the last tile of positive weight in *last_tile)
// when rounding leaves no such tile.
template <typename WFN>
__device__ __forceinline__ int locate_tile(int ntiles, WFN weight, double u, int lane, double* before,
                                  double* total_out, int* last_tile) {
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
  *total_out = total;
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

// Inverse-CDF draw from the softmax of `row` (statistics rs, tile partials
// `part`) with uniform u.  One wavefront.
template <typename DT, bool VL>
__device__ __forceinline__ int draw_from_row(const typename DT::raw* __restrict__ row, int64_t V,
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
    idx = tile_search<DT>(v, (float)(((double)u * total - before) / tscale), lane, &last_pos);
  } else {
    tile_search<DT>(v, INFINITY, lane, &last_pos);
  }
  if (idx < 0) {
    *fl |= FLAG_CDF_CLAMP;
    idx = last_pos >= 0 ? last_pos : 0;
  }
  return tt * TILE + idx;
}

// ---------------------------------------------------------------------------
// groups: layout of one SD sequence / SMC particle
// ---------------------------------------------------------------------------
struct Group {
  int64_t d0;  // first draft row
  int kb;      // draft length
  int64_t fr0; // first row in the group-major row order (= 2*d0 + g)
  bool ok;
};

__device__ __forceinline__ Group group_of(int64_t g, int K, const int32_t* __restrict__ offsets, int64_t rows_d) {
  Group G;
  if (!offsets) {
    G.d0 = g * K;
    G.kb = K;
    G.ok = true;
  } else {
    const int64_t a = offsets[g], e = offsets[g + 1];
    G.d0 = a;
    G.kb = (int)(e - a);
    G.ok = a >= 0 && e >= a && e - a <= K && e <= rows_d;
  }
  G.fr0 = 2 * G.d0 + g;
  return G;
}

// The group holding group-major row fr: largest g with 2*offsets[g] + g <= fr.
__device__ __forceinline__ int64_t find_group(int64_t fr, int64_t ngroups, int K, const int32_t* __restrict__ offsets) {
  if (!offsets) return fr / (2 * K + 1);
  int64_t lo = 0, hi = ngroups - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (2 * (int64_t)offsets[mid] + mid <= fr) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}



// Phase A of wavefront w of nw.  Calls on_group(g) (wave-uniform) whenever this
// wavefront completes group g's tile count.
template <typename DT, bool VL, typename ONGROUP>
__device__ __forceinline__ void stream_phase(const StreamArgs& a, int64_t w, int64_t nw, int lane, ONGROUP on_group) {
  using raw = typename DT::raw;
  const int64_t f0 = w * a.total_tiles / nw, f1 = (w + 1) * a.total_tiles / nw;
  if (f0 >= f1) return;
  int64_t g = find_group(f0 / a.ntiles, a.ngroups, a.K, a.offsets);
  Group G = group_of(g, a.K, a.offsets, a.rows_d);
  int64_t fr_end = G.fr0 + 2 * G.kb + 1;
  uint32_t done = 0;
  uint32_t bad = 0;
  for (int64_t f = f0; f < f1; f++) {
    const int64_t fr = f / a.ntiles;
    const int64_t tile = f - fr * a.ntiles;
    while (fr >= fr_end && g + 1 < a.ngroups) {  // next group
      if (done) {
        const uint32_t need = (uint32_t)((2 * G.kb + 1) * a.ntiles);
        if (wave_add(a.gcount + g, done, lane) + done == need) on_group(g);
        done = 0;
      }
      g++;
      G = group_of(g, a.K, a.offsets, a.rows_d);
      fr_end = G.fr0 + 2 * G.kb + 1;
    }
    const int64_t rr = fr - G.fr0;
    const raw* row = nullptr;
    if (G.ok && rr >= 0 && rr <= 2 * G.kb) {
      if (rr <= G.kb) {
        const int64_t tr = G.d0 + g + rr;
        if (tr < a.rows_t) row = static_cast<const raw*>(a.target) + tr * a.V;
      } else {
        const int64_t dr = G.d0 + rr - G.kb - 1;
        if (dr < a.rows_d) row = static_cast<const raw*>(a.draft) + dr * a.V;
      }
    }
    if (row) {
      float v[PER_LANE];
      load_tile<DT, VL>(row, a.V, tile, lane, v);
      const float2 pt = tile_partial(v, a.c);
      if (lane == 0) a.part[f] = pt;
    } else {
      bad = FLAG_BAD_INPUT;
    }
    done++;
  }
  if (done) {
    const uint32_t need = (uint32_t)((2 * G.kb + 1) * a.ntiles);
    if (wave_add(a.gcount + g, done, lane) + done == need) on_group(g);
  }
  if (lane == 0) raise_flags(a.flags, bad);
}

// ---------------------------------------------------------------------------
// sd_verify: one fused kernel
// ---------------------------------------------------------------------------
struct SdDecision {  // published by the decider of a sequence that rejected a draft
  float Mt, Md;
  double St, Sd;
};

template <typename DT, bool VL>
__global__ __launch_bounds__(BLOCK) void k_sd_fused(SdFusedArgs a) {
  using raw = typename DT::raw;
  __shared__ float sM[WAVES_PER_BLOCK][MAXR];
  __shared__ double sS[WAVES_PER_BLOCK][MAXR];
  const int lane = threadIdx.x % WAVE;
  const int wib = threadIdx.x / WAVE;
  const int64_t w = (int64_t)blockIdx.x * WAVES_PER_BLOCK + wib;
  const int64_t nw = (int64_t)gridDim.x * WAVES_PER_BLOCK;
  const raw* target = static_cast<const raw*>(a.s.target);
  const raw* draft = static_cast<const raw*>(a.s.draft);
  const int ntiles = a.s.ntiles;
  const float c = a.s.c;
  const int64_t V = a.s.V;
  uint32_t fl = 0;
  SdDecision* rec = reinterpret_cast<SdDecision*>(a.rec);

  // ---- decider: merge, accept test, bonus draw or publish the rejection ----
  auto decide = [&](int64_t b) {
    const Group G = group_of(b, a.s.K, a.s.offsets, a.s.rows_d);
    if (!G.ok) {  // malformed CSR offsets: nothing of this sequence is read
      fl |= FLAG_BAD_INPUT;
      return;
    }
    const int kb = G.kb;
    const int64_t t0 = G.d0 + b;
    const float2* pg = a.s.part + G.fr0 * ntiles;
    merge_group_rows(pg, 2 * kb + 1, ntiles, c, sM[wib], sS[wib], lane);
    int n = kb;
    for (int j0 = 0; j0 < kb; j0 += WAVE) {
      const int j = j0 + lane;
      bool reject = false;
      if (j < kb) {
        const int32_t x = a.tokens[G.d0 + j];
        const RowStat st = stat_of(sM[wib], sS[wib], j);
        const RowStat sd = stat_of(sM[wib], sS[wib], kb + 1 + j);
        if (!st.ok || !sd.ok) fl |= FLAG_NONFINITE;
        if (x < 0 || x >= V) {
          fl |= FLAG_BAD_INPUT;
          reject = true;
        } else {
          const float zt = DT::to_f32(target[(t0 + j) * V + x]);
          const float zd = DT::to_f32(draft[(G.d0 + j) * V + x]);
          const double rho = exp(log_prob(zt, st, c) - log_prob(zd, sd, c));
          reject = !((double)a.uniforms[t0 + j] < rho);
        }
      }
      const uint64_t bal = __ballot(reject);
      if (bal && n == kb) n = j0 + __builtin_ctzll(bal);
    }
    if (lane == 0) {
      a.num_accepted[b] = n;
      a.s.gcount[b] = 0;  // every phase-A wavefront of b has counted
    }
    if (n == kb) {
      const RowStat sk = stat_of(sM[wib], sS[wib], kb);
      if (!sk.ok) fl |= FLAG_NONFINITE;
      const int y = draw_from_row<DT, VL>(target + (t0 + kb) * V, V, pg + (int64_t)kb * ntiles, ntiles, sk, c,
                                          a.uniforms[t0 + kb], lane, &fl);
      if (lane == 0) {
        a.final_token[b] = y;
        store_release(a.dec + b, DEC_BONUS);
      }
    } else {
      if (lane == 0) {
        SdDecision d;
        d.Mt = sM[wib][n];
        d.St = sS[wib][n];
        d.Md = sM[wib][kb + 1 + n];
        d.Sd = sS[wib][kb + 1 + n];
        rec[b] = d;
        store_release(a.dec + b, (uint32_t)n + 1u);
      }
    }
  };

  stream_phase<DT, VL>(a.s, w, nw, lane, decide);

  // ---- residual slots: one per (sequence, tile) ----------------------------
  const int64_t nslots = a.s.ngroups * ntiles;
  const uint64_t t_end = wall_clock64() + kSpinTicks;  // one deadline for every wait of this wavefront
  for (int64_t slot = w; slot < nslots; slot += nw) {
    const int64_t b = slot / ntiles;
    const int tile = (int)(slot - b * ntiles);
    const Group G = group_of(b, a.s.K, a.s.offsets, a.s.rows_d);
    uint32_t d = 0;
    if (G.ok) {
      while ((d = load_acquire(a.dec + b)) == 0) {
        __builtin_amdgcn_s_sleep(4);
        if (wall_clock64() > t_end) {
          fl |= FLAG_SPIN_TIMEOUT;
          break;
        }
      }
    } else {
      fl |= FLAG_BAD_INPUT;
    }
    const bool residual = d != 0 && d != DEC_BONUS;
    const int n = residual ? (int)d - 1 : 0;
    const int64_t t0 = G.d0 + b;
    SdDecision dd{};
    if (residual) {
      dd = rec[b];
      float vt[PER_LANE], vd[PER_LANE], r[PER_LANE];
      load_tile<DT, VL>(target + (t0 + n) * V, V, tile, lane, vt);
      load_tile<DT, VL>(draft + (G.d0 + n) * V, V, tile, lane, vd);
      residual_weights(vt, vd, dd.Mt, dd.Md, c, (float)(1.0 / dd.St), (float)(1.0 / dd.Sd), r);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < PER_LANE; e++) s += r[e];
      s = wave_sum(s);
      if (lane == 0) a.rmass[slot] = s;
    }
    if (wave_add(a.rcount + b, 1u, lane) + 1u != (uint32_t)ntiles) continue;
    // last slot of sequence b
    if (residual) {
      const float* rm = a.rmass + b * ntiles;
      auto weight = [&](int t) -> double { return (double)rm[t]; };
      const float u = a.uniforms[t0 + G.kb];
      double before = 0.0, total = 0.0;
      int last_tile = -1;
      const int t = locate_tile(ntiles, weight, (double)u, lane, &before, &total, &last_tile);
      int y;
      if (!(total > 0.0)) {
        // p_n and q_n agree to rounding: draw from p_n with the same uniform
        fl |= FLAG_ZERO_RESIDUAL;
        RowStat st;
        st.M = dd.Mt;
        st.S = dd.St;
        st.ok = true;
        y = draw_from_row<DT, VL>(target + (t0 + n) * V, V, a.s.part + (G.fr0 + n) * ntiles, ntiles, st, c, u,
                                  lane, &fl);
      } else {
        const int tt = t >= 0 ? t : last_tile;
        float vt[PER_LANE], vd[PER_LANE], r[PER_LANE];
        load_tile<DT, VL>(target + (t0 + n) * V, V, tt, lane, vt);
        load_tile<DT, VL>(draft + (G.d0 + n) * V, V, tt, lane, vd);
        residual_weights(vt, vd, dd.Mt, dd.Md, c, (float)(1.0 / dd.St), (float)(1.0 / dd.Sd), r);
        int last_pos = -1, idx = -1;
        if (t >= 0) idx = tile_search<DT>(r, (float)((double)u * total - before), lane, &last_pos);
        else tile_search<DT>(r, INFINITY, lane, &last_pos);
        if (idx < 0) {
          fl |= FLAG_CDF_CLAMP;
          idx = last_pos >= 0 ? last_pos : 0;
        }
        y = tt * TILE + idx;
      }
      if (lane == 0) a.final_token[b] = y;
    } else if (d == 0 && lane == 0) {
      a.final_token[b] = 0;  // malformed sequence or timeout: unspecified
      a.num_accepted[b] = 0;
    }
    if (lane == 0) {  // every slot of b has read its decision
      a.rcount[b] = 0;
      a.dec[b] = 0;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) fl |= __shfl_xor(fl, off, WAVE);
  if (lane == 0) raise_flags(a.s.flags, fl);
}

// ---------------------------------------------------------------------------
// smc_reweight_resample: one fused kernel
// ---------------------------------------------------------------------------
template <typename DT, bool VL>
__global__ __launch_bounds__(BLOCK) void k_smc_fused(SmcFusedArgs a) {
  using raw = typename DT::raw;
  __shared__ float sM[WAVES_PER_BLOCK][MAXR];
  __shared__ double sS[WAVES_PER_BLOCK][MAXR];
  const int lane = threadIdx.x % WAVE;
  const int wib = threadIdx.x / WAVE;
  const int64_t w = (int64_t)blockIdx.x * WAVES_PER_BLOCK + wib;
  const int64_t nw = (int64_t)gridDim.x * WAVES_PER_BLOCK;
  const raw* target = static_cast<const raw*>(a.s.target);
  const raw* draft = static_cast<const raw*>(a.s.draft);
  const int ntiles = a.s.ntiles;
  const float c = a.s.c;
  const int64_t V = a.s.V;
  const int K = a.s.K;
  const int N = a.N;
  uint32_t fl = 0;

  // ---- prompt: ESS, threshold, systematic resampling, page-table gather ----
  auto resample = [&](int64_t p) {
    const int64_t base = p * N;
    double M = -INFINITY;
    for (int k0 = 0; k0 < N; k0 += WAVE)
      if (k0 + lane < N) M = fmax(M, (double)a.ws_logw[base + k0 + lane]);
    M = wave_max_f64(M);
    const bool zero = !(M > -INFINITY);
    if (M == INFINITY || M != M) fl |= FLAG_NONFINITE;
    double Sw = 0.0, Sw2 = 0.0;
    int last_pos = -1;
    if (!zero) {
      for (int k0 = 0; k0 < N; k0 += WAVE) {
        const int k = k0 + lane;
        const double wk = k < N ? exp((double)a.ws_logw[base + k] - M) : 0.0;
        Sw += wave_sum_f64(wk);
        Sw2 += wave_sum_f64(wk * wk);
        int lp = wk > 0.0 ? k : -1;
        for (int off = 32; off >= 1; off >>= 1) lp = max(lp, __shfl_xor(lp, off, WAVE));
        last_pos = max(last_pos, lp);
      }
    } else {
      fl |= FLAG_ZERO_WEIGHTS;
    }
    const double E = zero ? 0.0 : Sw * Sw / Sw2;
    const bool do_res = !zero && E < (double)a.ess_frac * (double)N;
    const double u = (double)a.resample_u[p];
    const bool gather = a.pt_in != nullptr && a.L > 0;
    const int64_t L = a.L;
    double run = 0.0;
    int carry = 0;  // first slot of the chunk's first particle
    for (int k0 = 0; k0 < N; k0 += WAVE) {
      const int i = k0 + lane;
      const float lw = i < N ? a.ws_logw[base + i] : 0.0f;
      int lo, hi;  // particle i supplies the slots [lo, hi)
      if (do_res) {
        // slot k descends from the first i with C_i > (u + k) / N, so particle i
        // receives k in [ceil(N C_{i-1} - u), ceil(N C_i - u)); consecutive
        // ranges share their end points, so every slot is covered exactly once
        const double wi = i < N ? exp((double)lw - M) : 0.0;
        const double incl = wave_incl_scan_f64(wi, lane);
        const double Ci = (run + incl) / Sw;
        double h = ceil((double)N * Ci - u);
        if (i >= last_pos) {  // the last particle with positive weight ends at N
          if (i == last_pos && h < (double)N) fl |= FLAG_CDF_CLAMP;
          h = (double)N;
        }
        hi = (int)fmin(fmax(h, 0.0), (double)N);
        run += __shfl(incl, WAVE - 1, WAVE);
      } else {
        hi = i + 1;
      }
      if (i >= N) hi = N;
      int prev = __shfl_up(hi, 1, WAVE);
      lo = lane == 0 ? carry : prev;
      hi = max(hi, lo);
      carry = __shfl(hi, WAVE - 1, WAVE);
      if (i < N) {
        for (int k = lo; k < hi; k++) a.ancestors[base + k] = i;
        a.logw_out[base + i] = do_res ? 0.0f : lw;
      }
      if (gather) {
        // rows of the slots this chunk supplies, one wavefront-wide copy each
        const int kbeg = __shfl(lo, 0, WAVE);
        for (int k = kbeg; k < carry; k++) {
          const uint64_t own = __ballot(lo <= k && k < hi);
          const int64_t src = base + k0 + __builtin_ctzll(own);
          const int32_t* __restrict__ from = a.pt_in + src * L;
          int32_t* __restrict__ to = a.pt_out + (base + k) * L;
          for (int64_t l = lane; l < L; l += WAVE) to[l] = from[l];
        }
      }
    }
    if (lane == 0) {
      a.ess[p] = (float)E;
      a.resampled[p] = do_res ? 1 : 0;
      a.pcount[p] = 0;
    }
  };

  // ---- particle: reweight and the (K+1)-th token ---------------------------
  auto particle = [&](int64_t i) {
    const int64_t t0 = i * (K + 1), d0 = i * K;
    const float2* pg = a.s.part + i * (2 * K + 1) * ntiles;
    merge_group_rows(pg, 2 * K + 1, ntiles, c, sM[wib], sS[wib], lane);
    double delta = 0.0;
    for (int j0 = 0; j0 < K; j0 += WAVE) {
      const int j = j0 + lane;
      double dj = 0.0;
      if (j < K) {
        const int32_t x = a.tokens[d0 + j];
        const RowStat st = stat_of(sM[wib], sS[wib], j);
        const RowStat sd = stat_of(sM[wib], sS[wib], K + 1 + j);
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
    const RowStat sk = stat_of(sM[wib], sS[wib], K);
    if (!sk.ok) fl |= FLAG_NONFINITE;
    const float lw = (float)((double)a.logw_in[i] + delta);
    if (lw != lw || lw == INFINITY) fl |= FLAG_NONFINITE;
    const int y = draw_from_row<DT, VL>(target + (t0 + K) * V, V, pg + (int64_t)K * ntiles, ntiles, sk, c,
                                        a.bonus_u[i], lane, &fl);
    if (lane == 0) {
      a.bonus_token[i] = y;
      a.ws_logw[i] = lw;
      a.s.gcount[i] = 0;
    }
    if (wave_add(a.pcount + i / N, 1u, lane) + 1u == (uint32_t)N) resample(i / N);
  };

  stream_phase<DT, VL>(a.s, w, nw, lane, particle);
  for (int off = 32; off >= 1; off >>= 1) fl |= __shfl_xor(fl, off, WAVE);
  if (lane == 0) raise_flags(a.s.flags, fl);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
// Workgroups of BLOCK threads the current device holds at once for `kernel`
// (queried once per device and kernel).  The persistent grids never exceed it.
static int resident_blocks(const void* kernel) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({dev, kernel});
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, BLOCK, 0) != hipSuccess) return 0;
  cache[{dev, kernel}] = cus * per_cu;
  return cus * per_cu;
}

static unsigned grid_for(int64_t total_tiles, int resident) {
  // enough wavefronts for one tile each, capped at what stays resident
  int64_t blocks = (total_tiles + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks > resident) blocks = resident;
  return (unsigned)(blocks < 1 ? 1 : blocks);
}

template <typename DT, bool VL>
static hipError_t launch_sd_t(const SdFusedArgs& a, hipStream_t s) {
  const int resident = resident_blocks(reinterpret_cast<const void*>(&k_sd_fused<DT, VL>));
  if (resident <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL((k_sd_fused<DT, VL>), dim3(grid_for(a.s.total_tiles, resident)), dim3(BLOCK), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sd(const SdFusedArgs& a, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_sd_t<Bf16, true>(a, s) : launch_sd_t<Bf16, false>(a, s);
  return vec ? launch_sd_t<F32, true>(a, s) : launch_sd_t<F32, false>(a, s);
}

template <typename DT, bool VL>
static hipError_t launch_smc_t(const SmcFusedArgs& a, hipStream_t s) {
  const int resident = resident_blocks(reinterpret_cast<const void*>(&k_smc_fused<DT, VL>));
  if (resident <= 0) return hipErrorInvalidDevice;
  hipLaunchKernelGGL((k_smc_fused<DT, VL>), dim3(grid_for(a.s.total_tiles, resident)), dim3(BLOCK), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_smc(const SmcFusedArgs& a, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_smc_t<Bf16, true>(a, s) : launch_smc_t<Bf16, false>(a, s);
  return vec ? launch_smc_t<F32, true>(a, s) : launch_smc_t<F32, false>(a, s);
}

}  // namespace smcsd
