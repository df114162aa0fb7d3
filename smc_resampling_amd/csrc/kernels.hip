// kernels.hip -- HIP kernels (gfx950) of the verify-and-sample step.
//
// Each library call launches two kernels on the caller's stream.
//
// k_stream (both operations): the logit rows are laid out group by group (a
// group is an SD sequence or an SMC particle; its rows are target rows
// 0..K_b, then draft rows 0..K_b-1) and cut into 2048-logit tiles.  Each
// wavefront streams a contiguous range of tiles with the next tiles' loads in
// flight, and stores softmax partials (max, sum of exponentials) and the logit
// of each row's draft token.  It is the only kernel that reads the logit
// stream, and it holds nothing else, so it runs at full occupancy.
//
// k_sd_tail (sd_verify; "Faster LLM Inference via Sequential Monte Carlo",
// sec. 1; variable lengths as in "PACER", Methodik): one workgroup per
// (sequence, 4 tiles).  Each merges its sequence's partials into row
// statistics and tests u_j < p_j(x_j) / q_j(x_j) up to the first rejection n
// (every workgroup of a sequence reaches the same decision).  n = K_b: the
// workgroup whose tiles hold u * (total mass) of p_{K_b} draws the bonus token.
// n < K_b: each wavefront stores the mass of max(0, p_n - q_n) over its tile;
// the last workgroup of the sequence to finish locates the tile that holds
// u * (total mass) and draws the token inside it.
//
// k_smc_tail (smc_reweight_resample; same page, sec. 2 steps 3-4; sec. 3): one
// wavefront per particle: log-weight increment sum_j log p_j(x_j) - log
// q_j(x_j) and the (K+1)-th token drawn from p_K; the last particle of a
// prompt to finish computes the Kish ESS, resamples systematically when it is
// below the threshold, and gathers the page-table rows by ancestor.
//
// Counters live in the caller's workspace and every call returns them to zero.
#include <map>
#include <mutex>

#include "device.h"
#include "launch.h"

namespace smcsd {

constexpr int MAXR = 2 * SMCSD_MAX_K + 1;     // rows per group

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void raise_flags(uint32_t* flags, uint32_t bits) {
  if (flags && bits) atomicOr(flags, bits);
}

// Cross-wavefront communication.  Every value one wavefront hands to another
// (tile partials, decisions, residual masses, log-weights, counters) is
// written and read with agent-scope relaxed atomics, which on gfx950 are
// write-through / read-through at the device coherence point (`sc1`) and need
// no writeback or invalidation of the XCD-local L2.  A writer waits for its
// stores to complete before it bumps a counter or sets a flag; a reader that
// has seen the counter or flag then reads the values from the same point.
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), (uint64_t)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float2* p, float2 v) {
  const uint64_t b = ((uint64_t)__float_as_uint(v.y) << 32) | __float_as_uint(v.x);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __uint_as_float(
      __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ double ld_dev(const double* p) {
  return __longlong_as_double((long long)__hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<double*>(p)),
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float2 ld_dev(const float2* p) {
  const uint64_t b =
      __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float2*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
}
// wait until every memory operation this wavefront issued has completed
__device__ __forceinline__ void stores_done() {
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// one add per wavefront (lane 0, after the wavefront's stores completed); the
// old value is broadcast to every lane
__device__ __forceinline__ uint32_t wave_add(uint32_t* p, uint32_t v, int lane) {
  stores_done();
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, WAVE);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return old;
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

// reductions inside each quad of lanes; every lane receives its quad's result
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f32<DPP_QUAD_1032>(v));
  return fmaxf(v, dpp_f32<DPP_QUAD_2301>(v));
}
__device__ __forceinline__ double quad_sum(double v) {
  v += dpp_f64<DPP_QUAD_1032>(v);
  return v + dpp_f64<DPP_QUAD_2301>(v);
}

// Row statistics of `nrows` consecutive rows of partials into the
// wavefront's LDS slice (one wavefront; 4 lanes per row, 16 rows per pass, so
// a group of up to 16 rows is merged after a single round of loads):
// M = max of the partials' mc (log2 domain), S = sum of s * 2^(mc - M).
__device__ __forceinline__ void merge_group_rows(const float2* __restrict__ part, int nrows, int ntiles,
                                                 float* sM, double* sS, int lane) {
  const int sub = lane & 3;
  for (int r0 = 0; r0 < nrows; r0 += WAVE / 4) {
    const int r = r0 + (lane >> 2);
    const bool live = r < nrows;
    const float2* pr = part + (int64_t)(live ? r : 0) * ntiles;
    float m = -INFINITY;
    if (live)
      for (int t = sub; t < ntiles; t += 4) m = fmaxf(m, pr[t].x);
    const float M = quad_max(m);
    double acc = 0.0;
    if (live && M != -INFINITY) {
      for (int t = sub; t < ntiles; t += 4) {
        const float2 pt = pr[t];
        if (pt.x != -INFINITY) acc += (double)pt.y * exp2((double)pt.x - (double)M);
      }
    }
    const double S = quad_sum(acc);
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
  rs.ok = (rs.M > -INFINITY) && (rs.M < INFINITY) && (rs.S >= 0.5) && (rs.S < INFINITY);
  return rs;
}

// Residual weights max(0, p - q) of chunk ch of one tile of a (target, draft)
// row pair, p = 2^(z_t c - Mt) * st, q = 2^(z_d c - Md) * sd (Mt, Md in the
// log2 domain, st = 1 / S_t, sd = 1 / S_d).
template <typename DT>
__device__ __forceinline__ void residual_chunk(const Raw<DT>& rt, const Raw<DT>& rd, int ch, float Mt, float Md,
                                               float c, float st, float sd, float (&r)[DT::VEC]) {
  // p and q are rounded products: a fused multiply-subtract would keep one of
  // them exact and make p - q nonzero for equal rows
#pragma clang fp contract(off)
  float vt[DT::VEC], vd[DT::VEC];
  unpack<DT>(rt, ch, vt);
  unpack<DT>(rd, ch, vd);
#pragma unroll
  for (int k = 0; k < DT::VEC; k++) {
    const float p = __builtin_amdgcn_exp2f(fmaf(vt[k], c, -Mt)) * st;
    const float q = __builtin_amdgcn_exp2f(fmaf(vd[k], c, -Md)) * sd;
    r[k] = fmaxf(p - q, 0.0f);
  }
}

// Wave-level search over per-tile weights W_t (t < ntiles <= 256) in ascending
// tile order: the first tile whose inclusive prefix exceeds u * total, and the
// prefix before it; -1 (with the last tile of positive weight in *last_tile)
// when rounding leaves no such tile.  Each weight is read once.
constexpr int kMaxTileChunks = 4;  // ntiles <= 256, i.e. V <= 524288

template <typename WFN>
__device__ __forceinline__ int locate_tile(int ntiles, WFN weight, double u, int lane, double* before,
                                           double* total_out, int* last_tile) {
  double incl[kMaxTileChunks], W[kMaxTileChunks];
  double total = 0.0;
  int lastt = -1;
#pragma unroll
  for (int k = 0; k < kMaxTileChunks; k++) {
    const int t = k * WAVE + lane;
    W[k] = t < ntiles ? weight(t) : 0.0;
  }
#pragma unroll
  for (int k = 0; k < kMaxTileChunks; k++) {
    incl[k] = total + wave_incl_scan_f64(W[k], lane);
    total = __shfl(incl[k], WAVE - 1, WAVE);
    int lt = W[k] > 0.0 ? k * WAVE + lane : -1;
    for (int off = 32; off >= 1; off >>= 1) lt = max(lt, __shfl_xor(lt, off, WAVE));
    if (lt >= 0) lastt = lt;
  }
  *total_out = total;
  *last_tile = lastt;
  const double target = u * total;
#pragma unroll
  for (int k = 0; k < kMaxTileChunks; k++) {
    const uint64_t bal = __ballot(incl[k] > target);
    if (bal) {
      const int src = __builtin_ctzll(bal);
      *before = __shfl(incl[k] - W[k], src, WAVE);
      return k * WAVE + src;
    }
  }
  return -1;
}

// Inverse-CDF draw from the softmax of `row` (statistics rs, tile partials
// `part`) with uniform u.  One wavefront.
// Inverse-CDF draw from the softmax of `row` (statistics rs, per-tile
// partials `part`) with uniform u.  One wavefront.  Returns -1 when the
// located tile lies outside [tb, tb + tn) (another workgroup holds it).
template <typename DT, bool VL>
__device__ __forceinline__ int draw_from_row(const typename DT::raw* __restrict__ row, int64_t V,
                                             const float2* __restrict__ part, int ntiles, const RowStat& rs,
                                             float c, float u, int lane, uint32_t* fl, int tb, int tn) {
  auto weight = [&](int t) -> double {
    const float2 pt = part[t];
    return pt.x == -INFINITY ? 0.0 : (double)pt.y * exp2((double)pt.x - (double)rs.M);
  };
  double before = 0.0, total = 0.0;
  int last_tile = -1;
  const int t = locate_tile(ntiles, weight, (double)u, lane, &before, &total, &last_tile);
  const int tt = t >= 0 ? t : (last_tile >= 0 ? last_tile : ntiles - 1);
  if (tt < tb || tt >= tb + tn) return -1;
  const float mt = part[tt].x;
  const Raw<DT> raw = load_raw<DT, VL>(row, V, tt, lane);
  auto wfn = [&](int ch, float (&w)[DT::VEC]) {
    unpack<DT>(raw, ch, w);
#pragma unroll
    for (int k = 0; k < DT::VEC; k++) w[k] = __builtin_amdgcn_exp2f(fmaf(w[k], c, -mt));
  };
  int last_pos = -1;
  int idx = -1;
  if (t >= 0) {
    const double tscale = exp2((double)mt - (double)rs.M);
    idx = tile_search<DT>(wfn, (float)(((double)u * total - before) / tscale), lane, &last_pos);
  } else {
    tile_search<DT>(wfn, INFINITY, lane, &last_pos);
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



// Counters sit 64 bytes apart so that atomics on different groups do not
// share a cache line.
constexpr int CSTRIDE = 16;

// Position of the streaming cursor: the group holding row `fr`.
struct Cursor {
  int64_t g, fr_end;
  Group G;
};

__device__ __forceinline__ Cursor cursor_at(int64_t fr, const StreamArgs& a) {
  Cursor c;
  c.g = find_group(fr, a.ngroups, a.K, a.offsets);
  c.G = group_of(c.g, a.K, a.offsets, a.rows_d);
  c.fr_end = c.G.fr0 + 2 * c.G.kb + 1;
  return c;
}

__device__ __forceinline__ Cursor cursor_advance(Cursor c, int64_t fr, const StreamArgs& a) {
  while (fr >= c.fr_end && c.g + 1 < a.ngroups) {
    c.g++;
    c.G = group_of(c.g, a.K, a.offsets, a.rows_d);
    c.fr_end = c.G.fr0 + 2 * c.G.kb + 1;
  }
  return c;
}

// Row `fr` of the cursor's group (null when the layout is malformed); *bonus
// is set for the group's last target row, whose tiles keep their own partials.
template <typename raw>
__device__ __forceinline__ const raw* row_at(const Cursor& c, int64_t fr, const StreamArgs& a, bool* bonus) {
  const int64_t rr = fr - c.G.fr0;
  *bonus = rr == c.G.kb;
  if (!c.G.ok || rr < 0 || rr > 2 * c.G.kb) return nullptr;
  if (rr <= c.G.kb) {
    const int64_t tr = c.G.d0 + c.g + rr;
    return tr < a.rows_t ? static_cast<const raw*>(a.target) + tr * a.V : nullptr;
  }
  const int64_t dr = c.G.d0 + rr - c.G.kb - 1;
  return dr < a.rows_d ? static_cast<const raw*>(a.draft) + dr * a.V : nullptr;
}


// ---------------------------------------------------------------------------
// k_stream: softmax partials and token logits of every tile
// ---------------------------------------------------------------------------
// Wavefront w of nw streams tiles [f0, f1) with PF tiles' loads in flight
// while one is reduced.  The partial of a tile is (MC, S): MC = max over the
// tile of z c (log2 domain, c = log2(e) / T) and S = sum 2^(z c - MC), formed
// from per-lane maxima and sums so that no exponential waits for a
// wavefront-wide maximum.  It depends on the tile's logits alone, so equal rows
// get bitwise equal statistics however the stream is divided.  The wavefront
// that streams the tile holding a row's draft token also stores that logit in
// tokz[row].
template <typename DT, bool VL, int PF>
__global__ __launch_bounds__(BLOCK) void k_stream(StreamArgs a) {
  using raw = typename DT::raw;
  const int lane = threadIdx.x % WAVE;
  const int64_t w = (int64_t)blockIdx.x * WAVES_PER_BLOCK + threadIdx.x / WAVE;
  const int64_t nw = (int64_t)gridDim.x * WAVES_PER_BLOCK;
  const int64_t f0 = w * a.total_tiles / nw, f1 = (w + 1) * a.total_tiles / nw;
  if (f0 >= f1) return;
  const int ntiles = a.ntiles;
  const float c = a.c;
  const int64_t fr_first = f0 / ntiles;
  const int t_first = (int)(f0 - fr_first * ntiles);
  // load cursor: issues the loads of tile f + PF while tile f is reduced
  int64_t lfr = fr_first;
  int lt = t_first;
  Cursor lc = cursor_at(lfr, a);
  auto fetch = [&]() {
    if (lt == 0) lc = cursor_advance(lc, lfr, a);
    bool bonus = false;
    const raw* row = row_at<raw>(lc, lfr, a, &bonus);
    Raw<DT> x = {};
    if (row) x = load_raw<DT, VL>(row, a.V, lt, lane);
    if (++lt == ntiles) {
      lt = 0;
      lfr++;
    }
    return x;
  };
  Raw<DT> q[PF + 1];
#pragma unroll
  for (int i = 0; i <= PF; i++) q[i] = f0 + i < f1 ? fetch() : Raw<DT>{};
  // reduce cursor: the row of the tile being reduced
  int64_t fr = fr_first;
  int t = t_first;
  Cursor rc = lc;
  rc = cursor_at(fr, a);
  bool bonus = false, valid = false;
  int tok_tile = -1;  // tile of this row that holds its draft token, if this wavefront streams it
  float tok_z = 0.0f;
  auto enter_row = [&]() {  // row fr starts (or the range starts inside it)
    rc = cursor_advance(rc, fr, a);
    const raw* row = row_at<raw>(rc, fr, a, &bonus);
    valid = row != nullptr;
    tok_tile = -1;
    if (valid && !bonus) {
      const int64_t rr = fr - rc.G.fr0;
      const int32_t tok = a.tokens[rc.G.d0 + (rr <= rc.G.kb ? rr : rr - rc.G.kb - 1)];
      const int64_t ft = fr * ntiles + tok / TILE;
      if (tok >= 0 && tok < a.V && ft >= f0 && ft < f1) {  // load it now, store it with its tile
        tok_tile = tok / TILE;
        tok_z = DT::to_f32(row[tok]);
      }
    }
  };
  enter_row();
  uint32_t bad = 0;
  for (int64_t f = f0; f < f1; f++) {
    const Raw<DT> cur = q[0];
#pragma unroll
    for (int i = 0; i < PF; i++) q[i] = q[i + 1];
    if (f + PF + 1 < f1) q[PF] = fetch();
    if (valid) {
      float v[PER_LANE];
#pragma unroll
      for (int ch = 0; ch < Raw<DT>::CHUNKS; ch++) {
        float u8[DT::VEC];
        unpack<DT>(cur, ch, u8);
#pragma unroll
        for (int k = 0; k < DT::VEC; k++) v[ch * DT::VEC + k] = u8[k];
      }
      // this lane's max and sum of 2^(z c - mc_lane), then the wavefront's
      // (MC, sum of s_lane 2^(mc_lane - MC)): a function of the tile alone
      float tm = -INFINITY;
#pragma unroll
      for (int e = 0; e < PER_LANE; e++) tm = fmaxf(tm, v[e]);
      const float mcl = tm * c;
      float sl = 0.0f;
      if (tm > -INFINITY) {
#pragma unroll
        for (int e = 0; e < PER_LANE; e++) sl += __builtin_amdgcn_exp2f(fmaf(v[e], c, -mcl));
      }
      const float MC = wave_max(mcl);
      const float S = wave_sum(tm > -INFINITY ? sl * __builtin_amdgcn_exp2f(mcl - MC) : 0.0f);
      const float2 pt = make_float2(MC, S);
      if (lane == 0) {
        a.part[f] = pt;
        if (t == tok_tile) a.tokz[fr] = tok_z;
      }
    } else {
      bad = FLAG_BAD_INPUT;
    }
    if (++t == ntiles) {
      t = 0;
      fr++;
      if (f + 1 < f1) enter_row();
    }
  }
  if (lane == 0) raise_flags(a.flags, bad);
}

// ---------------------------------------------------------------------------
// k_sd_tail: decision and final token.  grid = (ceil(ntiles / 4), B)
// ---------------------------------------------------------------------------
template <typename DT, bool VL>
__global__ __launch_bounds__(BLOCK) void k_sd_tail(SdTailArgs a) {
  using raw = typename DT::raw;
  __shared__ float sM[MAXR];
  __shared__ double sS[MAXR];
  __shared__ int sN;
  __shared__ uint32_t sFlags;
  __shared__ int sLast;
  const int lane = threadIdx.x % WAVE;
  const int wave = threadIdx.x / WAVE;
  const int64_t b = blockIdx.y;
  const raw* target = static_cast<const raw*>(a.s.target);
  const raw* draft = static_cast<const raw*>(a.s.draft);
  const int ntiles = a.s.ntiles;
  const float c = a.s.c;
  const int64_t V = a.s.V;
  const Group G = group_of(b, a.s.K, a.s.offsets, a.s.rows_d);
  if (!G.ok) {  // malformed CSR offsets: nothing of this sequence is read
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      raise_flags(a.s.flags, FLAG_BAD_INPUT);
      a.num_accepted[b] = 0;
      a.final_token[b] = 0;
    }
    return;
  }
  const int kb = G.kb;
  const int64_t t0 = G.d0 + b;
  const float2* pg = a.s.part + G.fr0 * ntiles;
  uint32_t fl = 0;
  if (wave == 0) {
    merge_group_rows(pg, 2 * kb + 1, ntiles, sM, sS, lane);
    int n = kb;
    for (int j0 = 0; j0 < kb; j0 += WAVE) {
      const int j = j0 + lane;
      bool reject = false;
      if (j < kb) {
        const int32_t x = a.s.tokens[G.d0 + j];
        const RowStat st = stat_of(sM, sS, j);
        const RowStat sd = stat_of(sM, sS, kb + 1 + j);
        if (!st.ok || !sd.ok) fl |= FLAG_NONFINITE;
        if (x < 0 || x >= V) {
          fl |= FLAG_BAD_INPUT;
          reject = true;
        } else {
          const float zt = a.s.tokz[G.fr0 + j];
          const float zd = a.s.tokz[G.fr0 + kb + 1 + j];
          const double rho = exp(log_prob(zt, st, c) - log_prob(zd, sd, c));
          reject = !((double)a.uniforms[t0 + j] < rho);
        }
      }
      const uint64_t bal = __ballot(reject);
      if (bal && n == kb) n = j0 + __builtin_ctzll(bal);
    }
    for (int off = 32; off >= 1; off >>= 1) fl |= __shfl_xor(fl, off, WAVE);
    if (lane == 0) {
      sN = n;
      sFlags = fl;
    }
  }
  __syncthreads();
  const int n = sN;
  fl = 0;
  const float u = a.uniforms[t0 + kb];
  const int tile = blockIdx.x * WAVES_PER_BLOCK + wave;
  if (n == kb) {
    // bonus draw from p_{K_b}: only the workgroup holding the located tile draws
    if (wave == 0) {
      const RowStat sk = stat_of(sM, sS, kb);
      if (!sk.ok) fl |= FLAG_NONFINITE;
      const int y = draw_from_row<DT, VL>(target + (t0 + kb) * V, V, pg + (int64_t)kb * ntiles, ntiles, sk, c, u,
                                          lane, &fl, (int)blockIdx.x * WAVES_PER_BLOCK, WAVES_PER_BLOCK);
      if (lane == 0) {
        if (y >= 0) a.final_token[b] = y;
        if (blockIdx.x == 0) a.num_accepted[b] = n;
        raise_flags(a.s.flags, fl | (blockIdx.x == 0 ? sFlags : 0u));
      }
    }
    return;
  }
  // residual mass of max(0, p_n - q_n) over this wavefront's tile
  const RowStat st = stat_of(sM, sS, n), sd = stat_of(sM, sS, kb + 1 + n);
  const float stf = (float)(1.0 / st.S), sdf = (float)(1.0 / sd.S);
  if (tile < ntiles) {
    const Raw<DT> rt = load_raw<DT, VL>(target + (t0 + n) * V, V, tile, lane);
    const Raw<DT> rd = load_raw<DT, VL>(draft + (G.d0 + n) * V, V, tile, lane);
    float s = 0.0f;
#pragma unroll
    for (int ch = 0; ch < Raw<DT>::CHUNKS; ch++) {
      float r[DT::VEC];
      residual_chunk<DT>(rt, rd, ch, st.M, sd.M, c, stf, sdf, r);
#pragma unroll
      for (int k = 0; k < DT::VEC; k++) s += r[k];
    }
    s = wave_sum(s);
    if (lane == 0) st_dev(a.rmass + b * ntiles + tile, s);
  }
  stores_done();  // every wavefront's mass is stored before the workgroup counts it
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t mine = (uint32_t)min(WAVES_PER_BLOCK, ntiles - (int)blockIdx.x * WAVES_PER_BLOCK);
    const uint32_t old = __hip_atomic_fetch_add(a.rcount + b * CSTRIDE, mine, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    sLast = old + mine == (uint32_t)ntiles;
    if (blockIdx.x == 0) {
      a.num_accepted[b] = n;
      raise_flags(a.s.flags, sFlags);
    }
  }
  __syncthreads();
  if (!sLast || wave != 0) return;
  // last workgroup of sequence b: locate the tile, then draw inside it
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const float* rm = a.rmass + b * ntiles;
  auto weight = [&](int t) -> double { return (double)ld_dev(rm + t); };
  double before = 0.0, total = 0.0;
  int last_tile = -1;
  const int t = locate_tile(ntiles, weight, (double)u, lane, &before, &total, &last_tile);
  int y;
  if (!(total > 0.0)) {
    // p_n and q_n agree to rounding: draw from p_n with the same uniform
    fl |= FLAG_ZERO_RESIDUAL;
    y = draw_from_row<DT, VL>(target + (t0 + n) * V, V, pg + (int64_t)n * ntiles, ntiles, st, c, u, lane, &fl, 0,
                              ntiles);
  } else {
    const int tt = t >= 0 ? t : last_tile;
    const Raw<DT> rt = load_raw<DT, VL>(target + (t0 + n) * V, V, tt, lane);
    const Raw<DT> rd = load_raw<DT, VL>(draft + (G.d0 + n) * V, V, tt, lane);
    auto wfn = [&](int ch, float (&w)[DT::VEC]) { residual_chunk<DT>(rt, rd, ch, st.M, sd.M, c, stf, sdf, w); };
    int last_pos = -1, idx = -1;
    if (t >= 0) idx = tile_search<DT>(wfn, (float)((double)u * total - before), lane, &last_pos);
    else tile_search<DT>(wfn, INFINITY, lane, &last_pos);
    if (idx < 0) {
      fl |= FLAG_CDF_CLAMP;
      idx = last_pos >= 0 ? last_pos : 0;
    }
    y = tt * TILE + idx;
  }
  if (lane == 0) {
    a.final_token[b] = y;
    st_dev(a.rcount + b * CSTRIDE, 0u);  // every workgroup of b has counted
    raise_flags(a.s.flags, fl);
  }
}

// ---------------------------------------------------------------------------
// k_smc_tail: one wavefront per particle, then per prompt.  grid = ceil(P N / 4)
// ---------------------------------------------------------------------------
template <typename DT, bool VL>
__global__ __launch_bounds__(BLOCK) void k_smc_tail(SmcTailArgs a) {
  using raw = typename DT::raw;
  __shared__ float sM[WAVES_PER_BLOCK][MAXR];
  __shared__ double sS[WAVES_PER_BLOCK][MAXR];
  const int lane = threadIdx.x % WAVE;
  const int wib = threadIdx.x / WAVE;
  const int64_t i = (int64_t)blockIdx.x * WAVES_PER_BLOCK + wib;
  if (i >= a.s.ngroups) return;
  const raw* target = static_cast<const raw*>(a.s.target);
  const int ntiles = a.s.ntiles;
  const float c = a.s.c;
  const int64_t V = a.s.V;
  const int K = a.s.K;
  const int N = a.N;
  uint32_t fl = 0;
  // ---- particle: reweight and the (K+1)-th token ---------------------------
  const int64_t t0 = i * (K + 1), d0 = i * K, fr0 = i * (2 * K + 1);
  const float2* pg = a.s.part + fr0 * ntiles;
  merge_group_rows(pg, 2 * K + 1, ntiles, sM[wib], sS[wib], lane);
  double delta = 0.0;
  for (int j0 = 0; j0 < K; j0 += WAVE) {
    const int j = j0 + lane;
    double dj = 0.0;
    if (j < K) {
      const int32_t x = a.s.tokens[d0 + j];
      const RowStat st = stat_of(sM[wib], sS[wib], j);
      const RowStat sd = stat_of(sM[wib], sS[wib], K + 1 + j);
      if (!st.ok || !sd.ok) fl |= FLAG_NONFINITE;
      if (x < 0 || x >= V) {
        fl |= FLAG_BAD_INPUT;
      } else {
        dj = log_prob(a.s.tokz[fr0 + j], st, c) - log_prob(a.s.tokz[fr0 + K + 1 + j], sd, c);
      }
    }
    delta += wave_sum_f64(dj);
  }
  const RowStat sk = stat_of(sM[wib], sS[wib], K);
  if (!sk.ok) fl |= FLAG_NONFINITE;
  const float lw = (float)((double)a.logw_in[i] + delta);
  if (lw != lw || lw == INFINITY) fl |= FLAG_NONFINITE;
  const int y = draw_from_row<DT, VL>(target + (t0 + K) * V, V, pg + (int64_t)K * ntiles, ntiles, sk, c,
                                      a.bonus_u[i], lane, &fl, 0, ntiles);
  if (lane == 0) {
    a.bonus_token[i] = y;
    st_dev(a.ws_logw + i, lw);
  }
  const int64_t p = i / N;
  if (wave_add(a.pcount + p * CSTRIDE, 1u, lane) + 1u == (uint32_t)N) {
    // ---- prompt: ESS, threshold, systematic resampling, page-table gather ----
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int64_t base = p * N;
    double M = -INFINITY;
    for (int k0 = 0; k0 < N; k0 += WAVE)
      if (k0 + lane < N) M = fmax(M, (double)ld_dev(a.ws_logw + base + k0 + lane));
    M = wave_max_f64(M);
    const bool zero = !(M > -INFINITY);
    if (M == INFINITY || M != M) fl |= FLAG_NONFINITE;
    double Sw = 0.0, Sw2 = 0.0;
    int last_pos = -1;
    if (!zero) {
      for (int k0 = 0; k0 < N; k0 += WAVE) {
        const int k = k0 + lane;
        const double wk = k < N ? exp((double)ld_dev(a.ws_logw + base + k) - M) : 0.0;
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
      const int ii = k0 + lane;
      const float lwi = ii < N ? ld_dev(a.ws_logw + base + ii) : 0.0f;
      int hi;  // particle ii supplies the slots [lo, hi)
      if (do_res) {
        // slot k descends from the first i with C_i > (u + k) / N, so particle i
        // receives k in [ceil(N C_{i-1} - u), ceil(N C_i - u)); consecutive
        // ranges share their end points, so every slot is covered exactly once
        const double wi = ii < N ? exp((double)lwi - M) : 0.0;
        const double incl = wave_incl_scan_f64(wi, lane);
        double h = ceil((double)N * ((run + incl) / Sw) - u);
        if (ii >= last_pos) {  // the last particle with positive weight ends at N
          if (ii == last_pos && h < (double)N) fl |= FLAG_CDF_CLAMP;
          h = (double)N;
        }
        hi = (int)fmin(fmax(h, 0.0), (double)N);
        run += __shfl(incl, WAVE - 1, WAVE);
      } else {
        hi = ii + 1;
      }
      if (ii >= N) hi = N;
      const int prev = __shfl_up(hi, 1, WAVE);
      const int lo = lane == 0 ? carry : prev;
      hi = max(hi, lo);
      carry = __shfl(hi, WAVE - 1, WAVE);
      if (ii < N) {
        for (int k = lo; k < hi; k++) a.ancestors[base + k] = ii;
        a.logw_out[base + ii] = do_res ? 0.0f : lwi;
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
      st_dev(a.pcount + p * CSTRIDE, 0u);
    }
  }
  for (int off = 32; off >= 1; off >>= 1) fl |= __shfl_xor(fl, off, WAVE);
  if (lane == 0) raise_flags(a.s.flags, fl);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
// Workgroups of BLOCK threads the current device holds at once for `kernel`
// (queried once per device and kernel); the streaming grid is sized to it.
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

template <typename DT, bool VL>
static hipError_t launch_stream_t(const StreamArgs& a, hipStream_t s) {
  constexpr int PF = DT::VEC == 8 ? 2 : 1;  // tiles in flight beyond the one being reduced
  const void* k = reinterpret_cast<const void*>(&k_stream<DT, VL, PF>);
  const int resident = resident_blocks(k);
  if (resident <= 0) return hipErrorInvalidDevice;
  int64_t blocks = (a.total_tiles + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  if (blocks > resident) blocks = resident;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((k_stream<DT, VL, PF>), dim3((unsigned)blocks), dim3(BLOCK), 0, s, a);
  return hipGetLastError();
}

template <typename DT, bool VL>
static hipError_t launch_sd_t(const SdTailArgs& a, hipStream_t s) {
  hipError_t e = launch_stream_t<DT, VL>(a.s, s);
  if (e != hipSuccess) return e;
  const unsigned gx = (unsigned)((a.s.ntiles + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK);
  hipLaunchKernelGGL((k_sd_tail<DT, VL>), dim3(gx, (unsigned)a.s.ngroups), dim3(BLOCK), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sd(const SdTailArgs& a, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_sd_t<Bf16, true>(a, s) : launch_sd_t<Bf16, false>(a, s);
  return vec ? launch_sd_t<F32, true>(a, s) : launch_sd_t<F32, false>(a, s);
}

template <typename DT, bool VL>
static hipError_t launch_smc_t(const SmcTailArgs& a, hipStream_t s) {
  hipError_t e = launch_stream_t<DT, VL>(a.s, s);
  if (e != hipSuccess) return e;
  const unsigned g = (unsigned)((a.s.ngroups + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK);
  hipLaunchKernelGGL((k_smc_tail<DT, VL>), dim3(g), dim3(BLOCK), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_smc(const SmcTailArgs& a, bool bf16, bool vec, hipStream_t s) {
  if (bf16) return vec ? launch_smc_t<Bf16, true>(a, s) : launch_smc_t<Bf16, false>(a, s);
  return vec ? launch_smc_t<F32, true>(a, s) : launch_smc_t<F32, false>(a, s);
}

}  // namespace smcsd
