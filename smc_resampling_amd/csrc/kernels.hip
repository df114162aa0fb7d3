// kernels.hip -- HIP kernels (gfx950) of the verify-and-sample step.
//
// sd_verify, draft_sample and tree_verify launch two kernels on the caller's
// stream, smc_reweight_resample three.
//
// k_stream (every operation) reads every logit once.  The logit rows are
// taken group by group (a group is an SD sequence or an SMC particle: its
// target rows 0..K_b, then its draft rows 0..K_b-1), each row cut into
// segments of `seg` consecutive 2048-logit tiles; a unit is one (row,
// segment).  Wavefront w of W streams units [U w / W, U (w+1) / W) with the
// next tiles' loads in flight across unit, row and group boundaries, keeps
// per-lane running softmax statistics over a unit and stores the unit's
// (offset, sum of exponentials at that offset).  A unit's partial depends on its logits alone, so
// equal rows get bitwise-equal statistics however the work is spread.  The
// kernel holds nothing else, so it runs at high occupancy.
//
// k_sd_tail (sd_verify; "Faster LLM Inference via Sequential Monte Carlo",
// sec. 1; variable lengths as in "PACER", Methodik): one workgroup per
// sequence merges its partials into row statistics, tests
// u_j < p_j(x_j) / q_j(x_j) up to the first rejection n and draws the final
// token by inverse CDF: from p_{K_b} when n = K_b (tile located from the bonus
// row's partials, then searched), else from max(0, p_n - q_n) (every tile's
// mass, then the located tile searched).
//
// k_smc_tail (smc_reweight_resample; same page, sec. 2 steps 3-4): one
// workgroup per particle computes the log-weight increment
// sum_j log p_j(x_j) - log q_j(x_j) (and, for a power target, the bonus
// token's weight) and draws the (K+1)-th token.  k_smc_prompt, one to eight
// workgroups per prompt, then computes the Kish ESS, resamples systematically
// when it is below the threshold and gathers the page-table rows by ancestor
// (sec. 3).
//
// k_tree_tail (tree_verify): one workgroup per token tree walks it from the
// root.  k_draw_tail (draft_sample): one workgroup per row draws its token.
//
// No workgroup waits for, or hands data to, another: what a kernel needs from
// other workgroups was written by an earlier kernel, and the kernel boundary
// orders it.
#include <hip/hip_ext.h>

#include "device.h"
#include "launch.h"

namespace smcsd {

// Measurement knob, 0 in the library's build: see the streaming kernel's loads.
#ifndef SMCSD_TEMPORAL_ROWS
#define SMCSD_TEMPORAL_ROWS 0
#endif
// Measurement knob, 4 in the library's build: the most member workgroups a
// decision may be shared by (1: one workgroup per sequence or tree).
#ifndef SMCSD_MAX_MEMBERS
#define SMCSD_MAX_MEMBERS 4
#endif

// Phase timestamps of the decision kernels, for measurement builds only
// (-DSMCSD_PHASE_STAMPS=1; the library's build compiles every stamp away).
// Thread 0 of workgroup g < SMCSD_STAMP_WGS records, at its k-th event, the
// 100 MHz s_memrealtime clock and a code naming the phase that just ended
// (STAMP_* in launch.h); smcsd_phase_stamps copies them out.
#ifndef SMCSD_PHASE_STAMPS
#define SMCSD_PHASE_STAMPS 0
#endif
#if SMCSD_PHASE_STAMPS
__device__ unsigned long long g_stamps[SMCSD_STAMP_WGS * SMCSD_STAMP_EVENTS * 2];
__device__ __forceinline__ void stamp_wg(int64_t g, int k, unsigned code) {
  if (threadIdx.x == 0 && g < SMCSD_STAMP_WGS && k < SMCSD_STAMP_EVENTS) {
    const size_t i = ((size_t)g * SMCSD_STAMP_EVENTS + k) * 2;
    g_stamps[i] = __builtin_amdgcn_s_memrealtime();
    g_stamps[i + 1] = code;
  }
}
#else
__device__ __forceinline__ void stamp_wg(int64_t, int, unsigned) {}
#endif
__device__ __forceinline__ void stamp(int k, unsigned code) { stamp_wg(blockIdx.x, k, code); }

constexpr int MAXR = 2 * SMCSD_MAX_K + 1;  // rows per group
constexpr int MAX_TILES = 256;             // tiles per row (V <= 524288)

// ---------------------------------------------------------------------------
// status flags
// ---------------------------------------------------------------------------
__device__ __forceinline__ void raise_flags(uint32_t* flags, uint32_t bits) {
  if (flags && bits) atomicOr(flags, bits);
}
// ---------------------------------------------------------------------------
// groups
// ---------------------------------------------------------------------------
struct Group {
  int64_t d0;   // first draft row
  int kb;       // draft length
  int64_t fr0;  // first row in the group-major row order (= 2*d0 + g)
  bool ok;
};

__device__ __forceinline__ Group make_group(int64_t g, int64_t a, int64_t e, int K, int64_t rows_d) {
  Group G;
  G.d0 = a;
  G.kb = (int)(e - a);
  G.ok = a >= 0 && e >= a && e - a <= K && e <= rows_d;
  G.fr0 = 2 * a + g;
  return G;
}

__device__ __forceinline__ Group group_of(int64_t g, int K, const int32_t* __restrict__ offsets, int64_t rows_d) {
  if (!offsets) return make_group(g, g * K, (g + 1) * K, K, rows_d);
  return make_group(g, offsets[g], offsets[g + 1], K, rows_d);
}

// Logit row `rr` of group g (target rows 0..kb, then draft rows); null when
// it falls outside the buffers (malformed offsets).  In flat mode group g is
// target row g, and draft row g - rows_t past the target rows.
template <typename raw>
__device__ __forceinline__ const raw* group_row(const StepArgs& a, const Group& G, int64_t g, int64_t rr) {
  if (!G.ok || rr < 0 || rr > 2 * G.kb) return nullptr;
  if (rr <= G.kb) {
    const int64_t tr = G.d0 + g + rr;
    if (a.flat && tr >= a.rows_t) {
      const int64_t dr = tr - a.rows_t;
      return dr < a.rows_d ? static_cast<const raw*>(a.draft) + dr * a.V : nullptr;
    }
    return tr < a.rows_t ? static_cast<const raw*>(a.target) + tr * a.V : nullptr;
  }
  const int64_t dr = G.d0 + rr - G.kb - 1;
  return dr < a.rows_d ? static_cast<const raw*>(a.draft) + dr * a.V : nullptr;
}

// ---------------------------------------------------------------------------
// softmax partials
// ---------------------------------------------------------------------------
// Per-lane running statistics over a unit's tiles: s = sum 2^(z c - m) in the
// log2 domain, with the offset m never above the largest z c folded so far
// (so a row's sum is at least 1).
//
// lane_fold_tile_at_max folds a tile at the running maximum: m is the
// largest z c so far, and s is rescaled when it grows.
template <typename DT>
__device__ __forceinline__ void lane_fold_tile_at_max(const Raw<DT>& cur, float c, float& m, float& s) {
  // the values are unpacked from the raw tile where used (the raw registers
  // stay live for the whole fold; 32 unpacked values would not fit beside them)
  constexpr int CH = Raw<DT>::CHUNKS, VEC = DT::VEC;
  float w[VEC];
  float tm = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int ch = 0; ch < CH; ch++) {
    unpack<DT>(cur, ch, w);
#pragma unroll
    for (int k = 0; k < VEC; k++) {
      tm = fmaxf(tm, w[k]);
      nan |= w[k] != w[k];
    }
  }
  const float mn = fmaxf(m, tm * c);
  if (mn > -INFINITY) {
    float acc = s * __builtin_amdgcn_exp2f(m - mn);  // 0 while m is -inf (NaN stays NaN)
#pragma unroll
    for (int ch = 0; ch < CH; ch++) {
      unpack<DT>(cur, ch, w);
#pragma unroll
      for (int k = 0; k < VEC; k++) acc += __builtin_amdgcn_exp2f(fmaf(w[k], c, -mn));
    }
    s = acc;
    m = mn;
  } else if (nan) {
    // every value so far is -inf or NaN: keep a NaN visible
    s = __builtin_nanf("");
  }
}

// Hides from the compiler that a tile's raw registers still hold the bits a
// loop unpacked from them, so that the unpacked values are not kept live for a
// later loop (which unpacks again).
template <typename DT>
__device__ __forceinline__ void hide_bits(Raw<DT>& r) {
#pragma unroll
  for (int ch = 0; ch < Raw<DT>::CHUNKS; ch++) asm volatile("" : "+v"(r.q[ch]));
}

// lane_fold_tile keeps the offset where it is while every term stays at most
// kFoldCeil: the tile is folded at the current offset (unpack, fma, exp, add
// per logit: no maximum, no rescale), and the fold stands if the sum stays at
// most kFoldCeil.  A lane whose offset is still -inf (a unit's first tile)
// offsets at the largest value of its first chunk.  Otherwise (a value more
// than 64 above the offset in the log2 domain, a NaN or +inf, a first chunk of
// -inf) the tile is folded again at the running maximum.
constexpr float kFoldCeil = 18446744073709551616.0f;  // 2^64

template <typename DT>
__device__ __forceinline__ void lane_fold_tile(Raw<DT>& cur, float c, float& m, float& s) {
  constexpr int CH = Raw<DT>::CHUNKS, VEC = DT::VEC;
  float w[VEC];
  unpack<DT>(cur, 0, w);
  float m0 = w[0];
#pragma unroll
  for (int k = 1; k < VEC; k++) m0 = fmaxf(m0, w[k]);
  const float mo = m > -INFINITY ? m : m0 * c;
  float acc = s;  // 0, or NaN, while m is -inf
#pragma unroll
  for (int ch = 0; ch < CH; ch++) {
    if (ch) unpack<DT>(cur, ch, w);
#pragma unroll
    for (int k = 0; k < VEC; k++) acc += __builtin_amdgcn_exp2f(fmaf(w[k], c, -mo));
  }
  if (acc <= kFoldCeil) {  // false for NaN and +inf
    s = acc;
    m = mo;
  } else {
    // The second fold unpacks the tile again, so the first fold's unpacked
    // values die as they are used instead of staying live for this rare branch
    // (32 values per lane against the tile's 16 raw registers, which stay live
    // until the slot's next load anyway).
    hide_bits<DT>(cur);
    lane_fold_tile_at_max<DT>(cur, c, m, s);
  }
}

// Merge per-lane statistics (m2, s2) into (m, s).  A -inf offset contributes
// its sum times 0, so a NaN sum stays NaN.
__device__ __forceinline__ void lane_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn > -INFINITY) {
    s = s * (m > -INFINITY ? __builtin_amdgcn_exp2f(m - mn) : 0.0f) +
        s2 * (m2 > -INFINITY ? __builtin_amdgcn_exp2f(m2 - mn) : 0.0f);
    m = mn;
  } else {
    s = s + s2;
  }
}

// The wavefront's (MC, S) from per-lane (m, s): MC = the largest offset m,
// S = sum s 2^(m - MC).
// All -inf gives (-inf, 0); a NaN s stays NaN.
__device__ __forceinline__ float2 wave_partial(float m, float s) {
  const float M = wave_max_nonnan(m);  // m comes from fmaxf: never NaN
  const float sc = m > -INFINITY ? __builtin_amdgcn_exp2f(m - M) : 0.0f;
  return make_float2(M, wave_sum(s * sc));
}

// ---------------------------------------------------------------------------
// k_stream
// ---------------------------------------------------------------------------
// The group of the rows a wavefront streams.  With CSR offsets the wavefront
// keeps offsets[g0 + l] in lane l, so moving to the next group needs no load
// (a load inside the streaming loop would wait for every tile in flight).
// Indices are 32-bit (the planner rejects calls of more than INT32_MAX
// tiles, so every row, group and tile index fits): the streaming loop's
// scalar state then fits in scalar registers.
struct GroupCursor {
  int32_t g;
  int32_t d0, kb;  // the group's first draft row and draft length
  int32_t fr0;     // its first row in the group-major order
  int32_t fr1;     // one past its last row
  bool ok;
  int32_t g0;   // base of the offsets window
  int32_t win;  // offsets[g0 + lane]
};

// The group holding group-major row fr (largest g with 2*offsets[g] + g <=
// fr): each round probes 64 candidates at once.
__device__ __forceinline__ int64_t find_group_wave(int64_t fr, const StepArgs& a, int lane) {
  if (!a.offsets) return fr / (2 * a.K + 1);
  int64_t lo = 0, hi = a.ngroups;  // the answer lies in [lo, hi)
  while (hi - lo > 1) {
    const int64_t span = hi - lo;
    const int64_t p = span <= WAVE + 1 ? lo + 1 + lane : lo + (span * (lane + 1)) / (WAVE + 1);
    const bool live = p < hi;
    const bool le = live && 2 * (int64_t)a.offsets[p] + p <= fr;
    const uint64_t bal = __ballot(le);
    const int j = bal ? 63 - __builtin_clzll(bal) : -1;  // last probe at or below fr
    const int64_t pj = j >= 0 ? readlane_i64(p, j) : lo;
    const uint64_t above = __ballot(live && !le) & (j >= 0 ? ~((2ull << j) - 1) : ~0ull);
    const int64_t pk = above ? readlane_i64(p, __builtin_ctzll(above)) : hi;
    lo = uniform64(pj);
    hi = uniform64(pk);
  }
  return lo;
}

__device__ __forceinline__ void cursor_take(GroupCursor& cu, const Group& G) {
  cu.d0 = (int32_t)G.d0;
  cu.kb = G.kb;
  cu.ok = G.ok;
  // a malformed group (not ok) is never read; its row range only has to stay
  // finite, so that the cursor moves on
  cu.fr0 = G.ok ? (int32_t)G.fr0 : 0;
  cu.fr1 = G.ok ? (int32_t)(G.fr0 + 2 * (int64_t)G.kb + 1) : 0;
}

__device__ __forceinline__ void cursor_set(GroupCursor& cu, int32_t g, const StepArgs& a, int lane) {
  cu.g = g;
  if (!a.offsets) {
    cursor_take(cu, make_group(g, (int64_t)g * a.K, (int64_t)(g + 1) * a.K, a.K, a.rows_d));
    return;
  }
  int32_t o0, o1;
  if (g + 1 - cu.g0 >= WAVE || g < cu.g0) {  // refill the window
    cu.g0 = g;
    cu.win = a.offsets[min((int64_t)g + lane, a.ngroups)];
    // read it here: the wait for the load (and for every tile load issued
    // before it) then stays in this rare branch instead of following every
    // group change (the empty asm keeps the reads from being merged with the
    // other branch's)
    o0 = __builtin_amdgcn_readlane(cu.win, 0);
    o1 = __builtin_amdgcn_readlane(cu.win, 1);
    asm volatile("" ::"s"(o0), "s"(o1));
  } else {
    const int i = (int)(g - cu.g0);
    o0 = __builtin_amdgcn_readlane(cu.win, i);
    o1 = __builtin_amdgcn_readlane(cu.win, i + 1);
  }
  cursor_take(cu, make_group(g, o0, o1, a.K, a.rows_d));
}

// Row rr of the cursor's group (null outside the buffers).
template <typename raw>
__device__ __forceinline__ const raw* cursor_row(const StepArgs& a, const GroupCursor& cu, int32_t rr) {
  Group G;
  G.d0 = cu.d0;
  G.kb = cu.kb;
  G.fr0 = cu.fr0;
  G.ok = cu.ok;
  return group_row<raw>(a, G, cu.g, rr);
}

// TP: the call's segments span several tiles, so each group's bonus row also
// gets per-tile partials (with one-tile segments the segment partials are
// those already).  PW (SMC with a power target, whose groups are all 2K+1
// rows): each group's bonus row is reduced at its own scale cb, and also at
// the plain scale c into part1 (segment partials, group-major).
template <typename DT, bool VL, int NS, bool TP, bool PW>
__device__ __forceinline__ void stream_body(const StepArgs& a) {
  using raw = typename DT::raw;
  const int lane = threadIdx.x % WAVE;
  const int64_t w = (int64_t)blockIdx.x * WAVES_PER_BLOCK + wave_id();
  const int64_t W = (int64_t)gridDim.x * WAVES_PER_BLOCK;
  const int32_t u0 = (int32_t)(a.units * w / W), u1 = (int32_t)(a.units * (w + 1) / W);
  // the words the decision kernel after this one exchanges values through
  // start at 0 (plain stores: the kernel boundary orders them before it)
  for (int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x; i < a.xzn; i += (int64_t)gridDim.x * BLOCK) a.xz[i] = 0;
  if (u0 >= u1) return;
  const int nseg = a.nseg, seg = a.seg, ntiles = a.ntiles;
  const float c = a.c;
  uint32_t bad = 0;
  // load cursor: unit lu of row lfr, tile lt of [.., lte)
  int32_t lu = u0, lfr = u0 / nseg;
  int lsg = lu - lfr * nseg;
  int lt = lsg * seg, lte = min(ntiles, lt + seg);
  GroupCursor gc;
  gc.g0 = -WAVE;
  gc.win = 0;
  cursor_set(gc, (int32_t)find_group_wave(lfr, a, lane), a, lane);
  const raw* lrow = cursor_row<raw>(a, gc, lfr - gc.fr0);
  if (!lrow) bad = FLAG_BAD_INPUT;
  // tiles of a group's last target row (its bonus row) also get a partial of
  // their own, at tpart[lbon + tile]; lbon < 0 for every other row
  auto bonus_base = [&]() -> int32_t { return TP && lrow && lfr - gc.fr0 == gc.kb ? gc.g * ntiles : -1; };
  int32_t lbon = bonus_base();
  // Issues the loads of the next tile.  A row outside the buffers (malformed
  // offsets) is read as row 0 of the target, and its partials are not used.
  auto fetch = [&](int32_t& dst) {
#if SMCSD_TEMPORAL_ROWS > 0
    // build-time measurement knob: SD rows at the first draft positions
    // (target and draft row j < SMCSD_TEMPORAL_ROWS) loaded with the temporal
    // policy, so that a rejection's re-read might find them cached
    const int32_t rr = lfr - gc.fr0;
    const bool keep = !a.flat && a.cb == a.c &&
                      ((rr < SMCSD_TEMPORAL_ROWS) || (rr > gc.kb && rr <= gc.kb + SMCSD_TEMPORAL_ROWS));
    Raw<DT> x;
    if (keep) x = load_raw<DT, VL, 0>(lrow ? lrow : static_cast<const raw*>(a.target), a.V, lt, lane);
    else x = load_raw<DT, VL>(lrow ? lrow : static_cast<const raw*>(a.target), a.V, lt, lane);
#else
    const Raw<DT> x = load_raw<DT, VL>(lrow ? lrow : static_cast<const raw*>(a.target), a.V, lt, lane);
#endif
    dst = lbon < 0 ? -1 : lbon + lt;
    if (++lt == lte) {
      if (++lu < u1) {
        if (++lsg == nseg) {
          lsg = 0;
          lfr++;
          if (lfr >= gc.fr1) cursor_set(gc, gc.g + 1, a, lane);
          lrow = cursor_row<raw>(a, gc, lfr - gc.fr0);
          if (!lrow) bad = FLAG_BAD_INPUT;
          lbon = bonus_base();
        }
        lt = lsg * seg;
        lte = min(ntiles, lt + seg);
      }
    }
    return x;
  };
  // tiles in [u0, u1): seg per unit, fewer in a row's last segment
  const int last_seg = ntiles - (nseg - 1) * seg;
  const int32_t T = (u1 - u0) * seg - (u1 / nseg - u0 / nseg) * (seg - last_seg);
  // reduce cursor: tile ct of [.., cte) of the current unit.  Finished units'
  // partials wait in lanes (unit pbase + l in lane l) and are stored 64 at a
  // time: a store is a memory operation the loads' wait counter also counts.
  int csg = u0 % nseg;
  int ct = csg * seg, cte = min(ntiles, ct + seg);
  // the scale of the row being reduced: c, or cb for a group's bonus row when
  // the call gives that row its own (SMC with a power target, whose groups are
  // all 2K+1 rows: the row within its group is the row index modulo 2K+1)
  const bool split = PW || a.cb != c;
  const int grows = 2 * a.K + 1;
  int crr = split ? (u0 / nseg) % grows : 0;
  float cc = split && crr == a.K ? a.cb : c;
  float m = -INFINITY, s = 0.0f;
  // PW: the group of the row being reduced, and the bonus row's unit at scale c
  int32_t cgrp = PW ? (u0 / nseg) / grows : 0;
  float m1 = -INFINITY, s1 = 0.0f;
  float2 pb = make_float2(0.0f, 0.0f);
  int32_t pbase = u0;
  int pn = 0;
  auto reduce = [&](Raw<DT>& x, int32_t dst) {
    mask_tail<DT>(x, a.V, ct, lane);
    // a bonus-row tile is folded on its own first, then into the unit's statistics
    const float pm = m, ps = s;
    if (TP && dst >= 0) {
      m = -INFINITY;
      s = 0.0f;
    }
    lane_fold_tile<DT>(x, cc, m, s);
    if constexpr (PW) {
      if (crr == a.K) lane_fold_tile<DT>(x, c, m1, s1);
    }
    if (TP && dst >= 0) {
      const float2 tp = wave_partial(m, s);
      if (lane == 0) a.tpart[dst] = tp;
      lane_merge(m, s, pm, ps);
    }
    if (++ct == cte) {
      const float2 pt = wave_partial(m, s);
      if (lane == pn) pb = pt;
      if (++pn == WAVE) {
        a.part[pbase + lane] = pb;
        pbase += WAVE;
        pn = 0;
      }
      m = -INFINITY;
      s = 0.0f;
      if constexpr (PW) {
        if (crr == a.K) {
          const float2 p1 = wave_partial(m1, s1);
          if (lane == 0) a.part1[cgrp * nseg + csg] = p1;
          m1 = -INFINITY;
          s1 = 0.0f;
        }
      }
      if (++csg == nseg) {
        csg = 0;
        if (split) {
          if (++crr == grows) {
            crr = 0;
            if constexpr (PW) cgrp++;
          }
          cc = crr == a.K ? a.cb : c;
        }
      }
      ct = csg * seg;
      cte = min(ntiles, ct + seg);
    }
  };
  // NS tiles in flight.  Slot i always lives in the same registers (a
  // rotating copy would wait for loads still in flight), and in the main loop
  // every slot is refilled unconditionally, so a reduction waits only for its
  // own tile.
  Raw<DT> q[NS];
  int32_t qd[NS];
  if (T >= 2 * NS) {
#pragma unroll
    for (int i = 0; i < NS; i++) q[i] = fetch(qd[i]);
    int32_t left = T;
    do {
#pragma unroll
      for (int i = 0; i < NS; i++) {
        reduce(q[i], qd[i]);
        q[i] = fetch(qd[i]);
      }
      left -= NS;
    } while (left >= 2 * NS);
    // NS <= left < 2 NS: the slots hold the next NS tiles, left - NS remain
    const int more = (int)(left - NS);
#pragma unroll
    for (int i = 0; i < NS; i++) {
      reduce(q[i], qd[i]);
      if (i < more) q[i] = fetch(qd[i]);
    }
#pragma unroll
    for (int i = 0; i < NS; i++)
      if (i < more) reduce(q[i], qd[i]);
  } else {
    // fewer than 2 NS tiles
    const int t = (int)T;
#pragma unroll
    for (int i = 0; i < NS; i++)
      if (i < t) q[i] = fetch(qd[i]);
#pragma unroll
    for (int i = 0; i < NS; i++) {
      if (i < t) {
        reduce(q[i], qd[i]);
        if (NS + i < t) q[i] = fetch(qd[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NS; i++)
      if (NS + i < t) reduce(q[i], qd[i]);
  }
  if (lane < pn) a.part[pbase + lane] = pb;
  if (lane == 0) raise_flags(a.flags, bad);
}

// NS tiles in flight per wavefront, at the occupancy the registers allow.
template <typename DT, bool VL, int NS, bool TP, bool PW>
__global__ __launch_bounds__(BLOCK) void k_stream(StepArgs a) {
  stream_body<DT, VL, NS, TP, PW>(a);
}

// Calls with one-tile segments (a few tiles per wavefront; bf16 rows that
// take 16-byte loads, the element loads would spill here): two tiles
// in flight at six wavefronts per SIMD, so that more wavefronts' reductions
// overlap the loads (measured 8-9 % faster on 37 MB calls, 1.6 % slower on a
// 10.6 GB call, where the deeper pipeline wins).
template <typename DT, bool VL>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(6, 6))) void k_stream_wide(StepArgs a) {
  stream_body<DT, VL, 2, false, false>(a);
}

// ---------------------------------------------------------------------------
// tails: workgroup-shared state
// ---------------------------------------------------------------------------
struct TailLds {
  // per row of the group (and, for a power target, the bonus row at the
  // plain scale as row 2K+1)
  float M[MAXR + 1];         // row offset of z c (log2 domain; at most the row maximum, within 64 of it)
  double S[MAXR + 1];        // row sum of 2^(z c - M)
  double lS[MAXR + 1];       // log S
  float z[2 * SMCSD_MAX_K];  // logits of the draft tokens: target rows, then draft rows
  float u[SMCSD_MAX_K];      // accept uniforms
  int xok[SMCSD_MAX_K];      // draft token inside [0, V)
  float2 P[MAX_TILES];       // segment partials of the row a draw uses
  double W[MAX_TILES];       // per-tile masses of a draw
  float Tm[MAX_TILES];       // per-tile log2 maxima of a draw
  double before, target;
  int sel, clamp, n, y;
  uint32_t fl;
};
struct PromptLds {
  float lw[SMCSD_MAX_N];
  int hi[SMCSD_MAX_N];   // particle i supplies the slots [hi[i-1], hi[i])
  int anc[SMCSD_MAX_N];
};

__device__ __forceinline__ RowStat stat_of(const TailLds& L, int r) {
  RowStat rs;
  rs.M = L.M[r];
  rs.S = L.S[r];
  rs.lS = L.lS[r];
  rs.ok = (rs.M > -INFINITY) && (rs.M < INFINITY) && (rs.S >= 0.5) && (rs.S < INFINITY);
  return rs;
}

// Fold partial (pm, ps) into running statistics (m, s): log2-domain offsets,
// fp64 sums.  The rescaling factor 2^(smaller - larger) <= 1 comes from the
// fp32 exponential (relative error about 1e-7); a factor of a -inf offset is 0
// and keeps a NaN sum NaN.
__device__ __forceinline__ void fold(float& m, double& s, float pm, double ps) {
  if (pm > m) {
    s = s * (double)(m > -INFINITY ? __builtin_amdgcn_exp2f(m - pm) : 0.0f) + ps;
    m = pm;
  } else {
    s += ps * (double)(pm > -INFINITY ? __builtin_amdgcn_exp2f(pm - m) : 0.0f);
  }
}

// Row statistics of rows [0, R) of one group from its segment partials (row
// r's at part[r * nseg + k], written by the previous kernel) into L.M / L.S /
// L.lS, and with `extra` one more row, row R, whose nseg partials lie at extra
// (further on in the same workspace).  Whole workgroup, 16 threads per row,
// fixed combination order, so equal rows get equal statistics.
template <int CTRL>
__device__ __forceinline__ void fold_dpp(float& m, double& s) {
  fold(m, s, dpp_f32m<CTRL>(m), dpp_f64<CTRL>(s));
}

constexpr int DPP_WAVE_SHR1 = 0x138;
constexpr int DPP_QUAD_XOR1 = 0xB1, DPP_QUAD_XOR2 = 0x4E, DPP_ROW_MIRROR = 0x140, DPP_ROW_HALF_MIRROR = 0x141;

template <int NT>
__device__ __forceinline__ void merge_rows_to(const float2* __restrict__ part, int R, int nseg, float* Mo,
                                              double* So, double* lSo, const float2* extra = nullptr) {
  constexpr int TPR = 16;  // threads per row: one DPP row
  const int sub = threadIdx.x & (TPR - 1);
  // the group's partials (and the extra row's) through one buffer resource:
  // 32-bit offsets
  const int xoff = extra ? (int)(extra - part) : 0;  // in partials
  const int RR = extra ? R + 1 : R;
  const __amdgpu_buffer_rsrc_t rs =
      buffer_over(part, (uint32_t)((extra ? xoff + nseg : R * nseg) * (int)sizeof(float2)));
  for (int r0 = 0; r0 < RR; r0 += NT / TPR) {
    const int r = r0 + (int)threadIdx.x / TPR;
    float m = -INFINITY;
    double s = 0.0;
    if (r < RR) {
      // at most MAX_TILES / 16 = 16 partials per thread, in batches of GB
      // loads in flight (8, or 4 in the smaller workgroups that keep fewer
      // registers; indices past the row clamped, so the loads need no branch;
      // straight-line code, so loads issued before the call are not waited
      // for here), folded in ascending k
      constexpr int GB = NT >= 1024 ? 8 : 4;
      constexpr int NB = MAX_TILES / (GB * TPR);
      const int row0 = r < R ? r * nseg : xoff;
#pragma unroll
      for (int h = 0; h < NB; h++) {
        const int k0 = sub + h * GB * TPR;
        if (h > 0 && nseg <= h * GB * TPR) break;
        u32x2 v[GB];
#pragma unroll
        for (int j = 0; j < GB; j++)
          v[j] = __builtin_amdgcn_raw_buffer_load_b64(rs, (row0 + min(k0 + j * TPR, nseg - 1)) * 8, 0, 0);
#pragma unroll
        for (int j = 0; j < GB; j++)
          if (k0 + j * TPR < nseg) fold(m, s, __uint_as_float(v[j][0]), (double)__uint_as_float(v[j][1]));
      }
    }
    // lanes i and 15-i, then 7-i inside each half, then the quads: lane 0 of
    // the row ends up holding all 16 (the same order for every row)
    fold_dpp<DPP_ROW_MIRROR>(m, s);
    fold_dpp<DPP_ROW_HALF_MIRROR>(m, s);
    fold_dpp<DPP_QUAD_XOR1>(m, s);
    fold_dpp<DPP_QUAD_XOR2>(m, s);
    if (r < RR && sub == 0) {
      Mo[r] = m;
      So[r] = s;
      lSo[r] = log(s);
    }
  }
}
template <int NT>
__device__ __forceinline__ void merge_rows(const float2* __restrict__ part, int R, int nseg, TailLds& L) {
  merge_rows_to<NT>(part, R, nseg, L.M, L.S, L.lS);
}

// Partials of the bonus row kb of group g (first row fr0): its tile partials
// when the call keeps them, else its segment partials.  *np entries of *per
// tiles each.
__device__ __forceinline__ const float2* bonus_partials(const StepArgs& s, int64_t fr0, int64_t g, int kb, int* np,
                                                        int* per) {
  *np = s.tp ? s.ntiles : s.nseg;
  *per = s.tp ? 1 : s.seg;
  return s.tp ? s.tpart + g * s.ntiles : s.part + (fr0 + kb) * s.nseg;
}

// The n partials at src into L.P.  Whole workgroup.
template <int NT>
__device__ __forceinline__ void stage_partials(const float2* __restrict__ src, int n, TailLds& L) {
  for (int k = threadIdx.x; k < n; k += NT) L.P[k] = src[k];
}

// ---------------------------------------------------------------------------
// ordered searches
// ---------------------------------------------------------------------------
// Over weights W_k (k < n <= 256) in ascending order: the first k with
// base + (inclusive prefix) > target(total), and the prefix before it; -1
// (with the last k of positive weight in *last) when there is none.  One
// wavefront.
template <typename WFN, typename TFN>
__device__ __forceinline__ int locate(int n, WFN weight, double base, TFN target_of, int lane, double* before,
                                      double* target_out, int* last) {
  constexpr int CH = MAX_TILES / WAVE;
  double incl[CH], W[CH];
  double run = base;
  int lastk = -1;
#pragma unroll
  for (int k = 0; k < CH; k++) {
    W[k] = 0.0;
    incl[k] = run;
    if (k * WAVE < n) {
      const int t = k * WAVE + lane;
      W[k] = t < n ? weight(t) : 0.0;
      incl[k] = run + wave_incl_scan_f64(W[k], lane);
      run = readlane_f64(incl[k], WAVE - 1);
      const uint64_t pos = __ballot(W[k] > 0.0);
      if (pos) lastk = k * WAVE + 63 - __builtin_clzll(pos);
    }
  }
  const double target = target_of(run - base);
  *target_out = target;
  *last = lastk;
#pragma unroll
  for (int k = 0; k < CH; k++) {
    if (k * WAVE < n) {
      const uint64_t bal = __ballot(incl[k] > target && k * WAVE + lane < n);
      if (bal) {
        const int src = __builtin_ctzll(bal);
        *before = readlane_f64(incl[k] - W[k], src);
        return k * WAVE + src;
      }
    }
  }
  *before = run;
  return -1;
}

// Softmax partial (MC, S) of one tile held in registers, formed like the
// streaming partials.
template <typename DT>
__device__ __forceinline__ float2 tile_partial_of(const Raw<DT>& r, float c) {
  float m = -INFINITY, s = 0.0f;
  lane_fold_tile_at_max<DT>(r, c, m, s);
  return wave_partial(m, s);
}

struct NoIdleWork {
  __device__ void operator()() const {}
};

// Inverse-CDF draw from softmax(z c) of `row` (row offset M, log2 domain)
// with uniform u.  L.P holds np partials of the row, each over `per` tiles (a
// bonus row's own tile partials, or segment partials).  Whole workgroup;
// every thread gets the token.  While wavefront 0 reloads and searches the
// located tile, the other wavefronts run `idle` (memory operations it leaves
// in flight do not hold up the closing barrier, which orders LDS only).
template <typename DT, bool VL, int NW = WAVES_PER_BLOCK, typename Idle = NoIdleWork>
__device__ int draw_softmax(const typename DT::raw* __restrict__ row, const StepArgs& a, float c, float M, double u,
                            int np, int per, TailLds& L, uint32_t& fl, Idle idle = Idle()) {
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  // 1. the segment
  if (wave == 0) {
    auto wt = [&](int k) -> double {
      const float2 p = L.P[k];
      return p.x > -INFINITY ? (double)p.y * exp2((double)p.x - (double)M) : 0.0;
    };
    double before = 0.0, target = 0.0;
    int last = -1;
    const int k = locate(np, wt, 0.0, [&](double tot) { return u * tot; }, lane, &before, &target, &last);
    if (lane == 0) {
      L.sel = k >= 0 ? k : (last >= 0 ? last : np - 1);
      L.clamp = k < 0;
      L.before = before;
      L.target = target;
    }
  }
  __syncthreads();
  const int sg = L.sel;
  const int tb = sg * per, te = min(a.ntiles, tb + per);
  int tt;
  double before_t;
  float mt;
  bool clamp = L.clamp;
  if (te - tb == 1) {
    tt = tb;
    before_t = L.before;
    mt = L.P[sg].x;
  } else {
    // 2. the tile inside the segment
    for (int t = tb + wave; t < te; t += NW) {
      const Raw<DT> r = load_tile<DT, VL>(row, a.V, t, lane);
      const float2 pt = tile_partial_of<DT>(r, c);
      if (lane == 0) {
        L.Tm[t - tb] = pt.x;
        L.W[t - tb] = pt.x > -INFINITY ? (double)pt.y * exp2((double)pt.x - (double)M) : 0.0;
      }
    }
    __syncthreads();
    if (wave == 0) {
      auto wt = [&](int k) -> double { return L.W[k]; };
      double before = 0.0, target = 0.0;
      int last = -1;
      const double tgt = clamp ? INFINITY : L.target;
      const int k = locate(te - tb, wt, L.before, [&](double) { return tgt; }, lane, &before, &target, &last);
      if (lane == 0) {
        L.sel = tb + (k >= 0 ? k : (last >= 0 ? last : te - tb - 1));
        L.clamp = k < 0;
        L.before = before;
      }
    }
    __syncthreads();
    tt = L.sel;
    clamp = L.clamp;
    before_t = L.before;
    mt = L.Tm[tt - tb];
  }
  // 3. the token inside the tile
  if (wave == 0) {
    const Raw<DT> raw = load_tile<DT, VL>(row, a.V, tt, lane);
    auto wfn = [&](int ch, float (&w)[DT::VEC]) {
      unpack<DT>(raw, ch, w);
#pragma unroll
      for (int k = 0; k < DT::VEC; k++) w[k] = __builtin_amdgcn_exp2f(fmaf(w[k], c, -mt));
    };
    int last_pos = -1;
    const double tscale = exp2((double)mt - (double)M);
    const float tgt = clamp ? INFINITY : (float)((L.target - before_t) / tscale);
    int idx = tile_search<DT>(wfn, tgt, lane, &last_pos);
    if (idx < 0) {
      fl |= FLAG_CDF_CLAMP;
      idx = last_pos >= 0 ? last_pos : 0;
    }
    if (lane == 0) L.y = tt * TILE + idx;
  } else {
    idle();
  }
  lds_barrier();
  return L.y;
}

// Residual weights max(0, p - q) of one tile of a (target, draft) row pair,
// p = 2^(z_t c - At), q = 2^(z_d c - Ad), with At = Mt + log2 S_t and
// Ad = Md + log2 S_d (the normalisation folded into the exponent).  p and q
// come out of the same operations, so equal rows give p - q = 0 exactly.
template <typename DT>
__device__ __forceinline__ void residual_weights(const Raw<DT>& rt, const Raw<DT>& rd, float At, float Ad, float c,
                                                 float (&r)[PER_LANE]) {
#pragma unroll
  for (int ch = 0; ch < Raw<DT>::CHUNKS; ch++) {
    float vt[DT::VEC], vd[DT::VEC];
    unpack<DT>(rt, ch, vt);
    unpack<DT>(rd, ch, vd);
#pragma unroll
    for (int k = 0; k < DT::VEC; k++) {
      const float p = __builtin_amdgcn_exp2f(fmaf(vt[k], c, -At));
      const float q = __builtin_amdgcn_exp2f(fmaf(vd[k], c, -Ad));
      // p, q <= 1, so max(p - q, 0) is p - q clamped to [0, 1]: the
      // subtraction's own output clamp
      r[ch * DT::VEC + k] = __builtin_amdgcn_fmed3f(p - q, 0.0f, 1.0f);
    }
  }
}

// the log2-domain normalisation M + log2 S of a row
__device__ __forceinline__ float log2_norm(const RowStat& rs) {
  return (float)((double)rs.M + rs.lS * 1.4426950408889634);
}

// ---------------------------------------------------------------------------
// tails: per-group inputs
// ---------------------------------------------------------------------------
// The token work of a workgroup of NT threads runs on its highest threads
// (slot NT - 1 - threadIdx.x), which the statistics merge (on the lowest
// threads) leaves idle: the two dependent round trips of the token logits
// (token, then its logit) overlap the merge's round trip and fold.
template <int NT>
__device__ __forceinline__ int token_slot() {
  return NT - 1 - (int)threadIdx.x;
}

// Draft token of this thread's row (slots t < 2 kb: target row t, then draft
// row t - kb, both with token x_{t mod kb}).
template <int NT>
__device__ __forceinline__ int32_t token_of(const StepArgs& a, const Group& G) {
  const int tid = token_slot<NT>(), kb = G.kb;
  return tid < 2 * kb ? a.tokens[G.d0 + (tid < kb ? tid : tid - kb)] : 0;
}

// Logit of this thread's draft token and whether the token lies in [0, V).
template <typename DT, int NT>
__device__ __forceinline__ float token_logit(const StepArgs& a, const Group& G, int64_t g, int32_t x, int* ok) {
  using raw = typename DT::raw;
  const int tid = token_slot<NT>(), kb = G.kb;
  *ok = 1;
  if (tid >= 2 * kb) return 0.0f;
  *ok = x >= 0 && x < a.V;
  const raw* row = group_row<raw>(a, G, g, tid < kb ? tid : tid + 1);
  return *ok && row ? DT::to_f32(row[x]) : 0.0f;
}

template <int NT>
__device__ __forceinline__ void store_tokens(float z, int ok, float u, int kb, TailLds& L) {
  const int tid = token_slot<NT>();
  if (tid < 2 * kb) {
    L.z[tid] = z;
    if (tid < kb) {
      L.u[tid] = u;
      L.xok[tid] = ok;
    }
  }
}

// OR of a per-thread value across the workgroup into L.fl (after a barrier).
__device__ __forceinline__ void or_flags(uint32_t v, TailLds& L) {
  v = wave_or_flags(v);
  if ((threadIdx.x % WAVE) == 0 && v) atomicOr(&L.fl, v);
}

// ---------------------------------------------------------------------------
// k_sd_tail: one workgroup of SD_WAVES wavefronts per sequence
// ---------------------------------------------------------------------------
constexpr int SD_WAVES = 16;
constexpr int SD_BLOCK = SD_WAVES * WAVE;

template <typename DT, bool VL>
__global__ __launch_bounds__(SD_BLOCK) void k_sd_tail(SdArgs a) {
  using raw = typename DT::raw;
  __shared__ TailLds L;
  const StepArgs& s = a.s;
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  // workgroup -> (sequence b, member k of S), as for token trees: the S
  // members of a sequence are 8 workgroup indices apart (one L2 when
  // workgroups are dealt to the 8 XCDs in turn), each decides the whole
  // sequence alike, and they share the residual pass, member k weighing the
  // tiles t = k (mod S) and reading the others' masses from their words.
  const int S = a.split;
  int64_t b = blockIdx.x;
  int k = 0;
  if (S > 1) {
    const int x = (int)blockIdx.x % 8, r = (int)blockIdx.x / 8;
    k = r % S;
    b = x + 8 * (r / S);
    if (b >= s.ngroups) return;
  }
  const int ntiles = s.ntiles;
  const Group G = group_of(b, s.K, s.offsets, s.rows_d);
  int ev = 0;
  auto sstamp = [&](unsigned code) {
    if (k == 0) stamp_wg(b, ev, code);
    ev++;
  };
  sstamp(0);
  if (s.offsets && threadIdx.x == 0) {
    uint32_t bad = G.ok ? 0u : FLAG_BAD_INPUT;
    if (b == 0 && s.offsets[0] != 0) bad = FLAG_BAD_INPUT;
    if (b == s.ngroups - 1 && s.offsets[s.ngroups] != s.rows_d) bad = FLAG_BAD_INPUT;
    raise_flags(s.flags, bad);
  }
  if (!G.ok) return;  // malformed CSR offsets: nothing of this sequence is read
  const int kb = G.kb;
  const int64_t t0 = G.d0 + b;
  const float2* pg = s.part + G.fr0 * s.nseg;
  if (threadIdx.x == 0) L.fl = 0;
  const int32_t xt = token_of<SD_BLOCK>(s, G);
  const int slot = token_slot<SD_BLOCK>();
  const float uj = slot < kb ? a.uniforms[t0 + slot] : 0.0f;
  const float ufin = a.uniforms[t0 + kb];
  // the merge runs on the lowest threads while the highest ones wait for the
  // tokens, then for their logits
  merge_rows<SD_BLOCK>(pg, 2 * kb + 1, s.nseg, L);
  int bnp, bper;
  const float2* bp = bonus_partials(s, G.fr0, b, kb, &bnp, &bper);
  stage_partials<SD_BLOCK>(bp, bnp, L);
  int ok = 1;
  const float z = token_logit<DT, SD_BLOCK>(s, G, b, xt, &ok);
  store_tokens<SD_BLOCK>(z, ok, uj, kb, L);
  __syncthreads();
  sstamp(STAMP_SD_MERGED);
  uint32_t fl = 0;
  // accept test up to the first rejection
  if (wave == 0) {
    int n = kb;
    for (int j0 = 0; j0 < kb; j0 += WAVE) {
      const int j = j0 + lane;
      bool reject = false;
      if (j < kb) {
        const RowStat st = stat_of(L, j), sd = stat_of(L, kb + 1 + j);
        if (!st.ok || !sd.ok) fl |= FLAG_NONFINITE;
        if (!L.xok[j]) {
          fl |= FLAG_BAD_INPUT;
          reject = true;
        } else {
          // rho = p/q from the fp64 log difference; the fp32 exponential
          // keeps its relative error near 1e-6
          const double d = log_prob(L.z[j], st, s.c) - log_prob(L.z[kb + j], sd, s.c);
          const double rho = (double)__builtin_amdgcn_exp2f((float)(d * 1.4426950408889634));
          reject = !((double)L.u[j] < rho);
        }
      }
      const uint64_t bal = __ballot(reject);
      if (bal && n == kb) n = j0 + __builtin_ctzll(bal);
    }
    if (lane == 0) L.n = n;
  }
  __syncthreads();
  sstamp(STAMP_SD_TESTED);
  const int n = L.n;
  const raw* trow = group_row<raw>(s, G, b, n);
  int y = 0;
  int owner = 0;  // the member that draws the final token
  if (n == kb) {
    // every draft accepted: the bonus token from p_{K_b}, drawn by member 0
    const RowStat sk = stat_of(L, kb);
    if (!sk.ok) fl |= FLAG_NONFINITE;
    if (k == 0) y = draw_softmax<DT, VL, SD_WAVES>(trow, s, s.c, sk.M, (double)ufin, bnp, bper, L, fl);
    sstamp(STAMP_SD_BONUS_DRAWN);
  } else {
    // residual max(0, p_n - q_n): each wavefront weighs its tiles and keeps
    // the weights of the last one in registers for the search
    const raw* drow = group_row<raw>(s, G, b, kb + 1 + n);
    const RowStat st = stat_of(L, n), sd = stat_of(L, kb + 1 + n);
    const float At = log2_norm(st), Ad = log2_norm(sd);
    float w[PER_LANE];
    int held = -1;
    uint64_t* xw = a.xchg + b * ntiles;  // this sequence's words (tag 1)
    for (int t = k + S * wave; t < ntiles; t += S * SD_WAVES) {
      const Raw<DT> rt = load_tile<DT, VL>(trow, s.V, t, lane);
      const Raw<DT> rd = load_tile<DT, VL>(drow, s.V, t, lane);
      residual_weights<DT>(rt, rd, At, Ad, s.c, w);
      held = t;
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < PER_LANE; e++) m += w[e];
      m = wave_sum(m);
      if (lane == 0) {
        L.W[t] = (double)m;
        if (S > 1) tagged_put(xw + t, 1u, m);
      }
    }
    if (S > 1) {
      // the other members' tile masses
      for (int t = threadIdx.x; t < ntiles; t += SD_BLOCK) {
        if (t % S == k) continue;
        float v = 0.0f;
        if (!tagged_get(xw + t, 1u, &v)) fl |= FLAG_WAIT_EXPIRED;  // outputs unspecified
        L.W[t] = (double)v;
      }
    }
    __syncthreads();
    sstamp(STAMP_SD_RESIDUAL_PASS);
    if (wave == 0) {
      auto wt = [&](int k) -> double { return L.W[k]; };
      double before = 0.0, target = 0.0, total = 0.0;
      int last = -1;
      const int k = locate(
          ntiles, wt, 0.0,
          [&](double tot) {
            total = tot;
            return (double)ufin * tot;
          },
          lane, &before, &target, &last);
      if (lane == 0) {
        L.sel = total > 0.0 ? (k >= 0 ? k : last) : -1;
        L.clamp = k < 0;
        L.target = target - before;  // the target inside the located tile
      }
    }
    __syncthreads();
    sstamp(STAMP_SD_LOCATED);
    const int tt = L.sel;
    if (tt >= 0) {
      // the wavefront that weighed tile tt draws inside it
      owner = tt % S;
      if (k == owner && wave == (tt / S) % SD_WAVES) {
        if (held != tt) {
          const Raw<DT> rt = load_tile<DT, VL>(trow, s.V, tt, lane);
          const Raw<DT> rd = load_tile<DT, VL>(drow, s.V, tt, lane);
          residual_weights<DT>(rt, rd, At, Ad, s.c, w);
        }
        auto wfn = [&](int ch, float (&x)[DT::VEC]) {
#pragma unroll
          for (int k = 0; k < DT::VEC; k++) x[k] = w[ch * DT::VEC + k];
        };
        int last_pos = -1;
        int idx = tile_search<DT>(wfn, L.clamp ? INFINITY : (float)L.target, lane, &last_pos);
        if (idx < 0) {
          fl |= FLAG_CDF_CLAMP;
          idx = last_pos >= 0 ? last_pos : 0;
        }
        if (lane == 0) L.y = tt * TILE + idx;
      }
      __syncthreads();
      sstamp(STAMP_SD_RESIDUAL_DRAWN);
      y = L.y;
    } else {
      // p_n and q_n agree to rounding: draw from p_n with the same uniform
      // (member 0)
      fl |= FLAG_ZERO_RESIDUAL;
      if (k == 0) {
        stage_partials<SD_BLOCK>(pg + (int64_t)n * s.nseg, s.nseg, L);
        __syncthreads();
        y = draw_softmax<DT, VL, SD_WAVES>(trow, s, s.c, st.M, (double)ufin, s.nseg, s.seg, L, fl);
      }
      sstamp(STAMP_SD_FALLBACK_DRAWN);
    }
  }
  or_flags(fl, L);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (k == 0 && a.num_accepted) a.num_accepted[b] = n;  // absent for a plain draw (no draft tokens)
    if (k == owner) a.final_token[b] = y;
    raise_flags(s.flags, L.fl);
  }
}

// ---------------------------------------------------------------------------
// k_draw_tail: the final draw alone, when no sequence has draft tokens (fixed
// K = 0: every group is one row and n = K_b = 0).  The same merge and the same
// draw as k_sd_tail, at a quarter of its threads, so that thousands of rows
// (one draft position of many particles) run as resident small workgroups.
// ---------------------------------------------------------------------------
template <typename DT, bool VL>
__global__ __launch_bounds__(BLOCK, VL ? 8 : 1) void k_draw_tail(SdArgs a) {
  using raw = typename DT::raw;
  __shared__ TailLds L;
  const StepArgs& s = a.s;
  const int64_t b = blockIdx.x;
  const Group G = group_of(b, 0, nullptr, 0);
  if (threadIdx.x == 0) L.fl = 0;
  const float u = a.uniforms[b];
  merge_rows<BLOCK>(s.part + G.fr0 * s.nseg, 1, s.nseg, L);
  int bnp, bper;
  const float2* bp = bonus_partials(s, G.fr0, b, 0, &bnp, &bper);
  stage_partials<BLOCK>(bp, bnp, L);
  __syncthreads();
  uint32_t fl = 0;
  const RowStat sk = stat_of(L, 0);
  if (!sk.ok) fl |= FLAG_NONFINITE;
  const int y = draw_softmax<DT, VL>(group_row<raw>(s, G, b, 0), s, s.c, sk.M, (double)u, bnp, bper, L, fl);
  or_flags(fl, L);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (a.num_accepted) a.num_accepted[b] = 0;
    a.final_token[b] = y;
    raise_flags(s.flags, L.fl);
  }
}

// ---------------------------------------------------------------------------
// k_tree_tail: one workgroup of TREE_WAVES wavefronts per token tree
// ("Faster LLM Inference via Sequential Monte Carlo", sec. 4: tree-based SD;
// multi-draft speculative sampling over the tree).  The workgroup merges the
// statistics of every target and draft row of the tree and gathers each
// node's token logits in its parent's rows, then walks from the root: at
// node u, child c is accepted iff u_c < r(x_c) / q_u(x_c) with r the running
// distribution (p_u, then max(0, r - q_u) / Z after each rejected child).  A
// rejection costs one pass of the whole workgroup over u's row pair: the
// first rebuilds max(0, p_u - q_u) elementwise, a later one continues from
// the previous pass's weights (held in LDS where they fit, else rebuilt from
// p_u and q_u with the masses Z of the earlier rejections), and the tile
// masses of max(0, r - q_u) give the new Z.  The walk ends at a leaf (bonus
// draw from p_leaf, as in sd_verify) or when every child of u is rejected
// (inverse-CDF draw from the last pass's weights: the tile is located from
// the pass's tile masses, then searched).
// ---------------------------------------------------------------------------
constexpr int TREE_MAX = SMCSD_TREE_MAX_NODES;
// 8 wavefronts: with 2 waves per SIMD the walk keeps its state in registers
// (no scratch spills, whose stores every barrier would wait for)
constexpr int TREE_WAVES = 8;
constexpr int TREE_BLOCK = TREE_WAVES * WAVE;
// Tiles whose residual weights a node's passes keep in LDS (bf16 with 16-byte
// loads: 16 tiles, 128 KiB, every tile up to V = 32768; the walk's one
// workgroup per CU leaves that LDS unused): the node's next pass continues the
// residual chain from them (one exponential a logit pair, no target-row
// loads), and the final draw reads its tile's weights there.
template <typename DT, bool VL>
constexpr int tree_held_tiles() {
  return DT::VEC == 8 && VL ? 16 : 0;
}

struct TreeLds {
  TailLds t;  // draw scratch: staged partials, tile masses, located tile
  float Mt[TREE_MAX], Md[TREE_MAX];      // row offsets (log2 domain): target row of node n, local draft row k
  double St[TREE_MAX], Sd[TREE_MAX];     // row sums of 2^(z c - M)
  double lSt[TREE_MAX], lSd[TREE_MAX];   // their natural logs
  int par[TREE_MAX];                     // local parent of node n (-1 at the root)
  int drow[TREE_MAX];                    // local draft row of node n, -1 for a leaf
  float zt[TREE_MAX], zd[TREE_MAX];      // node n's token logit in its parent's target / draft row
  int xok[TREE_MAX];                     // node n's token lies in [0, V)
  float ut[TREE_MAX];                    // uniforms (the root's slot: the final draw)
  uint64_t kids[TREE_MAX / WAVE];        // children of the current node, as bits
  int wcnt[TREE_WAVES];                    // nodes with children per wavefront (draft-row scan)
  double Z[TREE_MAX];                    // masses of the current node's rejections
  float iz[TREE_MAX];                    // 1 / Z (0: that rejection left r unchanged)
  int bad, accept;
  int lost;  // a wait for another member's tile mass ran out: wait no more
};

// Row statistics of the RA rows at partA (into Mt/St/lSt) and the RB rows at
// partB (into Md/Sd/lSd), each row's nseg partials folded exactly as
// merge_rows_to folds them (16 threads per row, ascending partial index per
// thread, the same DPP fold), so a row gets the statistics it would get there;
// the loads of both sets are issued before any is folded.
template <int NT>
__device__ __forceinline__ void merge_tree_rows(const float2* __restrict__ partA, int RA,
                                                const float2* __restrict__ partB, int RB, int nseg, TreeLds& L) {
  constexpr int TPR = 16;
  constexpr int GB = 4;
  constexpr int NB = MAX_TILES / (GB * TPR);
  const int sub = threadIdx.x & (TPR - 1);
  const int R = RA + RB;
  for (int r0 = 0; r0 < R; r0 += NT / TPR) {
    const int r = r0 + (int)threadIdx.x / TPR;
    float m = -INFINITY;
    double s = 0.0;
    if (r < R) {
      const float2* row = r < RA ? partA + (int64_t)r * nseg : partB + (int64_t)(r - RA) * nseg;
#pragma unroll
      for (int h = 0; h < NB; h++) {
        const int k0 = sub + h * GB * TPR;
        if (h > 0 && nseg <= h * GB * TPR) break;
        float2 v[GB];
#pragma unroll
        for (int j = 0; j < GB; j++) v[j] = row[min(k0 + j * TPR, nseg - 1)];
#pragma unroll
        for (int j = 0; j < GB; j++)
          if (k0 + j * TPR < nseg) fold(m, s, v[j].x, (double)v[j].y);
      }
    }
    fold_dpp<DPP_ROW_MIRROR>(m, s);
    fold_dpp<DPP_ROW_HALF_MIRROR>(m, s);
    fold_dpp<DPP_QUAD_XOR1>(m, s);
    fold_dpp<DPP_QUAD_XOR2>(m, s);
    if (r < R && sub == 0) {
      if (r < RA) {
        L.Mt[r] = m;
        L.St[r] = s;
        L.lSt[r] = log(s);
      } else {
        L.Md[r - RA] = m;
        L.Sd[r - RA] = s;
        L.lSd[r - RA] = log(s);
      }
    }
  }
}

__device__ __forceinline__ RowStat stat_at(const float* M, const double* S, const double* lS, int r) {
  RowStat rs;
  rs.M = M[r];
  rs.S = S[r];
  rs.lS = lS[r];
  rs.ok = (rs.M > -INFINITY) && (rs.M < INFINITY) && (rs.S >= 0.5) && (rs.S < INFINITY);
  return rs;
}

// Weights of one tile of node u's row pair after `nrej` earlier rejections at
// u: r = p, then r <- max(0, r - q) * iz[j] for each earlier rejection j (r
// unchanged where iz[j] = 0); w = max(0, r - q) (sub) or w = r (!sub).  With
// no earlier rejection this is exactly residual_weights, as in sd_verify.
template <typename DT>
__device__ __forceinline__ void tree_weights(const Raw<DT>& rt, const Raw<DT>& rd, float At, float Ad, float c,
                                             const float* iz, int nrej, bool sub, float (&w)[PER_LANE]) {
  if (nrej == 0 && sub) {
    residual_weights<DT>(rt, rd, At, Ad, c, w);
    return;
  }
#pragma unroll
  for (int ch = 0; ch < Raw<DT>::CHUNKS; ch++) {
    float r[DT::VEC], q[DT::VEC];
    unpack<DT>(rt, ch, r);
    unpack<DT>(rd, ch, q);
#pragma unroll
    for (int k = 0; k < DT::VEC; k++) {
      r[k] = __builtin_amdgcn_exp2f(fmaf(r[k], c, -At));
      q[k] = __builtin_amdgcn_exp2f(fmaf(q[k], c, -Ad));
    }
    // the earlier rejections, one chunk at a time
    for (int j = 0; j < nrej; j++) {
      const float z = iz[j];
      if (z > 0.0f) {
#pragma unroll
        for (int k = 0; k < DT::VEC; k++) r[k] = fmaxf(r[k] - q[k], 0.0f) * z;
      }
    }
#pragma unroll
    for (int k = 0; k < DT::VEC; k++) w[ch * DT::VEC + k] = sub ? fmaxf(r[k] - q[k], 0.0f) : r[k];
  }
}

template <typename DT, bool VL>
__global__ __launch_bounds__(TREE_BLOCK) void k_tree_tail(TreeArgs a) {
  using raw = typename DT::raw;
  constexpr int HT = tree_held_tiles<DT, VL>();
  __shared__ TreeLds L;
  // residual weights of the node's last pass, tiles < HT, four elements a
  // 16-byte slot: [tile][element / 4][lane]
  constexpr int Q4 = PER_LANE / 4;
  __shared__ float4 HW[HT > 0 ? HT * Q4 * WAVE : 1];
  const StepArgs& s = a.s;
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  const int tid = threadIdx.x;
  // workgroup -> (tree b, member k of S).  The S members of a tree are 8
  // workgroup indices apart, so that, with workgroups dealt to the 8 XCDs in
  // turn, they share one L2; indices past the last tree have nothing to do.
  // Every member walks the whole tree (the same loads and arithmetic, so the
  // same decisions); a rejection pass is shared: member k weighs the tiles
  // t = k (mod S) and the members exchange their tiles' masses.
  const int S = a.split;
  int b = blockIdx.x, k = 0;
  if (S > 1) {
    const int x = (int)blockIdx.x % 8, r = (int)blockIdx.x / 8;
    k = r % S;
    b = x + 8 * (r / S);
    if (b >= a.B) return;
  }
  const int ntiles = s.ntiles;
  int ev = 0;
  auto tstamp = [&](unsigned code) {
    if (k == 0) stamp_wg(b, ev, code);
    ev++;
  };
  tstamp(0);
  const int64_t n0 = a.node_off[b], d0 = a.draft_off[b];
  const int64_t M64 = a.node_off[b + 1] - n0, D64 = a.draft_off[b + 1] - d0;
  // offsets that do not describe a tree inside the buffers: nothing is read
  bool ok = M64 >= 1 && M64 <= TREE_MAX && D64 >= 0 && D64 < M64 && n0 >= 0 && n0 + M64 <= s.rows_t && d0 >= 0 &&
            d0 + D64 <= s.rows_d;
  if (b == 0) ok = ok && n0 == 0 && d0 == 0;
  if (b == a.B - 1) ok = ok && n0 + M64 == s.rows_t && d0 + D64 == s.rows_d;
  if (!ok) {
    if (tid == 0) raise_flags(s.flags, FLAG_BAD_INPUT);
    return;
  }
  const int M = (int)M64, D = (int)D64;
  if (tid == 0) {
    L.t.fl = 0;
    L.bad = 0;
    L.lost = 0;
  }
  // parents, tokens and uniforms, one thread per node
  int pn = -1;
  int32_t xn = 0;
  float un = 0.0f;
  if (tid < M) {
    pn = a.parent[n0 + tid];
    xn = a.tokens[n0 + tid];
    un = a.uniforms[n0 + tid];
  }
  // statistics of the tree's target rows (flat rows n0 ..) and draft rows
  // (flat rows rows_t + d0 ..), all partial loads in one round trip
  merge_tree_rows<TREE_BLOCK>(s.part + n0 * s.nseg, M, s.part + (s.rows_t + d0) * s.nseg, D, s.nseg, L);
  if (tid < M) {
    L.par[tid] = pn;
    L.drow[tid] = 0;
    L.ut[tid] = un;
  }
  __syncthreads();
  tstamp(STAMP_TREE_MERGED);
  // tree order: the root's parent is -1, every other parent comes earlier;
  // mark the nodes that have children
  bool badn = false;
  if (tid < M) {
    if (tid == 0) {
      badn = pn != -1;
    } else {
      badn = pn < 0 || pn >= tid;
      if (!badn) L.drow[pn] = 1;
    }
  }
  __syncthreads();
  const int has = tid < M ? L.drow[tid] : 0;
  const uint64_t hb = __ballot(has != 0);
  if (lane == 0) L.wcnt[wave] = __builtin_popcountll(hb);
  const uint64_t anyb = __ballot(badn);
  if (lane == 0 && anyb) atomicOr(&L.bad, 1);
  __syncthreads();
  // draft row of a node with children: its rank among them (node order)
  int before = 0, total = 0;
  for (int w = 0; w < TREE_WAVES; w++) {
    const int cnt = L.wcnt[w];
    before += w < wave ? cnt : 0;
    total += cnt;
  }
  const int rank = before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(hb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)hb, 0));
  if (tid < M) L.drow[tid] = has ? rank : -1;
  if (total != D && tid == 0) L.bad = 1;
  __syncthreads();
  if (L.bad) {
    if (tid == 0) raise_flags(s.flags, FLAG_BAD_INPUT);
    return;
  }
  // each node's token logit in its parent's target row and draft row
  if (tid >= 1 && tid < M) {
    const int pp = L.par[tid];
    const bool xv = xn >= 0 && xn < s.V;
    const raw* tr = static_cast<const raw*>(s.target) + (n0 + pp) * s.V;
    const raw* dr = static_cast<const raw*>(s.draft) + (d0 + L.drow[pp]) * s.V;
    L.zt[tid] = xv ? DT::to_f32(tr[xn]) : 0.0f;
    L.zd[tid] = xv ? DT::to_f32(dr[xn]) : 0.0f;
    L.xok[tid] = xv;
  }
  __syncthreads();
  tstamp(STAMP_TREE_GATHERED);
  uint32_t fl = 0;
  const double ufin = (double)L.ut[0];
  int u = 0, depth = 0, y = 0;
  int owner = 0;        // the member that draws the final token
  uint32_t npass = 0;   // passes so far: the tag of a pass's exchanged masses
  for (;;) {
    // the children of u, as bits of node indices (M <= TREE_MAX = 4 wavefronts of nodes)
    const uint64_t kb = __ballot(tid < M && L.par[tid] == u);
    if (lane == 0 && wave < TREE_MAX / WAVE) L.kids[wave] = kb;
    __syncthreads();
    const int dr = L.drow[u];
    const RowStat st = stat_at(L.Mt, L.St, L.lSt, u);
    if (!st.ok) fl |= FLAG_NONFINITE;
    const raw* trow = static_cast<const raw*>(s.target) + (n0 + u) * s.V;
    if (dr < 0) {
      // a leaf: the bonus token from p_u (its tile or segment partials),
      // drawn by member 0
      if (k == 0) {
        int bnp, bper;
        const float2* bp = bonus_partials(s, n0 + u, n0 + u, 0, &bnp, &bper);
        tstamp(STAMP_TREE_LEAF);
        stage_partials<TREE_BLOCK>(bp, bnp, L.t);
        __syncthreads();
        y = draw_softmax<DT, VL, TREE_WAVES>(trow, s, s.c, st.M, ufin, bnp, bper, L.t, fl);
        tstamp(STAMP_TREE_DRAWN);
      }
      break;
    }
    const RowStat sd = stat_at(L.Md, L.Sd, L.lSd, dr);
    if (!sd.ok) fl |= FLAG_NONFINITE;
    const raw* drw = static_cast<const raw*>(s.draft) + (d0 + dr) * s.V;
    const float At = log2_norm(st), Ad = log2_norm(sd);
    // weights of tile t of u's row pair after nr earlier rejections (cached
    // loads: a second pass at u reads the same tiles again)
    auto tile_w = [&](int t, int nr, bool sub, float (&w)[PER_LANE]) {
      const Raw<DT> rt = load_tile<DT, VL, 0>(trow, s.V, t, lane);
      const Raw<DT> rd = load_tile<DT, VL, 0>(drw, s.V, t, lane);
      tree_weights<DT>(rt, rd, At, Ad, s.c, L.iz, nr, sub, w);
    };
    // the word through which tile t's mass of the pass tagged `tag` travels
    auto xslot = [&](uint32_t tag, int t) { return a.xchg + ((int64_t)b * 2 + (tag & 1u)) * ntiles + t; };
    auto store_mass = [&](int t, const float (&w)[PER_LANE], uint32_t tag) {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < PER_LANE; e++) m += w[e];
      m = wave_sum(m);
      if (lane == 0) {
        L.t.W[t] = (double)m;
        if (S > 1) tagged_put(xslot(tag, t), tag, m);
      }
    };
    // The weights of tile t in a pass with nr earlier rejections (sub:
    // max(0, r - q), else r).  A sub pass whose previous rejection left mass
    // (Z > 0) continues from that pass's weights W held in LDS: r = W / Z,
    // w = max(0, r - q), the same operations as the chain rebuilt from p and
    // q, with one exponential a logit pair instead of two.  Every sub pass
    // stores its weights of the held tiles for the next.  Tile t = k + S j is
    // always weighed by wavefront j % TREE_WAVES and held in slot j < HT, so
    // its LDS slice needs no barrier.
    auto weigh = [&](int t, Raw<DT>& rt, Raw<DT>& rd, bool cont, int nr, bool sub, float (&w)[PER_LANE]) {
      mask_tail<DT>(rd, s.V, t, lane);
      const int hj = t / S;
      if (cont) {
        const float z = L.iz[nr - 1];
#pragma unroll
        for (int i = 0; i < Q4; i++) {
          const float4 h = HW[(hj * Q4 + i) * WAVE + lane];
          w[4 * i] = h.x;
          w[4 * i + 1] = h.y;
          w[4 * i + 2] = h.z;
          w[4 * i + 3] = h.w;
        }
#pragma unroll
        for (int ch = 0; ch < Raw<DT>::CHUNKS; ch++) {
          float q[DT::VEC];
          unpack<DT>(rd, ch, q);
#pragma unroll
          for (int k = 0; k < DT::VEC; k++) {
            const int e = ch * DT::VEC + k;
            const float qk = __builtin_amdgcn_exp2f(fmaf(q[k], s.c, -Ad));
            w[e] = fmaxf(w[e] * z - qk, 0.0f);
          }
        }
      } else {
        mask_tail<DT>(rt, s.V, t, lane);
        tree_weights<DT>(rt, rd, At, Ad, s.c, L.iz, nr, sub, w);
      }
      if (HT > 0 && sub && hj < HT) {
#pragma unroll
        for (int i = 0; i < Q4; i++)
          HW[(hj * Q4 + i) * WAVE + lane] = make_float4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
      }
    };
    // one pass over u's row pair: every tile's mass into L.t.W, this
    // member's tiles weighed here and the others' masses read from their
    // words; with bf16 16-byte loads (registers to spare) a wavefront issues
    // the loads of two of its tiles before weighing either, so a 16-tile pair
    // costs one round trip to memory, not two.  A member writes a bank of
    // words again two passes later, which it reaches only after every member
    // has published the pass in between, hence read this bank: two banks
    // (by the pass's parity) keep every word until all have read it.
    constexpr bool PAIR = DT::VEC == 8 && VL;
    auto pass = [&](int nr, bool sub) {
      const uint32_t tag = ++npass;
#if SMCSD_PHASE_STAMPS >= 2
      tstamp(STAMP_TREE_PASS_START);
#endif
      if constexpr (!PAIR) {
        for (int t = k + S * wave; t < ntiles; t += S * TREE_WAVES) {
          float w[PER_LANE];
          tile_w(t, nr, sub, w);
          store_mass(t, w, tag);
        }
      } else {
        const bool cont = HT > 0 && sub && nr > 0 && L.iz[nr - 1] > 0.0f;
        for (int t0 = k + S * wave; t0 < ntiles; t0 += 2 * S * TREE_WAVES) {
          const int t1 = t0 + S * TREE_WAVES;
          const int t1c = t1 < ntiles ? t1 : t0;  // a tile of the row either way
          const bool c0 = cont && t0 / S < HT, c1 = cont && t1 / S < HT;
          // both rows' tiles are loaded even where the weights continue from
          // LDS: the loads stay one unconditional batch (measured faster than
          // skipping the target row's, which comes from cache then)
          Raw<DT> rt0 = load_raw<DT, VL, 0>(trow, s.V, t0, lane);
          Raw<DT> rd0 = load_raw<DT, VL, 0>(drw, s.V, t0, lane);
          Raw<DT> rt1 = load_raw<DT, VL, 0>(trow, s.V, t1c, lane);
          Raw<DT> rd1 = load_raw<DT, VL, 0>(drw, s.V, t1c, lane);
          float w[PER_LANE];
          weigh(t0, rt0, rd0, c0, nr, sub, w);
          store_mass(t0, w, tag);
          if (t1 < ntiles) {
            weigh(t1, rt1, rd1, c1, nr, sub, w);
            store_mass(t1, w, tag);
          }
        }
      }
#if SMCSD_PHASE_STAMPS >= 2
      if (tid == 0) tstamp(STAMP_TREE_PASS_WEIGHED);
#endif
      if (S > 1) {
        for (int t = tid; t < ntiles; t += TREE_BLOCK) {
          if (t % S == k) continue;
          float v = 0.0f;
          if (!L.lost && !tagged_get(xslot(tag, t), tag, &v)) {
            fl |= FLAG_WAIT_EXPIRED;  // this tree's outputs are unspecified
            L.lost = 1;
          }
          L.t.W[t] = (double)v;
        }
      }
    };
    // thread 0's acceptance test of child c after nr rejections at u: the
    // ratio r(x) / q(x) of its token
    auto accepts = [&](int c, int nr) -> bool {
      if (!L.xok[c]) {
        fl |= FLAG_BAD_INPUT;
        return false;
      }
      // p(x) / q(x) as in sd_verify (the fp32 exponential of the fp64 log
      // difference); each earlier rejection j turns r(x) / q(x) into
      // max(0, r(x) / q(x) - 1) / Z_j
      const double lp = log_prob(L.zt[c], st, s.c), lq = log_prob(L.zd[c], sd, s.c);
      double ratio = (double)__builtin_amdgcn_exp2f((float)((lp - lq) * 1.4426950408889634));
      for (int j = 0; j < nr; j++)
        if (L.Z[j] > 0.0) ratio = fmax(ratio - 1.0, 0.0) / L.Z[j];
      return (double)L.ut[c] < ratio;
    };
    // the children of u in node order
    int kw = 0;
    uint64_t bits = L.kids[0];
    auto next_child = [&]() -> int {
      while (!bits && ++kw < TREE_MAX / WAVE) bits = L.kids[kw];
      if (!bits) return -1;
      const int c = kw * WAVE + __builtin_ctzll(bits);
      bits &= bits - 1;
      return c;
    };
    int nrej = 0, next = -1;
    int cnode = next_child();  // u has children: a node without is a leaf
    if (tid == 0) L.accept = accepts(cnode, 0);
    lds_barrier();
    for (;;) {
      if (L.accept) {
        next = cnode;
        break;
      }
      // rejected: one pass for the mass of max(0, r - q); wavefront 0 then
      // forms its total and thread 0 tests the next child right away
      pass(nrej, true);
      lds_barrier();
#if SMCSD_PHASE_STAMPS >= 2
      tstamp(STAMP_TREE_PASS_GATHERED);
#endif
      const int cn = next_child();
      if (wave == 0) {
        double z = 0.0;
        for (int t = lane; t < ntiles; t += WAVE) z += L.t.W[t];
        z = wave_sum_f64(z);
        if (lane == 0) {
          L.Z[nrej] = z;
          L.iz[nrej] = z > 0.0 ? (float)(1.0 / z) : 0.0f;
          if (!(z > 0.0)) fl |= FLAG_ZERO_RESIDUAL;  // r and q agree: r stays
          if (cn >= 0) L.accept = accepts(cn, nrej + 1);
        }
      }
      lds_barrier();
      nrej++;
      if (cn < 0) break;  // every child rejected
      cnode = cn;
    }
    tstamp((next >= 0 ? STAMP_TREE_ACCEPTED : STAMP_TREE_REJECTED) + (unsigned)min(nrej, 99));
    if (next >= 0) {
      u = next;
      depth++;
      lds_barrier();  // L.kids is rewritten for the next node
      continue;
    }
    // every child rejected: the final token from the last pass's weights, or,
    // when that pass left no mass, from r itself (sd_verify's p_n fallback
    // for the first rejection)
    const int last = nrej - 1;
    const bool zero = !(L.Z[last] > 0.0);
    if (zero) {
      pass(last, false);
      lds_barrier();
    }
    if (wave == 0) {
      auto wt = [&](int k) -> double { return L.t.W[k]; };
      double bef = 0.0, target = 0.0;
      int lastk = -1;
      const int k = locate(ntiles, wt, 0.0, [&](double tt) { return ufin * tt; }, lane, &bef, &target, &lastk);
      if (lane == 0) {
        L.t.sel = k >= 0 ? k : (lastk >= 0 ? lastk : 0);
        L.t.clamp = k < 0;
        L.t.target = target - bef;  // the target inside the located tile
      }
    }
    lds_barrier();
    const int tt = L.t.sel;
    owner = tt % S;
    if (k == owner && wave == (tt / S) % TREE_WAVES) {
      // the located tile's weights as its pass weighed them (held in LDS, or
      // recomputed the same way by the wavefront that weighed it, which reads
      // the tile again, likely from its cache)
      float w[PER_LANE];
      if (HT > 0 && !zero && tt / S < HT) {
#pragma unroll
        for (int i = 0; i < Q4; i++) {
          const float4 h = HW[(tt / S * Q4 + i) * WAVE + lane];
          w[4 * i] = h.x;
          w[4 * i + 1] = h.y;
          w[4 * i + 2] = h.z;
          w[4 * i + 3] = h.w;
        }
      } else {
        tile_w(tt, last, !zero, w);
      }
      auto wfn = [&](int ch, float (&x)[DT::VEC]) {
#pragma unroll
        for (int k = 0; k < DT::VEC; k++) x[k] = w[ch * DT::VEC + k];
      };
      int last_pos = -1;
      int idx = tile_search<DT>(wfn, L.t.clamp ? INFINITY : (float)L.t.target, lane, &last_pos);
      if (idx < 0) {
        fl |= FLAG_CDF_CLAMP;
        idx = last_pos >= 0 ? last_pos : 0;
      }
      if (lane == 0) L.t.y = tt * TILE + idx;
    }
    lds_barrier();
    y = L.t.y;
    tstamp(STAMP_TREE_DRAWN);
    break;
  }
  or_flags(fl, L.t);
  __syncthreads();
  if (tid == 0) {
    if (k == 0) {
      a.num_accepted[b] = depth;
      a.last_node[b] = u;
    }
    if (k == owner) a.final_token[b] = y;
    raise_flags(s.flags, L.t.fl);
  }
}

// ---------------------------------------------------------------------------
// k_smc_tail: one workgroup per particle; the last particle of a prompt runs
// the prompt's ESS, resampling and page-table gather
// ---------------------------------------------------------------------------
// dst row k = src row anc[k], for k < N, rows of W elements.  Whole
// workgroup: each wavefront copies GR rows at a time, two 64-element column
// blocks per pass, with all GR x 2 loads issued before their stores.  Row and
// column indices past the end are clamped to the last row and column, for
// the stores too: a clamped lane writes the value that element gets anyway,
// and with no branch around the stores the loads stay ahead of them.  (The
// pointers are not restrict-qualified: loads from read-only memory would be
// free to sink down to their stores.)
using i32x4 = int __attribute__((ext_vector_type(4)));

template <typename E>
__device__ __forceinline__ void gather_rows(const E* src, E* dst, int N, int64_t W,
                                            const int* anc) {
  constexpr int GR = 4, GC = 2;
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  for (int k0 = wave * GR; k0 < N; k0 += WAVES_PER_BLOCK * GR) {
    int64_t from[GR];
#pragma unroll
    for (int j = 0; j < GR; j++) from[j] = (int64_t)anc[min(k0 + j, N - 1)] * W;
    for (int64_t l0 = 0; l0 < W; l0 += GC * WAVE) {
      E v[GR][GC];
      int64_t col[GC];
#pragma unroll
      for (int h = 0; h < GC; h++) col[h] = min(l0 + h * WAVE + lane, W - 1);
#pragma unroll
      for (int j = 0; j < GR; j++)
#pragma unroll
        for (int h = 0; h < GC; h++) v[j][h] = src[from[j] + col[h]];
#pragma unroll
      for (int j = 0; j < GR; j++)
#pragma unroll
        for (int h = 0; h < GC; h++) dst[(int64_t)min(k0 + j, N - 1) * W + col[h]] = v[j][h];
    }
  }
}

// Prompt p's work; with parts > 1 the prompt is shared by that many
// workgroups: each forms the ESS and the ancestors itself (the same values),
// part 0 stores them, and each gathers its own share of the page-table rows.
__device__ void smc_prompt_tail(const SmcArgs& a, int64_t p, PromptLds& Q, int part = 0, int parts = 1) {
  const StepArgs& s = a.s;
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  const int N = a.N;
  const int64_t base = p * N;
  uint32_t fl = 0;
  const float ru = a.resample_u[p];  // issued early: nothing below waits on it until the slot ranges
  if (a.lwords) {
    // from the particles' tagged words (this workgroup is the prompt's last
    // particle's: see k_smc_tail)
    for (int k = threadIdx.x; k < N; k += BLOCK) {
      float v = 0.0f;
      if (!tagged_get(a.lwords + base + k, 1u, &v)) raise_flags(s.flags, FLAG_WAIT_EXPIRED);
      Q.lw[k] = v;
    }
  } else {
    for (int k = threadIdx.x; k < N; k += BLOCK) Q.lw[k] = a.ws_logw[base + k];
  }
  __syncthreads();
  if (wave == 0) {
    float mf = -INFINITY;
    for (int k = lane; k < N; k += WAVE) mf = fmaxf(mf, Q.lw[k]);
    mf = wave_max(mf);
    const double M = (double)mf;
    const bool zero = !(M > -INFINITY);
    if (M == INFINITY || M != M) fl |= FLAG_NONFINITE;
    double Sw = 0.0, Sw2 = 0.0;
    int last_pos = -1;
    if (!zero) {
      for (int k0 = 0; k0 < N; k0 += WAVE) {
        const int k = k0 + lane;
        const double wk = k < N ? exp((double)Q.lw[k] - M) : 0.0;
        Sw += wave_sum_f64(wk);
        Sw2 += wave_sum_f64(wk * wk);
        const uint64_t pos = __ballot(wk > 0.0);
        if (pos) last_pos = k0 + 63 - __builtin_clzll(pos);
      }
    } else {
      fl |= FLAG_ZERO_WEIGHTS;
    }
    const double E = zero ? 0.0 : Sw * Sw / Sw2;
    const bool do_res = !zero && E < (double)a.ess_frac * (double)N;
    const double u = (double)ru;
    double run = 0.0;
    int carry = 0;  // first slot of the chunk's first particle
    for (int k0 = 0; k0 < N; k0 += WAVE) {
      const int ii = k0 + lane;
      int hi;  // particle ii supplies the slots [lo, hi)
      if (do_res) {
        // slot k descends from the first i with C_i > (u + k) / N, so particle
        // i receives k in [ceil(N C_{i-1} - u), ceil(N C_i - u)); consecutive
        // ranges share their end points, so every slot is covered once
        const double wi = ii < N ? exp((double)Q.lw[ii] - M) : 0.0;
        const double incl = wave_incl_scan_f64(wi, lane);
        double h = ceil((double)N * ((run + incl) / Sw) - u);
        if (ii >= last_pos) {  // the last particle with positive weight ends at N
          if (ii == last_pos && h < (double)N) fl |= FLAG_CDF_CLAMP;
          h = (double)N;
        }
        hi = (int)fmin(fmax(h, 0.0), (double)N);
        run += readlane_f64(incl, WAVE - 1);
      } else {
        hi = ii + 1;
      }
      if (ii >= N) hi = N;
      const int prev = __builtin_amdgcn_update_dpp(0, hi, DPP_WAVE_SHR1, 0xF, 0xF, false);  // lane - 1
      const int lo = lane == 0 ? carry : prev;
      hi = max(hi, lo);
      carry = __builtin_amdgcn_readlane(hi, WAVE - 1);
      if (ii < N) {
        Q.hi[ii] = hi;
        if (part == 0) a.logw[base + ii] = do_res ? 0.0f : Q.lw[ii];
      }
    }
    if (lane == 0 && part == 0) {
      a.ess[p] = (float)E;
      a.resampled[p] = do_res ? 1 : 0;
    }
    fl = wave_or_flags(fl);
    if (lane == 0 && part == 0) raise_flags(s.flags, fl);
  }
  __syncthreads();
  // slot k's ancestor: the first particle whose range ends past k (the range
  // ends never decrease and the last one is N), found by bisection, one
  // thread per slot
  for (int k = threadIdx.x; k < N; k += BLOCK) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (Q.hi[mid] > k) hi = mid;
      else lo = mid + 1;
    }
    if (part == 0) a.ancestors[base + k] = lo;
    Q.anc[k] = lo;
  }
  __syncthreads();
  // page-table rows by ancestor (the identity when the prompt kept its
  // particles): this part's rows r0 .. r1-1
  const int r0 = (int)((int64_t)N * part / parts), r1 = (int)((int64_t)N * (part + 1) / parts);
  if (a.pt_in && a.L > 0 && r0 < r1) {
    const int64_t L = a.L;
    const int32_t* __restrict__ src = a.pt_in + base * L;
    int32_t* __restrict__ dst = a.pt_out + (base + r0) * L;
    if ((L % 4) == 0 && (((uintptr_t)src | (uintptr_t)dst) & 15) == 0)
      gather_rows(reinterpret_cast<const i32x4*>(src), reinterpret_cast<i32x4*>(dst), r1 - r0, L / 4, Q.anc + r0);
    else
      gather_rows(src, dst, r1 - r0, L, Q.anc + r0);
  }
}

// With vector loads, the form followed by a prompt kernel keeps at most 64
// VGPRs (8 wavefronts per SIMD), so that 8 workgroups fit on a compute unit
// and 2048 particles run at once; the form that also does the prompts' work
// (MERGED: calls of at most 512 particles) takes up to 80, 6 workgroups a
// compute unit, with half the scalar spills (16 particles: 18.75 -> 18.2 us a
// call; the 64 cap is the faster one on 2048 particles, 20.6 against 23.0 us
// of decisions).  The element-wise loads need more registers than either.
template <typename DT, bool VL, bool MERGED>
__global__ __launch_bounds__(BLOCK, VL ? (MERGED ? 6 : 8) : 1) void k_smc_tail(SmcArgs a) {
  using raw = typename DT::raw;
  // the particle's work in L; the prompt's, in the prompt's last particle's
  // workgroup, in Q over the same LDS
  __shared__ union {
    TailLds L;
    PromptLds Q;
  } U;
  TailLds& L = U.L;
  const StepArgs& s = a.s;
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  const int64_t i = blockIdx.x;
  const int K = s.K;
  const Group G = group_of(i, K, nullptr, s.rows_d);
  const float2* pg = s.part + G.fr0 * s.nseg;
  if (threadIdx.x == 0) L.fl = 0;
  const int32_t xt = token_of<BLOCK>(s, G);
  const float lw_in = a.logw[i];
  const float ub = a.bonus_u[i];
  // power target: the bonus row at the plain scale too, as row 2K+1
  merge_rows_to<BLOCK>(pg, 2 * K + 1, s.nseg, L.M, L.S, L.lS, a.power ? s.part1 + i * s.nseg : nullptr);
  int bnp, bper;
  const float2* bp = bonus_partials(s, G.fr0, i, K, &bnp, &bper);
  stage_partials<BLOCK>(bp, bnp, L);
  int ok = 1;
  const float z = token_logit<DT, BLOCK>(s, G, i, xt, &ok);
  store_tokens<BLOCK>(z, ok, 0.0f, K, L);
  __syncthreads();
  uint32_t fl = 0;
  float lw = 0.0f;
  // wavefront 1 forms the new log-weight while wavefront 0 locates the bonus
  // draw's tile, and stores it while wavefront 0 reloads and searches that tile
  if (wave == 1) {
    double delta = 0.0;
    for (int j0 = 0; j0 < K; j0 += WAVE) {
      const int j = j0 + lane;
      double dj = 0.0;
      if (j < K) {
        const RowStat st = stat_of(L, j), sd = stat_of(L, K + 1 + j);
        if (!st.ok || !sd.ok) fl |= FLAG_NONFINITE;
        if (!L.xok[j]) fl |= FLAG_BAD_INPUT;
        else dj = (double)a.beta * log_prob(L.z[j], st, s.c) - log_prob(L.z[K + j], sd, s.c);
      }
      delta += wave_sum_f64(dj);
    }
    if (a.power) {
      // the (K+1)-th token comes from the normalised p_K^beta, so its weight
      // is Z_beta = sum_y p_K(y)^beta = exp(LSE(beta a) - beta LSE(a)), with
      // LSE(beta a) = M ln 2 + ln S from the bonus row's statistics at its own
      // scale and LSE(a) from those at the plain scale (row 2K+1); beta is
      // taken as the ratio of the two scales the statistics were formed with
      const RowStat sb = stat_of(L, K), s1 = stat_of(L, 2 * K + 1);
      if (!s1.ok) fl |= FLAG_NONFINITE;
      const double bb = (double)s.cb / (double)s.c;
      delta += ((double)sb.M - bb * (double)s1.M) * 0.69314718055994530942 + (sb.lS - bb * s1.lS);
    }
    lw = (float)((double)lw_in + delta);
    if (lw != lw || lw == INFINITY) fl |= FLAG_NONFINITE;
  }
  const RowStat sk = stat_of(L, K);
  if (!sk.ok) fl |= FLAG_NONFINITE;
  auto store_lw = [&]() {
    if (wave == 1 && lane == 0) {
      if (a.lwords) tagged_put(a.lwords + i, 1u, lw);
      else a.ws_logw[i] = lw;
    }
  };
  // the bonus row's statistics and draw are at its own scale (beta / T)
  const int y = draw_softmax<DT, VL>(group_row<raw>(s, G, i, K), s, s.cb, sk.M, (double)ub, bnp, bper, L, fl,
                                     store_lw);
  or_flags(fl, L);
  __syncthreads();
  if (threadIdx.x == 0) {
    a.bonus_token[i] = y;
    raise_flags(s.flags, L.fl);
  }
  // The prompt's ESS, resampling and page gather, by its last particle's
  // workgroup once every particle's log-weight word has arrived (the planner
  // takes this path only when every workgroup of the call fits on the device
  // at once, so the ones it waits for are running).
  if (a.lwords && i % a.N == a.N - 1) {
    __syncthreads();  // L's last reads, before Q reuses its LDS
    smc_prompt_tail(a, i / a.N, U.Q);
  }
}

// One workgroup per prompt, after every particle's log-weight is stored (the
// kernel boundary orders them): ESS, systematic resampling, page-table gather.
__global__ __launch_bounds__(BLOCK) void k_smc_prompt(SmcArgs a) {
  __shared__ PromptLds Q;
  const int parts = (int)(gridDim.x / (a.s.ngroups / a.N));  // workgroups per prompt
  smc_prompt_tail(a, blockIdx.x / parts, Q, (int)(blockIdx.x % parts), parts);
}

// ---------------------------------------------------------------------------
// host: plans and launches
// ---------------------------------------------------------------------------
// Workgroups the current device holds at once for `kernel`, queried on every
// call (the runtime answers both queries in about 0.1 us of host time, so the
// library keeps no state for them).
static int resident_blocks(const void* kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, BLOCK, 0) != hipSuccess) return 0;
  return cus * per_cu;
}

// tiles in flight per wavefront (16 VGPRs per bf16 tile, 32 per fp32 tile)
template <typename DT>
constexpr int slots_of() {
  return DT::VEC == 8 ? 3 : 2;
}

template <typename K>
static const void* kptr(K k) {
  return reinterpret_cast<const void*>(k);
}

template <typename DT, bool TP, bool PW>
static const void* stream_kernel_t(bool vec) {
  return vec ? kptr(&k_stream<DT, true, slots_of<DT>(), TP, PW>) : kptr(&k_stream<DT, false, slots_of<DT>(), TP, PW>);
}

template <bool PW>
static const void* stream_kernel_p(bool bf16, bool vec, bool tp) {
  if (bf16) return tp ? stream_kernel_t<Bf16, true, PW>(vec) : stream_kernel_t<Bf16, false, PW>(vec);
  return tp ? stream_kernel_t<F32, true, PW>(vec) : stream_kernel_t<F32, false, PW>(vec);
}

static const void* stream_kernel(bool bf16, bool vec, bool tp, bool wide, bool pw) {
  if (bf16 && vec && wide && !pw) return kptr(&k_stream_wide<Bf16, true>);
  return pw ? stream_kernel_p<true>(bf16, vec, tp) : stream_kernel_p<false>(bf16, vec, tp);
}

// Segments long enough that each resident wavefront streams about 32 units;
// on large calls, where that would give units of 8 tiles or more, about 16
// (each unit ends in a wavefront reduction: on the 32 x 64-particle
// V = 151936 call, 85 units of 8 tiles per wavefront streamed at 6.65 TB/s,
// 17 units of 38 tiles at 6.73).  From TP_MIN_SEG tiles on, the bonus rows
// also get tile partials, so a draw re-reads one tile rather than its segment.
// bf16 calls with 16-byte loads whose segments are single tiles use
// k_stream_wide (not with a power target).  The streaming grid is what the
// device holds at once of the chosen kernel, fewer when there is not one unit
// per wavefront.
constexpr int SEG_MIN = 1, TP_MIN_SEG = 2, LONG_SEG = 8;

hipError_t plan_stream(int64_t rows, int ntiles, bool bf16, bool vec, bool pw, Plan* p) {
  const int64_t tiles = rows * ntiles;
  // the streaming kernel's indices are 32-bit (more tiles than this would be
  // 8.8 TB of bf16 logits); checked before anything asks the device
  if (tiles > INT32_MAX) return hipErrorNotSupported;
  const int resident = resident_blocks(stream_kernel(bf16, vec, false, false, pw));
  if (resident <= 0) return hipErrorInvalidDevice;
  const int64_t waves = (int64_t)resident * WAVES_PER_BLOCK;

  int64_t seg = tiles / (32 * waves);
  if (seg >= LONG_SEG) seg = tiles / (16 * waves);
  seg = seg < SEG_MIN ? SEG_MIN : seg;
  if (seg > ntiles) seg = ntiles;
  const int nseg = (int)((ntiles + seg - 1) / seg);
  p->seg = (ntiles + nseg - 1) / nseg;
  p->nseg = nseg;
  p->units = rows * nseg;
  p->tp = p->seg >= TP_MIN_SEG;
  p->pw = pw;
  p->wide = bf16 && vec && p->seg == 1 && !pw;
  const int held = p->wide ? resident_blocks(stream_kernel(bf16, vec, false, true, false)) : resident;
  if (held <= 0) return hipErrorInvalidDevice;
  const int64_t want = (p->units + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK;
  p->grid = (int)(want < held ? want : held);
  if (p->grid < 1) p->grid = 1;
  return hipSuccess;
}

// One kernel launch; with a start or stop event, through the launch that
// attaches them to the dispatch itself.
template <typename A>
static hipError_t launch(const void* kernel, unsigned grid, unsigned block, const A& arg, hipStream_t s,
                         hipEvent_t start, hipEvent_t stop) {
  void* args[] = {const_cast<A*>(&arg)};
  hipError_t e = start || stop ? hipExtLaunchKernel(kernel, dim3(grid), dim3(block), args, 0, s, start, stop, 0)
                               : hipLaunchKernel(kernel, dim3(grid), dim3(block), args, 0, s);
  return e == hipSuccess ? hipGetLastError() : e;
}

template <typename DT, bool VL>
static const void* sd_tail_kernel() {
  return kptr(&k_sd_tail<DT, VL>);
}
template <typename DT, bool VL>
static const void* draw_tail_kernel() {
  return kptr(&k_draw_tail<DT, VL>);
}

template <typename DT, bool VL>
static const void* smc_tail_kernel(bool merged) {
  return merged ? kptr(&k_smc_tail<DT, VL, true>) : kptr(&k_smc_tail<DT, VL, false>);
}

// Members per decision (a sequence or a tree): 4, else 2, while the
// 8 S ceil(n / 8) workgroups of the split grid all fit on the device at once
// (members wait for each other's tile masses) and every member has a tile to
// weigh; else 1 (no exchange).
static int member_split(int64_t n, int ntiles, const void* kernel, int block) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess)
    return 1;
  const int64_t held = (int64_t)cus * per_cu;
  for (int S = SMCSD_MAX_MEMBERS; S > 1; S /= 2)
    if (S <= ntiles && 8LL * S * ((n + 7) / 8) <= held) return S;
  return 1;
}

// The decision kernel's grid: one workgroup per decision, or for S members
// 8 S ceil(n / 8) (member k of decision b at index b % 8 + 8 (k + S (b / 8))).
static unsigned member_grid(int64_t n, int S) { return (unsigned)(S > 1 ? 8LL * S * ((n + 7) / 8) : n); }

hipError_t launch_sd(const SdArgs& args, const Plan& p, bool bf16, bool vec, hipStream_t s,
                     const KernelTimers& t) {
  SdArgs a = args;
  const bool draws = a.s.K == 0 && !a.s.offsets;  // draws only
  const void* k = draws ? (bf16 ? (vec ? draw_tail_kernel<Bf16, true>() : draw_tail_kernel<Bf16, false>())
                                : (vec ? draw_tail_kernel<F32, true>() : draw_tail_kernel<F32, false>()))
                        : (bf16 ? (vec ? sd_tail_kernel<Bf16, true>() : sd_tail_kernel<Bf16, false>())
                                : (vec ? sd_tail_kernel<F32, true>() : sd_tail_kernel<F32, false>()));
  a.split = draws || !a.xchg ? 1 : member_split(a.s.ngroups, a.s.ntiles, k, SD_BLOCK);
  if (a.split > 1) {
    a.s.xz = a.xchg;  // the streaming kernel zeroes the exchange words
    a.s.xzn = a.s.ngroups * a.s.ntiles;
  }
  hipError_t e = launch(stream_kernel(bf16, vec, p.tp, p.wide, p.pw), (unsigned)p.grid, BLOCK, a.s, s,
                        t.stream_start, t.stream_stop);
  if (e != hipSuccess) return e;
  if (draws) return launch(k, (unsigned)a.s.ngroups, BLOCK, a, s, t.tail_start, t.tail_stop);
  return launch(k, member_grid(a.s.ngroups, a.split), SD_BLOCK, a, s, t.tail_start, t.tail_stop);
}

constexpr int64_t SMC_MERGED_MAX = 512;

hipError_t launch_smc(const SmcArgs& args, const Plan& p, bool bf16, bool vec, hipStream_t s,
                      const KernelTimers& t) {
  SmcArgs a = args;
  auto tail_kernel = [&](bool merged) {
    return bf16 ? (vec ? smc_tail_kernel<Bf16, true>(merged) : smc_tail_kernel<Bf16, false>(merged))
                : (vec ? smc_tail_kernel<F32, true>(merged) : smc_tail_kernel<F32, false>(merged));
  };
  // the prompts' work inside the particle kernel on calls of at most
  // SMC_MERGED_MAX particles whose workgroups all fit on the device at once
  // (each prompt's last particle waits for the others' log-weights), else a
  // prompt kernel after it (measured: 20.0 -> 18.8 us on 16 particles, 1576
  // -> 1588 us on 2048, where the prompt kernel's own grid does the gathers
  // sooner than the last particles can)
  if (a.lwords && (a.s.ngroups > SMC_MERGED_MAX || resident_blocks(tail_kernel(true)) < a.s.ngroups))
    a.lwords = nullptr;
  const void* k = tail_kernel(a.lwords != nullptr);
  if (a.lwords) {
    a.s.xz = a.lwords;  // the streaming kernel zeroes the words
    a.s.xzn = a.s.ngroups;
  }
  hipError_t e = launch(stream_kernel(bf16, vec, p.tp, p.wide, p.pw), (unsigned)p.grid, BLOCK, a.s, s,
                        t.stream_start, t.stream_stop);
  if (e != hipSuccess) return e;
  if (a.lwords) return launch(k, (unsigned)a.s.ngroups, BLOCK, a, s, t.tail_start, t.tail_stop);
  e = launch(k, (unsigned)a.s.ngroups, BLOCK, a, s, t.tail_start, nullptr);
  if (e != hipSuccess) return e;
  // a prompt's page-table rows are shared by up to 8 workgroups, about 16 KiB
  // of rows each, so that large tables are copied by more than one CU a prompt
  int64_t parts = a.pt_in && a.L > 0 ? (int64_t)a.N * a.L / 4096 : 1;
  parts = parts < 1 ? 1 : parts > 8 ? 8 : parts;
  if (parts > a.N) parts = a.N;
  return launch(kptr(&k_smc_prompt), (unsigned)(a.s.ngroups / a.N * parts), BLOCK, a, s, nullptr, t.tail_stop);
}

template <typename DT, bool VL>
static const void* tree_tail_kernel() {
  return kptr(&k_tree_tail<DT, VL>);
}

hipError_t phase_stamps(void* dst, size_t bytes, bool clear) {
#if SMCSD_PHASE_STAMPS
  constexpr size_t kBytes = sizeof(g_stamps);
  if (dst) {
    hipError_t e = hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_stamps), bytes < kBytes ? bytes : kBytes, 0,
                                       hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
  }
  if (clear) {
    static const unsigned long long zeros[SMCSD_STAMP_WGS * SMCSD_STAMP_EVENTS * 2] = {};
    return hipMemcpyToSymbol(HIP_SYMBOL(g_stamps), zeros, kBytes, 0, hipMemcpyHostToDevice);
  }
  return hipSuccess;
#else
  (void)dst;
  (void)bytes;
  (void)clear;
  return hipErrorNotSupported;
#endif
}

hipError_t launch_tree(const TreeArgs& args, const Plan& p, bool bf16, bool vec, hipStream_t s,
                       const KernelTimers& t) {
  const void* k = bf16 ? (vec ? tree_tail_kernel<Bf16, true>() : tree_tail_kernel<Bf16, false>())
                       : (vec ? tree_tail_kernel<F32, true>() : tree_tail_kernel<F32, false>());
  TreeArgs a = args;
  a.split = member_split(a.B, a.s.ntiles, k, TREE_BLOCK);
  if (a.split > 1) {
    a.s.xz = a.xchg;  // the streaming kernel zeroes the exchange words
    a.s.xzn = (int64_t)a.B * 2 * a.s.ntiles;
  }
  hipError_t e = launch(stream_kernel(bf16, vec, p.tp, p.wide, p.pw), (unsigned)p.grid, BLOCK, a.s, s,
                        t.stream_start, t.stream_stop);
  if (e != hipSuccess) return e;
  return launch(k, member_grid(a.B, a.split), TREE_BLOCK, a, s, t.tail_start, t.tail_stop);
}

}  // namespace smcsd
