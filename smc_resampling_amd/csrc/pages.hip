// pages.hip -- paged-KV bookkeeping around SMC resampling: the metadata update
// of a page-based KV cache that makes resampling a pointer operation ("Faster
// LLM Inference via Sequential Monte Carlo", sec. 3), with the K+1 new tokens
// every step adds per particle (sec. 2).
//
// State (all device memory, owned by the caller): a pool of M pages of S token
// slots; per particle r a page-table row of L entries and a length len[r] (its
// first ceil(len/S) entries are page ids); ref[page] = entries naming the
// page; the free pages as a stack free[0 .. free_count-1].
//
// smc_pages_append   one workgroup: every particle's partially filled tail page
//                    that other rows share is copied on write (the sharer with
//                    the highest index keeps it, which is what handling the
//                    particles in index order gives), then new pages are popped
//                    from the top of the stack in particle order (an exclusive
//                    scan of the pages each particle needs).  Each thread holds
//                    a run of consecutive particles in registers through the
//                    phases, so the kernel makes a handful of dependent trips
//                    to memory, not a handful per particle.
// smc_pages_resample four launches.  The new rows are the ancestors' old
//                    rows, so a page's count changes by the sum of (copies - 1)
//                    over the old rows that name it: one wavefront takes 64
//                    rows at a time, one position at a time, and adds that sum
//                    once per run of lanes naming the same page (rows that
//                    share a page are neighbours after systematic resampling,
//                    so shared prefixes cost one atomic or none).  A run whose
//                    rows all die marks its first entry; the marked entries
//                    whose page reached zero are staged per row in entry
//                    order, one workgroup lays the rows out on the stack by a
//                    scan, and a fourth launch pushes them (each launch reads
//                    what the one before wrote: the kernel boundaries order
//                    it, and no workgroup hands data to another).
//                    Calls of at most 16 rows of at most 256 entries run in
//                    one workgroup instead: each wavefront keeps the entries
//                    it marks in registers and, after a barrier, pushes the
//                    freed ones itself (no marks, no staging).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "smcsd.h"

namespace smcsd {
namespace {

constexpr int PG_BLOCK = 1024;  // the append workgroup
constexpr int PG_MAX_RPT = 4;   // particles per append thread held in registers
constexpr int PB = 64;          // positions per resample workgroup (16 per wavefront)
constexpr uint32_t FLAG_PAGES_FULL = SMCSD_FLAG_PAGES_FULL, FLAG_PAGES_EXHAUSTED = SMCSD_FLAG_PAGES_EXHAUSTED;

struct AppendArgs {
  int64_t R;
  int L, S, A;
  int64_t M;
  int32_t* table;
  int32_t* len;
  int32_t* ref;
  const int32_t* free_pages;
  int32_t* free_count;
  int32_t* slots;
  int32_t* cow;
  int32_t* cow_count;
  uint32_t* flags;
  int32_t* keeper;  // [M] highest sharer index + 1 of each shared tail page (0 between calls)
  int32_t* sharers; // [M] rows whose tail the page is (0 between calls)
};

struct ResampleArgs {
  int64_t R;
  int N, L, S, W;  // W = 32-bit words of a row's entry marks
  int64_t M;
  const int32_t* ancestors;
  const int32_t* table_old;
  const int32_t* len_in;
  int32_t* len_out;
  int32_t* ref;
  int32_t* free_pages;
  int32_t* free_count;
  uint32_t* flags;
  uint32_t* first;   // [M] key of a page's first entry in the old rows (0 between calls)
  uint32_t* marks;   // [R, W] entries that start a run of dying rows (0 between calls)
  int32_t* counts;   // [R] freed pages per row
  int32_t* offsets;  // [R] exclusive scan of counts
  int32_t* staged;   // [R * L] freed pages of each row, in entry order
  int32_t* base;     // [1] the stack height before the push
};

__device__ __forceinline__ int64_t used_pages(int64_t len, int S) { return (len + S - 1) / S; }

__device__ __forceinline__ void raise_flags(uint32_t* flags, uint32_t bits) {
  if (flags && bits) atomicOr(flags, bits);
}

__device__ __forceinline__ int32_t ld_agent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory operation this wavefront issued has completed: the
// count updates are device-scope atomics performed at the L2, and the
// __syncthreads that follows each use (a workgroup-scope release and acquire
// around the barrier) then orders them before the other wavefronts' reads.
__device__ __forceinline__ void mem_done() {
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Exclusive prefix sum over the workgroup's NT threads in thread order; *total
// gets the sum.  lds holds NT / WAVE + 1 values.
template <int NT>
__device__ int64_t block_excl_scan(int64_t v, int64_t* lds, int64_t* total) {
  constexpr int NW = NT / WAVE;
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  int64_t x = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int64_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == WAVE - 1) lds[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t run = 0;
    for (int w = 0; w < NW; w++) {
      const int64_t t = lds[w];
      lds[w] = run;
      run += t;
    }
    lds[NW] = run;
  }
  __syncthreads();
  const int64_t r = lds[wave] + x - v;
  *total = lds[NW];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------
// Thread t of the workgroup holds particles base + i * PG_BLOCK + t (slot i <
// RPT), so the lanes of a wavefront are 64 consecutive particles in every
// slot: rows that share a tail page (copies of one ancestor, adjacent after
// systematic resampling) form runs of lanes, and each run touches the page's
// counters once.
struct PgRow {
  int32_t ln;    // length before the step (0 past the end or when rejected)
  int32_t tail;  // its partially filled tail page, -1 if none
  int32_t u0;    // pages it used before the step
  int32_t nn;    // pages the step adds
  int32_t run;   // last lane of a run of lanes with this tail: the run's length; else 0
  int32_t cow;   // 1 if the tail is copied on write
};

__device__ __forceinline__ int64_t pg_row(int64_t base, int i, int tid) { return base + (int64_t)i * PG_BLOCK + tid; }

// Lengths, tail pages and tail runs of the particles from base on, checked.
template <int RPT>
__device__ __forceinline__ uint32_t pg_load(const AppendArgs& a, int64_t base, PgRow (&st)[RPT]) {
  const int lane = threadIdx.x % WAVE;
  const int S = a.S;
  uint32_t err = 0;
#pragma unroll
  for (int i = 0; i < RPT; i++) {
    const int64_t r = pg_row(base, i, threadIdx.x);
    st[i].ln = r < a.R ? a.len[r] : 0;
  }
#pragma unroll
  for (int i = 0; i < RPT; i++) {
    const int64_t r = pg_row(base, i, threadIdx.x);
    st[i].tail = -1;
    st[i].u0 = st[i].nn = st[i].cow = 0;
    const int32_t ln = st[i].ln;
    if (r >= a.R) continue;
    if (ln < 0 || used_pages(ln, S) > a.L) {
      err |= FLAG_BAD_INPUT;
      st[i].ln = 0;
      continue;
    }
    const int32_t full = ln / S, rem = ln - full * S;
    st[i].u0 = full + (rem != 0);
    const int64_t u1 = full + ((int64_t)rem + a.A + S - 1) / S;
    if (u1 > a.L) err |= FLAG_PAGES_FULL;
    st[i].nn = (int32_t)(u1 - st[i].u0);
    if (rem) st[i].tail = a.table[r * a.L + st[i].u0 - 1];
  }
#pragma unroll
  for (int i = 0; i < RPT; i++) {
    if (st[i].ln % S && (st[i].tail < 0 || st[i].tail >= a.M)) {
      err |= FLAG_BAD_INPUT;
      st[i].tail = -1;
    }
    // runs of lanes naming one tail page
    // (the neighbours are read by every lane: a cross-lane read under a
    // condition would leave the lane it reads from inactive)
    const int32_t t = st[i].tail;
    const int32_t up = __shfl_up(t, 1), down = __shfl_down(t, 1);
    const bool starts = lane == 0 || up != t;
    const bool ends = lane == WAVE - 1 || down != t;
    const uint64_t heads = __ballot(starts);
    const uint64_t upto = lane == WAVE - 1 ? ~0ull : (2ull << lane) - 1;
    const int head = 63 - __builtin_clzll(heads & upto);
    st[i].run = t >= 0 && ends ? lane - head + 1 : 0;
  }
  return err;
}

// The sharing rule for the tails, and which particles copy theirs: every
// lane of a run but the last has a later sharer; the last keeps the page only
// if it is the page's highest sharer overall.
template <int RPT>
__device__ __forceinline__ uint32_t pg_share(const AppendArgs& a, int64_t base, PgRow (&st)[RPT]) {
  int32_t sh[RPT], kp[RPT], rf[RPT];
#pragma unroll
  for (int i = 0; i < RPT; i++) {
    sh[i] = kp[i] = rf[i] = 0;
    if (st[i].run) {
      sh[i] = ld_agent(&a.sharers[st[i].tail]);
      kp[i] = ld_agent(&a.keeper[st[i].tail]);
      rf[i] = a.ref[st[i].tail];
    }
  }
  uint32_t err = 0;
#pragma unroll
  for (int i = 0; i < RPT; i++) {
    if (st[i].run && sh[i] != rf[i]) err |= FLAG_BAD_INPUT;
    st[i].cow = st[i].tail >= 0 && (!st[i].run || kp[i] != (int32_t)(pg_row(base, i, threadIdx.x) + 1));
  }
  return err;
}

// Pages (low 32 bits) and copies (high 32 bits) each slot's particle takes.
__device__ __forceinline__ int64_t pg_take(const PgRow& r) { return ((int64_t)r.cow << 32) + r.nn + r.cow; }

// Exclusive prefix sums of v over the particles base .. base + RPT * PG_BLOCK - 1
// in index order (slot, then thread); *total gets the sum.  lds holds one
// value per slot and wavefront; two calls in a row use different halves of a
// buffer of twice that, so one barrier suffices.
template <int RPT>
__device__ __forceinline__ void pg_scan(const int64_t (&v)[RPT], int64_t (&ex)[RPT], int64_t* total, int64_t* lds) {
  constexpr int NW = PG_BLOCK / WAVE;
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  int64_t x[RPT];
#pragma unroll
  for (int i = 0; i < RPT; i++) {
    x[i] = v[i];
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
      const int64_t y = __shfl_up(x[i], d);
      if (lane >= d) x[i] += y;
    }
    if (lane == WAVE - 1) lds[i * NW + wave] = x[i];
  }
  __syncthreads();
  int64_t run = 0;
#pragma unroll
  for (int i = 0; i < RPT; i++) {
    for (int w = 0; w < NW; w++) {
      if (w == wave) ex[i] = run + x[i] - v[i];
      run += lds[i * NW + w];
    }
  }
  *total = run;
}

// Pops and writes of the particles from base on; off[i] is what the
// particles before slot i's particle took (pages, copies packed as pg_take).
template <int RPT>
__device__ __forceinline__ void pg_apply(const AppendArgs& a, int64_t base, const PgRow (&st)[RPT],
                                         const int64_t (&off)[RPT], int32_t fc) {
  const int S = a.S, A = a.A;
  // every stack entry these particles pop first, before any store
  int32_t qc[RPT], q0[RPT];
#pragma unroll
  for (int i = 0; i < RPT; i++) {
    const int64_t top = (int64_t)fc - (off[i] & 0xffffffffll);  // pops free[top - 1], free[top - 2], ...
    qc[i] = st[i].cow ? a.free_pages[top - 1] : -1;
    q0[i] = st[i].nn ? a.free_pages[top - 1 - st[i].cow] : -1;
  }
  bool bad_page = false;  // a stack entry outside the pool: not applied, flagged
#pragma unroll
  for (int i = 0; i < RPT; i++) {
    const int64_t r = pg_row(base, i, threadIdx.x);
    if (r >= a.R) continue;
    const PgRow& w = st[i];
    int32_t* row = a.table + r * a.L;
    const int64_t tn = (int64_t)fc - (off[i] & 0xffffffffll) - w.cow;  // new pages: free[tn - 1], ...
    if (w.cow) {
      const int64_t c = off[i] >> 32;
      if (qc[i] < 0 || qc[i] >= a.M) {
        bad_page = true;
      } else {
        a.cow[3 * c] = w.tail;
        a.cow[3 * c + 1] = qc[i];
        a.cow[3 * c + 2] = w.ln % S;
        a.ref[qc[i]] = 1;
        row[w.u0 - 1] = qc[i];
      }
    } else if (w.tail >= 0) {
      a.ref[w.tail] = 1;  // the page's last sharer keeps it; every other one copied
    }
    for (int32_t e = 0; e < w.nn; e++) {
      const int32_t q = e == 0 ? q0[i] : a.free_pages[tn - 1 - e];
      if (q < 0 || q >= a.M) {
        bad_page = true;
        continue;
      }
      a.ref[q] = 1;
      row[w.u0 + e] = q;
    }
    // slots: position ln + k is on the tail page (offset ln % S on) or on a new one
    int32_t off_in = w.ln % S;
    int32_t e = off_in ? -1 : 0;
    int32_t pg = off_in ? (w.cow ? qc[i] : w.tail) : q0[i];
    for (int k = 0; k < A; k++) {
      a.slots[r * A + k] = pg * S + off_in;
      if (++off_in == S && k + 1 < A) {
        off_in = 0;
        e++;
        pg = e == 0 ? q0[i] : a.free_pages[tn - 1 - e];
      }
    }
    a.len[r] = w.ln + A;
  }
  if (bad_page) raise_flags(a.flags, FLAG_BAD_INPUT);
}

template <int RPT>
__global__ __launch_bounds__(PG_BLOCK) void k_pages_append(AppendArgs a) {
  constexpr int NW = PG_BLOCK / WAVE;
  __shared__ int64_t lds[2 * RPT * NW];
  __shared__ uint32_t s_err;
  constexpr int64_t CH = (int64_t)PG_BLOCK * RPT;  // particles per chunk
  const int64_t nchunk = (a.R + CH - 1) / CH;
  const bool one = nchunk == 1;  // the particles stay in registers from phase to phase
  if (threadIdx.x == 0) s_err = 0;
  __syncthreads();
  PgRow st[RPT];
  uint32_t err = 0;
  // 1. count the rows sharing each partially filled tail page and note the
  //    highest of them (one update per run of lanes)
  for (int64_t c = 0; c < nchunk; c++) {
    err |= pg_load(a, c * CH, st);
#pragma unroll
    for (int i = 0; i < RPT; i++) {
      if (st[i].run) {
        atomicAdd(&a.sharers[st[i].tail], st[i].run);
        atomicMax(&a.keeper[st[i].tail], (int32_t)(pg_row(c * CH, i, threadIdx.x) + 1));
      }
    }
  }
  if (err) atomicOr(&s_err, err);
  mem_done();
  __syncthreads();
  // 2. the sharing rule, and the pages the step takes
  int64_t ex0[RPT], total = 0;
  int parity = 0;
  if (!s_err) {
    for (int64_t c = 0; c < nchunk; c++) {
      if (!one) pg_load(a, c * CH, st);
      err |= pg_share(a, c * CH, st);
      int64_t v[RPT], t;
#pragma unroll
      for (int i = 0; i < RPT; i++) v[i] = pg_take(st[i]);
      pg_scan(v, ex0, &t, lds + parity * RPT * NW);
      parity ^= 1;
      total += t;
    }
  }
  const int64_t pages = total & 0xffffffffll;
  const int32_t fc = *a.free_count;
  if (threadIdx.x == 0 && pages > fc) err |= FLAG_PAGES_EXHAUSTED;
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  const uint32_t fail = s_err;
  // 3. pop and apply, particles in index order
  if (!fail) {
    int64_t carry = 0;
    for (int64_t c = 0; c < nchunk; c++) {
      int64_t ex[RPT], t = 0;
#pragma unroll
      for (int i = 0; i < RPT; i++) ex[i] = ex0[i];
      if (!one) {
        pg_load(a, c * CH, st);
        pg_share(a, c * CH, st);
        int64_t v[RPT];
#pragma unroll
        for (int i = 0; i < RPT; i++) v[i] = pg_take(st[i]);
        pg_scan(v, ex, &t, lds + parity * RPT * NW);
        parity ^= 1;
      }
#pragma unroll
      for (int i = 0; i < RPT; i++) ex[i] += carry;
      pg_apply(a, c * CH, st, ex, fc);
      carry += t;
    }
    if (threadIdx.x == 0) {
      *a.free_count = (int32_t)(fc - pages);
      *a.cow_count = (int32_t)(total >> 32);
    }
  } else if (threadIdx.x == 0 && a.flags) {
    atomicOr(a.flags, fail);
  }
  mem_done();
  __syncthreads();
  // 4. leave the scratch at zero: the tail pages named before the step
  if (one) {
#pragma unroll
    for (int i = 0; i < RPT; i++) {
      if (st[i].run) {
        a.sharers[st[i].tail] = 0;
        a.keeper[st[i].tail] = 0;
      }
    }
    return;
  }
  // (chunked: a copied page's old id is in the copy list; a kept one is still
  // in its row, where a copy's new id would also be cleared, harmlessly)
  for (int64_t r = threadIdx.x; r < a.R; r += PG_BLOCK) {
    const int32_t ln = fail ? a.len[r] : a.len[r] - a.A;
    if (ln < 0 || used_pages(ln, a.S) > a.L || !(ln % a.S)) continue;
    const int32_t pg = a.table[r * a.L + used_pages(ln, a.S) - 1];
    if (pg >= 0 && pg < a.M) {
      a.sharers[pg] = 0;
      a.keeper[pg] = 0;
    }
  }
  const int64_t ncow = fail ? 0 : total >> 32;
  for (int64_t i = threadIdx.x; i < ncow; i += PG_BLOCK) {
    const int32_t pg = ld_agent(&a.cow[3 * i]);
    a.sharers[pg] = 0;
    a.keeper[pg] = 0;
  }
}

// ---------------------------------------------------------------------------
// resample
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t entry_key(const ResampleArgs& a, int64_t k, int64_t j) {
  return (uint32_t)(a.R * a.L - (k * a.L + j));  // larger for earlier entries; 0 = none
}

// Copies of each of the 64 rows of block rb: the slots of their prompts that
// name them (NT threads; copies[] zeroed before).  Returns bad-input bits.
template <int NT>
__device__ uint32_t delta_copies(const ResampleArgs& a, int64_t rb, int32_t* copies) {
  uint32_t bad = 0;
  const int N = a.N;
  const int64_t rl = (rb + WAVE < a.R ? rb + WAVE : a.R) - 1;
  const int64_t s1 = (rl / N + 1) * N < a.R ? (rl / N + 1) * N : a.R;
  for (int64_t r = (rb / N) * N + threadIdx.x; r < s1; r += NT) {
    const int32_t anc = a.ancestors[r];
    if (anc < 0 || anc >= N) {
      bad = FLAG_BAD_INPUT;
      continue;
    }
    const int64_t t = (r / N) * N + anc - rb;
    if (t >= 0 && t < WAVE) atomicAdd(&copies[t], 1);
  }
  return bad;
}

constexpr int JW = PB / WAVES_PER_BLOCK;  // positions per wavefront

// One wavefront: rows rb .. rb+63 as the lanes (c = this lane's row's
// copies), positions j0 .. j0+JW-1.  With write_len, also the rows' new
// lengths.  An entry that starts a run of dying rows offers its key as the
// page's first and is marked: in the marks array (MARKS), or in bit i of
// `held` with its page id left in pv[i].  Returns bad-input bits.
template <bool MARKS>
__device__ __forceinline__ uint32_t delta_positions(const ResampleArgs& a, int64_t rb, int j0, int32_t c,
                                                    bool write_len, int32_t (&pv)[JW], uint32_t& held) {
  const int lane = threadIdx.x % WAVE;
  const int N = a.N;
  uint32_t bad = 0;
  const int64_t k = rb + lane;
  const bool in = k < a.R;
  int32_t ln = in ? a.len_in[k] : 0;
  if (ln < 0 || ln > (int64_t)a.L * a.S) {
    bad = FLAG_BAD_INPUT;
    ln = 0;
  }
  if (write_len && in) {
    const int32_t anc = a.ancestors[k];
    if (anc >= 0 && anc < N) {
      const int32_t la = a.len_in[(k / N) * N + anc];
      if (la < 0 || la > (int64_t)a.L * a.S) bad = FLAG_BAD_INPUT;
      a.len_out[k] = la;
    }
  }
  const int32_t used = (int32_t)used_pages(ln, a.S);
  // nothing to do where every row is copied exactly once
  held = 0;
  if (!__ballot(in && c != 1 && used > j0)) return bad;
#pragma unroll
  for (int i = 0; i < JW; i++) pv[i] = in && j0 + i < used ? a.table_old[k * a.L + j0 + i] : -1;
  // A run of lanes naming one page holds valid entries only, so its sum of
  // (copies - 1) is a difference of two prefixes over the lanes, the same
  // at every position.
  const int32_t v = in ? c - 1 : 0;
  int32_t pre = v;  // inclusive prefix of v over the lanes
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int32_t y = __shfl_up(pre, d);
    if (lane >= d) pre += y;
  }
  const uint64_t dying_rows = __ballot(in && c == 0);
  // runs at every position first (no branches: the positions interleave) ...
  bool head[JW];
  int32_t end[JW], pre_end[JW];
#pragma unroll
  for (int i = 0; i < JW; i++) {
    bool valid = in && j0 + i < used;
    if (valid && (pv[i] < 0 || pv[i] >= a.M)) {
      bad = FLAG_BAD_INPUT;
      valid = false;
    }
    pv[i] = valid ? pv[i] : -1;
    const int32_t pp = __shfl_up(pv[i], 1);
    const bool starts = lane == 0 || pp != pv[i];
    head[i] = starts && valid;
    const uint64_t heads = __ballot(starts);
    const uint64_t later = lane == WAVE - 1 ? 0 : heads & (~0ull << (lane + 1));
    end[i] = later ? __builtin_ctzll(later) - 1 : WAVE - 1;
    pre_end[i] = __shfl(pre, end[i]);
  }
  // ... then one update per run
#pragma unroll
  for (int i = 0; i < JW; i++) {
    if (!head[i]) continue;
    const int32_t p = pv[i];
    const int32_t sum = pre_end[i] - pre + v;  // over lanes lane .. end
    if (sum) atomicAdd(&a.ref[p], sum);
    const int n = end[i] - lane + 1;
    const uint64_t run = (n == WAVE ? ~0ull : (1ull << n) - 1) << lane;
    if ((dying_rows & run) == run) {
      // every row of the run dies: its first entry may be the page's first
      const int64_t j = j0 + i;
      atomicMax(&a.first[p], entry_key(a, k, j));
      if (MARKS) atomicOr(&a.marks[k * a.W + j / 32], 1u << (j % 32));
      else held |= 1u << i;
    }
  }
  return bad;
}

// Workgroup (row block x, position block y): 64 rows as the lanes of every
// wavefront, JW positions per wavefront.
__global__ __launch_bounds__(BLOCK) void k_pages_delta(ResampleArgs a) {
  __shared__ int32_t copies[WAVE];
  const int lane = threadIdx.x % WAVE;
  const int64_t rb = (int64_t)blockIdx.x * WAVE;
  if (threadIdx.x < WAVE) copies[threadIdx.x] = 0;
  __syncthreads();
  uint32_t bad = delta_copies<BLOCK>(a, rb, copies);
  __syncthreads();
  int32_t pv[JW];
  uint32_t held;
  bad |= delta_positions<true>(a, rb, blockIdx.y * PB + wave_id() * JW, copies[lane],
                               blockIdx.y == 0 && wave_id() == 0, pv, held);
  if (bad) raise_flags(a.flags, bad);
}

// One wavefront, row k: the marked entries whose page reached zero and whose
// entry is that page's first, staged in entry order; the marks and keys are
// cleared, and the row's count stored.
__device__ void stage_row(const ResampleArgs& a, int64_t k) {
  const int lane = threadIdx.x % WAVE;
  int32_t n = 0;
  for (int w0 = 0; w0 < a.W; w0 += WAVE) {
    uint32_t* mk = a.marks + k * a.W + w0;
    const uint32_t word = w0 + lane < a.W ? ld_agent(mk + lane) : 0u;
    if (!__ballot(word != 0)) continue;
    const int nw = a.W - w0 < WAVE ? a.W - w0 : WAVE;
    for (int w = 0; w < nw; w += 2) {
      const uint32_t lo = __builtin_amdgcn_readlane(word, w);
      const uint32_t hi = w + 1 < nw ? __builtin_amdgcn_readlane(word, w + 1) : 0u;
      if (!(lo | hi)) continue;
      const int64_t j = (int64_t)(w0 + w) * 32 + lane;
      const bool marked = ((lane < 32 ? lo >> lane : hi >> (lane - 32)) & 1u) != 0;
      bool freed = false;
      int32_t p = -1;
      if (marked) {
        p = a.table_old[k * a.L + j];
        if (ld_agent(&a.first[p]) == entry_key(a, k, j)) {
          a.first[p] = 0;
          freed = ld_agent(&a.ref[p]) == 0;
        }
      }
      const uint64_t bal = __ballot(freed);
      if (freed) a.staged[k * a.L + n + __builtin_popcountll(bal & ((1ull << lane) - 1))] = p;
      n += __builtin_popcountll(bal);
    }
    if (word) mk[lane] = 0;
  }
  if (lane == 0) st_agent(&a.counts[k], n);
}

// Whole workgroup of NT threads, after every row's count is stored: the stack
// position of each row's pages (an exclusive scan of the counts, NT * 8 rows
// per trip to memory); thread 0 records the stack height before the push and
// raises it.  lds holds NT / WAVE + 1 values.
template <int NT>
__device__ void scan_offsets(const ResampleArgs& a, int64_t* lds) {
  constexpr int SCAN_RPT = 8;
  int64_t carry = 0;
  for (int64_t r0 = 0; r0 < a.R; r0 += (int64_t)NT * SCAN_RPT) {
    const int64_t r = r0 + (int64_t)threadIdx.x * SCAN_RPT;
    int32_t n[SCAN_RPT];
    int64_t v = 0;
#pragma unroll
    for (int i = 0; i < SCAN_RPT; i++) n[i] = r + i < a.R ? ld_agent(&a.counts[r + i]) : 0;
#pragma unroll
    for (int i = 0; i < SCAN_RPT; i++) v += n[i];
    int64_t t;
    int64_t off = carry + block_excl_scan<NT>(v, lds, &t);
#pragma unroll
    for (int i = 0; i < SCAN_RPT; i++) {
      if (r + i < a.R) st_agent(&a.offsets[r + i], (int32_t)off);
      off += n[i];
    }
    carry += t;
  }
  if (threadIdx.x == 0) {
    const int32_t fc = *a.free_count;
    st_agent(a.base, fc);
    if ((int64_t)fc + carry > a.M) raise_flags(a.flags, FLAG_BAD_INPUT);  // the counts were not consistent
    *a.free_count = (int32_t)((int64_t)fc + carry < a.M ? (int64_t)fc + carry : a.M);
  }
}

// One wavefront, row k: push the row's staged pages.
__device__ void push_row(const ResampleArgs& a, int64_t k) {
  const int lane = threadIdx.x % WAVE;
  const int64_t base = (int64_t)ld_agent(a.base) + ld_agent(&a.offsets[k]);
  const int32_t n = ld_agent(&a.counts[k]);
  for (int i = lane; i < n; i += WAVE)
    if (base + i < a.M) a.free_pages[base + i] = ld_agent(&a.staged[k * a.L + i]);
}

// One wavefront per row stages its freed pages and stores its count.
__global__ __launch_bounds__(BLOCK) void k_pages_stage(ResampleArgs a) {
  const int64_t k = (int64_t)blockIdx.x * WAVES_PER_BLOCK + wave_id();
  if (k < a.R) stage_row(a, k);
}

// One workgroup, after every row's count is stored (the kernel boundary
// orders them): the rows' stack positions.
__global__ __launch_bounds__(BLOCK) void k_pages_scan(ResampleArgs a) {
  __shared__ int64_t lds[WAVES_PER_BLOCK + 1];
  scan_offsets<BLOCK>(a, lds);
}

// One wavefront per row: push the staged pages.
__global__ __launch_bounds__(BLOCK) void k_pages_push(ResampleArgs a) {
  const int64_t k = (int64_t)blockIdx.x * WAVES_PER_BLOCK + wave_id();
  if (k < a.R) push_row(a, k);
}

// Small calls (at most 16 rows of at most 256 entries): the whole resample in
// one workgroup.  Wavefront w takes positions JW w .. JW w + JW-1 of every row
// (rows as lanes) and keeps the entries it marks, with their page ids, in
// registers.  After one barrier the counts are final: each such entry reads
// its page's count and first key together, and the entries whose page reached
// zero and that are the page's first go straight onto the stack, in row order
// and entry order within a row (a scan over (row, wavefront) in LDS).  No marks,
// no staging.
constexpr int PG_SMALL_ROWS = PG_BLOCK / WAVE;
constexpr int PG_SMALL_L = PG_SMALL_ROWS * JW;

__global__ __launch_bounds__(PG_BLOCK) void k_pages_resample_small(ResampleArgs a) {
  constexpr int NW = PG_BLOCK / WAVE;
  static_assert(NW * JW == PG_SMALL_L && NW <= WAVE, "one slice of positions per wavefront");
  __shared__ int32_t copies[WAVE];
  __shared__ int32_t off[NW][PG_SMALL_ROWS];  // freed entries of (wavefront, row), then their stack offsets
  __shared__ int32_t s_total;
  const int lane = threadIdx.x % WAVE, wave = wave_id();
  const int64_t fc = *a.free_count;
  if (threadIdx.x < WAVE) copies[threadIdx.x] = 0;
  __syncthreads();
  uint32_t bad = delta_copies<PG_BLOCK>(a, 0, copies);
  __syncthreads();
  const int j0 = wave * JW;
  int32_t pv[JW];
  uint32_t held;
  bad |= delta_positions<false>(a, 0, j0, copies[lane], wave == 0, pv, held);
  mem_done();
  __syncthreads();
  // the page counts and first keys are final
  int32_t first_key[JW], count[JW];
#pragma unroll
  for (int i = 0; i < JW; i++) {
    const bool h = (held >> i) & 1u;
    first_key[i] = h ? (int32_t)ld_agent(&a.first[pv[i]]) : 0;
    count[i] = h ? ld_agent(&a.ref[pv[i]]) : -1;
  }
  uint32_t freed = 0;
#pragma unroll
  for (int i = 0; i < JW; i++) {
    if (((held >> i) & 1u) && (uint32_t)first_key[i] == entry_key(a, lane, j0 + i)) {
      a.first[pv[i]] = 0;  // the scratch goes back to zero
      if (count[i] == 0) freed |= 1u << i;
    }
  }
  if (lane < PG_SMALL_ROWS) off[wave][lane] = __builtin_popcount(freed);
  __syncthreads();
  if (wave == 0) {
    // lane = row: exclusive over the wavefronts, then over the rows
    int32_t run = 0;
    if (lane < PG_SMALL_ROWS) {
      for (int w = 0; w < NW; w++) {
        const int32_t t = off[w][lane];
        off[w][lane] = run;
        run += t;
      }
    }
    int32_t pre = run;
#pragma unroll
    for (int d = 1; d < PG_SMALL_ROWS; d <<= 1) {
      const int32_t y = __shfl_up(pre, d);
      if (lane >= d) pre += y;
    }
    if (lane < PG_SMALL_ROWS)
      for (int w = 0; w < NW; w++) off[w][lane] += pre - run;
    if (lane == PG_SMALL_ROWS - 1) s_total = pre;
  }
  __syncthreads();
  if (freed) {
    int64_t pos = fc + off[wave][lane];
#pragma unroll
    for (int i = 0; i < JW; i++) {
      if ((freed >> i) & 1u) {
        if (pos < a.M) a.free_pages[pos] = pv[i];
        pos++;
      }
    }
  }
  if (threadIdx.x == 0) {
    const int64_t total = s_total;
    if (fc + total > a.M) bad |= FLAG_BAD_INPUT;  // the counts were not consistent
    *a.free_count = (int32_t)(fc + total < a.M ? fc + total : a.M);
  }
  if (bad) raise_flags(a.flags, bad);
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
constexpr size_t kPgAlign = SMCSD_WORKSPACE_ALIGN;
size_t pg_align(size_t x) { return (x + kPgAlign - 1) / kPgAlign * kPgAlign; }

struct PagesLayout {
  size_t a, b, marks, counts, offsets, staged, base, total;
};

int mark_words(int64_t L) { return (int)((L + 31) / 32); }

PagesLayout pages_layout(int64_t R, int64_t L, int64_t M) {
  PagesLayout l;
  l.a = 0;
  l.b = pg_align(l.a + 4 * (size_t)M);
  l.marks = pg_align(l.b + 4 * (size_t)M);
  l.counts = pg_align(l.marks + 4 * (size_t)(R * mark_words(L)));
  l.offsets = pg_align(l.counts + 4 * (size_t)R);
  l.staged = pg_align(l.offsets + 4 * (size_t)R);
  l.base = pg_align(l.staged + 4 * (size_t)(R * L));
  l.total = pg_align(l.base + 8);
  return l;
}

bool pages_shape_ok(int64_t R, int L, int S, int64_t M) {
  return R >= 0 && L >= 1 && S >= 1 && M >= 1 && M <= INT32_MAX && R * (int64_t)L <= INT32_MAX &&
         (int64_t)L * S <= INT32_MAX;
}

bool disjoint(const void* x, size_t nx, const void* y, size_t ny) {
  const char* a = static_cast<const char*>(x);
  const char* b = static_cast<const char*>(y);
  return a + nx <= b || b + ny <= a;
}

}  // namespace
}  // namespace smcsd

extern "C" {

size_t smc_pages_workspace_bytes(int32_t P, int32_t N, int32_t L, int64_t num_pages) {
  const int64_t R = (int64_t)P * N;
  if (P < 0 || N < 1 || L < 1 || num_pages < 1) return 0;
  return smcsd::pages_layout(R, L, num_pages).total;
}

int32_t smc_pages_append(int32_t P, int32_t N, int32_t L, int32_t page_size, int32_t new_tokens,
                         int64_t num_pages, int32_t* page_table, int32_t* seq_len, int32_t* ref_count,
                         const int32_t* free_pages, int32_t* free_count, int32_t* slots, int32_t* cow_list,
                         int32_t* cow_count, uint32_t* status_flags, void* workspace, size_t workspace_bytes,
                         void* stream) {
  using namespace smcsd;
  const int64_t R = (int64_t)P * N;
  if (P < 0 || N < 1 || new_tokens < 0 || !pages_shape_ok(R, L, page_size, num_pages)) return SMCSD_ERR_INVALID_ARG;
  if (R == 0) return SMCSD_OK;
  if (!page_table || !seq_len || !ref_count || !free_pages || !free_count || !cow_list || !cow_count ||
      (new_tokens > 0 && !slots))
    return SMCSD_ERR_INVALID_ARG;
  const PagesLayout l = pages_layout(R, L, num_pages);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace % kPgAlign) != 0) return SMCSD_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  AppendArgs a;
  a.R = R;
  a.L = L;
  a.S = page_size;
  a.A = new_tokens;
  a.M = num_pages;
  a.table = page_table;
  a.len = seq_len;
  a.ref = ref_count;
  a.free_pages = free_pages;
  a.free_count = free_count;
  a.slots = slots;
  a.cow = cow_list;
  a.cow_count = cow_count;
  a.flags = status_flags;
  a.keeper = reinterpret_cast<int32_t*>(ws + l.a);
  a.sharers = reinterpret_cast<int32_t*>(ws + l.b);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (R <= PG_BLOCK)
    hipLaunchKernelGGL(k_pages_append<1>, dim3(1), dim3(PG_BLOCK), 0, s, a);
  else if (R <= 2 * PG_BLOCK)
    hipLaunchKernelGGL(k_pages_append<2>, dim3(1), dim3(PG_BLOCK), 0, s, a);
  else
    hipLaunchKernelGGL(k_pages_append<PG_MAX_RPT>, dim3(1), dim3(PG_BLOCK), 0, s, a);
  return hipGetLastError() == hipSuccess ? SMCSD_OK : SMCSD_ERR_HIP;
}

int32_t smc_pages_resample(int32_t P, int32_t N, int32_t L, int32_t page_size, int64_t num_pages,
                           const int32_t* ancestors, const int32_t* page_table_old, const int32_t* seq_len_in,
                           int32_t* seq_len_out, int32_t* ref_count, int32_t* free_pages, int32_t* free_count,
                           uint32_t* status_flags, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace smcsd;
  const int64_t R = (int64_t)P * N;
  if (P < 0 || N < 1 || !pages_shape_ok(R, L, page_size, num_pages)) return SMCSD_ERR_INVALID_ARG;
  if (R == 0) return SMCSD_OK;
  if (!ancestors || !page_table_old || !seq_len_in || !seq_len_out || !ref_count || !free_pages || !free_count)
    return SMCSD_ERR_INVALID_ARG;
  if (!disjoint(seq_len_in, 4 * (size_t)R, seq_len_out, 4 * (size_t)R)) return SMCSD_ERR_INVALID_ARG;
  const PagesLayout l = pages_layout(R, L, num_pages);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace % kPgAlign) != 0) return SMCSD_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  ResampleArgs a;
  a.R = R;
  a.N = N;
  a.L = L;
  a.S = page_size;
  a.W = mark_words(L);
  a.M = num_pages;
  a.ancestors = ancestors;
  a.table_old = page_table_old;
  a.len_in = seq_len_in;
  a.len_out = seq_len_out;
  a.ref = ref_count;
  a.free_pages = free_pages;
  a.free_count = free_count;
  a.flags = status_flags;
  a.first = reinterpret_cast<uint32_t*>(ws + l.a);
  a.marks = reinterpret_cast<uint32_t*>(ws + l.marks);
  a.counts = reinterpret_cast<int32_t*>(ws + l.counts);
  a.offsets = reinterpret_cast<int32_t*>(ws + l.offsets);
  a.staged = reinterpret_cast<int32_t*>(ws + l.staged);
  a.base = reinterpret_cast<int32_t*>(ws + l.base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (R <= PG_SMALL_ROWS && L <= PG_SMALL_L) {
    hipLaunchKernelGGL(k_pages_resample_small, dim3(1), dim3(PG_BLOCK), 0, s, a);
    return hipGetLastError() == hipSuccess ? SMCSD_OK : SMCSD_ERR_HIP;
  }
  const unsigned rows = (unsigned)((R + WAVE - 1) / WAVE), cols = (unsigned)((L + PB - 1) / PB);
  hipLaunchKernelGGL(k_pages_delta, dim3(rows, cols), dim3(BLOCK), 0, s, a);
  if (hipGetLastError() != hipSuccess) return SMCSD_ERR_HIP;
  const unsigned grid = (unsigned)((R + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK);
  hipLaunchKernelGGL(k_pages_stage, dim3(grid), dim3(BLOCK), 0, s, a);
  if (hipGetLastError() != hipSuccess) return SMCSD_ERR_HIP;
  hipLaunchKernelGGL(k_pages_scan, dim3(1), dim3(BLOCK), 0, s, a);
  if (hipGetLastError() != hipSuccess) return SMCSD_ERR_HIP;
  hipLaunchKernelGGL(k_pages_push, dim3(grid), dim3(BLOCK), 0, s, a);
  return hipGetLastError() == hipSuccess ? SMCSD_OK : SMCSD_ERR_HIP;
}

}  // extern "C"
