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
//                    scan of the pages each particle needs).
// smc_pages_resample four launches: reference counts move from each old row to
//                    its new row (only entries that differ), the pages that
//                    reach zero are staged per row, a scan orders them by their
//                    first entry in the old rows, and they are pushed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "smcsd.h"

namespace smcsd {
namespace {

constexpr int PG_BLOCK = 1024;  // the single-workgroup kernels
constexpr int PG_WAVES = PG_BLOCK / WAVE;
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
  int N, L, S;
  int64_t M;
  const int32_t* ancestors;
  const int32_t* table_old;
  const int32_t* table_new;
  const int32_t* len_in;
  int32_t* len_out;
  int32_t* ref;
  int32_t* free_pages;
  int32_t* free_count;
  uint32_t* flags;
  uint32_t* first;   // [M] key of a page's first entry in the old rows (0 between calls)
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

// Exclusive prefix sum over the workgroup's threads in thread order; *total
// gets the sum.  lds holds PG_WAVES + 1 values.
__device__ int64_t block_excl_scan(int64_t v, int64_t* lds, int64_t* total) {
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
    for (int w = 0; w < PG_WAVES; w++) {
      const int64_t t = lds[w];
      lds[w] = run;
      run += t;
    }
    lds[PG_WAVES] = run;
  }
  __syncthreads();
  const int64_t r = lds[wave] + x - v;
  *total = lds[PG_WAVES];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int64_t block_sum(int64_t v, int64_t* lds) {
  int64_t total;
  block_excl_scan(v, lds, &total);
  return total;
}

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(PG_BLOCK) void k_pages_append(AppendArgs a) {
  __shared__ int64_t lds[PG_WAVES + 1];
  __shared__ uint32_t s_err;
  const int S = a.S, L = a.L, A = a.A;
  if (threadIdx.x == 0) s_err = 0;
  __syncthreads();
  uint32_t err = 0;
  // 1. lengths and tails: count the rows sharing each partially filled tail
  //    page and note the highest of them
  for (int64_t r = threadIdx.x; r < a.R; r += PG_BLOCK) {
    const int32_t ln = a.len[r];
    if (ln < 0 || used_pages(ln, S) > L) {
      err |= FLAG_BAD_INPUT;
      continue;
    }
    if (used_pages((int64_t)ln + A, S) > L) err |= FLAG_PAGES_FULL;
    if (ln % S) {
      const int32_t pg = a.table[r * L + used_pages(ln, S) - 1];
      if (pg < 0 || pg >= a.M) {
        err |= FLAG_BAD_INPUT;
        continue;
      }
      atomicAdd(&a.sharers[pg], 1);
      atomicMax(&a.keeper[pg], (int32_t)(r + 1));
    }
  }
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  // 2. the sharing rule, and the pages the step needs
  int64_t need = 0;
  if (!s_err) {
    for (int64_t r = threadIdx.x; r < a.R; r += PG_BLOCK) {
      const int32_t ln = a.len[r];
      need += used_pages((int64_t)ln + A, S) - used_pages(ln, S);
      if (ln % S) {
        const int32_t pg = a.table[r * L + used_pages(ln, S) - 1];
        if (ld_agent(&a.sharers[pg]) != a.ref[pg]) err |= FLAG_BAD_INPUT;
        need += ld_agent(&a.keeper[pg]) != (int32_t)(r + 1);
      }
    }
  }
  const int64_t total = block_sum(need, lds);
  const int32_t fc = *a.free_count;
  if (threadIdx.x == 0 && !s_err && total > fc) err |= FLAG_PAGES_EXHAUSTED;
  if (err) atomicOr(&s_err, err);
  __syncthreads();
  const uint32_t fail = s_err;
  // 3. pop and apply, particles in index order (chunks of the workgroup)
  int64_t carry_cow = 0;  // copies listed (the same in every thread)
  if (!fail) {
    int64_t carry_need = 0;
    for (int64_t r0 = 0; r0 < a.R; r0 += PG_BLOCK) {
      const int64_t r = r0 + threadIdx.x;
      int32_t ln = 0, tail = -1;
      int64_t u0 = 0, u1 = 0;
      int cow = 0;
      if (r < a.R) {
        ln = a.len[r];
        u0 = used_pages(ln, S);
        u1 = used_pages((int64_t)ln + A, S);
        if (ln % S) {
          tail = a.table[r * L + u0 - 1];
          cow = ld_agent(&a.keeper[tail]) != (int32_t)(r + 1);
        }
      }
      int64_t n_need, n_cow;
      const int64_t off = carry_need + block_excl_scan(cow + (u1 - u0), lds, &n_need);
      const int64_t coff = carry_cow + block_excl_scan(cow, lds, &n_cow);
      if (r < a.R) {
        int32_t* row = a.table + r * L;
        int64_t top = (int64_t)fc - off;  // this particle pops free[top - 1], free[top - 2], ...
        bool bad_page = false;            // a free-stack entry outside the pool: skipped, flagged
        if (cow) {
          const int32_t q = a.free_pages[--top];
          if (q < 0 || q >= a.M) {
            bad_page = true;
          } else {
            a.cow[3 * coff] = tail;
            a.cow[3 * coff + 1] = q;
            a.cow[3 * coff + 2] = ln % S;
            atomicSub(&a.ref[tail], 1);
            a.ref[q] = 1;
            row[u0 - 1] = q;
          }
        }
        for (int64_t j = u0; j < u1; j++) {
          const int32_t q = a.free_pages[--top];
          if (q < 0 || q >= a.M) {
            bad_page = true;
            continue;
          }
          a.ref[q] = 1;
          row[j] = q;
        }
        if (bad_page) raise_flags(a.flags, FLAG_BAD_INPUT);
        for (int t = 0; t < A; t++) {
          const int64_t pos = (int64_t)ln + t;
          a.slots[r * A + t] = row[pos / S] * S + (int32_t)(pos % S);
        }
        a.len[r] = ln + A;
      }
      carry_need += n_need;
      carry_cow += n_cow;
    }
    if (threadIdx.x == 0) {
      *a.free_count = (int32_t)(fc - total);
      *a.cow_count = (int32_t)carry_cow;
    }
  } else if (threadIdx.x == 0 && a.flags) {
    atomicOr(a.flags, fail);
  }
  __syncthreads();
  // 4. leave the scratch at zero: the tail pages named before the step (a
  //    copied page's old id is in the copy list; a kept one is still in its
  //    row, where a copy's new id would also be cleared, harmlessly)
  for (int64_t r = threadIdx.x; r < a.R; r += PG_BLOCK) {
    const int32_t ln = fail ? a.len[r] : a.len[r] - A;
    if (ln < 0 || used_pages(ln, S) > L || !(ln % S)) continue;
    const int32_t pg = a.table[r * L + used_pages(ln, S) - 1];
    if (pg >= 0 && pg < a.M) {
      a.sharers[pg] = 0;
      a.keeper[pg] = 0;
    }
  }
  for (int64_t i = threadIdx.x; i < carry_cow; i += PG_BLOCK) {
    const int32_t pg = ld_agent(&a.cow[3 * i]);
    a.sharers[pg] = 0;
    a.keeper[pg] = 0;
  }
}

// ---------------------------------------------------------------------------
// resample
// ---------------------------------------------------------------------------
// One wavefront per particle row: the length by ancestor, and the reference
// counts of the entries where the new row differs from the old one.
__device__ __forceinline__ uint32_t entry_key(const ResampleArgs& a, int64_t k, int64_t j) {
  return (uint32_t)(a.R * a.L - (k * a.L + j));  // larger for earlier entries; 0 = none
}

__device__ __forceinline__ bool row_lengths(const ResampleArgs& a, int64_t k, int32_t* ln_old, int32_t* ln_new) {
  const int32_t anc = a.ancestors[k];
  if (anc < 0 || anc >= a.N) return false;
  *ln_old = a.len_in[k];
  *ln_new = a.len_in[(k / a.N) * a.N + anc];
  const int64_t cap = (int64_t)a.L * a.S;
  return *ln_old >= 0 && *ln_old <= cap && *ln_new >= 0 && *ln_new <= cap;
}

__global__ __launch_bounds__(BLOCK) void k_pages_diff(ResampleArgs a) {
  const int lane = threadIdx.x % WAVE;
  const int64_t k = (int64_t)blockIdx.x * WAVES_PER_BLOCK + wave_id();
  if (k >= a.R) return;
  int32_t lo, ln;
  uint32_t bad = 0;
  if (!row_lengths(a, k, &lo, &ln)) {
    if (lane == 0) raise_flags(a.flags, FLAG_BAD_INPUT);
    return;
  }
  if (lane == 0) a.len_out[k] = ln;
  const int64_t uo = used_pages(lo, a.S), un = used_pages(ln, a.S);
  const int64_t um = uo > un ? uo : un;
  for (int64_t j = lane; j < um; j += WAVE) {
    const int32_t pn = j < un ? a.table_new[k * a.L + j] : -1;
    const int32_t po = j < uo ? a.table_old[k * a.L + j] : -1;
    if (pn == po) continue;
    if (j < un) {
      if (pn < 0 || pn >= a.M) bad = FLAG_BAD_INPUT;
      else atomicAdd(&a.ref[pn], 1);
    }
    if (j < uo) {
      if (po < 0 || po >= a.M) bad = FLAG_BAD_INPUT;
      else {
        atomicSub(&a.ref[po], 1);
        atomicMax(&a.first[po], entry_key(a, k, j));
      }
    }
  }
  if (bad) raise_flags(a.flags, bad);
}

// One wavefront per row: the old entries whose page reached zero and whose
// entry is that page's first, staged in entry order.
__global__ __launch_bounds__(BLOCK) void k_pages_freed(ResampleArgs a) {
  const int lane = threadIdx.x % WAVE;
  const int64_t k = (int64_t)blockIdx.x * WAVES_PER_BLOCK + wave_id();
  if (k >= a.R) return;
  int32_t lo, ln;
  int32_t n = 0;
  if (row_lengths(a, k, &lo, &ln)) {
    const int64_t uo = used_pages(lo, a.S), un = used_pages(ln, a.S);
    for (int64_t j0 = 0; j0 < uo; j0 += WAVE) {
      const int64_t j = j0 + lane;
      bool freed = false;
      int32_t po = -1;
      if (j < uo) {
        po = a.table_old[k * a.L + j];
        const int32_t pn = j < un ? a.table_new[k * a.L + j] : -1;
        freed = po != pn && po >= 0 && po < a.M && ld_agent(&a.ref[po]) == 0 &&
                ld_agent(&a.first[po]) == entry_key(a, k, j);
      }
      const uint64_t bal = __ballot(freed);
      if (freed) a.staged[k * a.L + n + __builtin_popcountll(bal & ((1ull << lane) - 1))] = po;
      n += __builtin_popcountll(bal);
    }
  }
  if (lane == 0) a.counts[k] = n;
}

// One workgroup: the stack positions of each row's freed pages.
__global__ __launch_bounds__(PG_BLOCK) void k_pages_scan(ResampleArgs a) {
  __shared__ int64_t lds[PG_WAVES + 1];
  int64_t carry = 0;
  for (int64_t r0 = 0; r0 < a.R; r0 += PG_BLOCK) {
    const int64_t r = r0 + threadIdx.x;
    int64_t t;
    const int64_t off = carry + block_excl_scan(r < a.R ? a.counts[r] : 0, lds, &t);
    if (r < a.R) a.offsets[r] = (int32_t)off;
    carry += t;
  }
  if (threadIdx.x == 0) {
    const int32_t fc = *a.free_count;
    *a.base = fc;
    if ((int64_t)fc + carry > a.M) raise_flags(a.flags, FLAG_BAD_INPUT);  // the counts were not consistent
    *a.free_count = (int32_t)((int64_t)fc + carry < a.M ? (int64_t)fc + carry : a.M);
  }
}

// One wavefront per row: push the staged pages; clear the scratch keys.
__global__ __launch_bounds__(BLOCK) void k_pages_push(ResampleArgs a) {
  const int lane = threadIdx.x % WAVE;
  const int64_t k = (int64_t)blockIdx.x * WAVES_PER_BLOCK + wave_id();
  if (k >= a.R) return;
  const int64_t base = (int64_t)*a.base + a.offsets[k];
  const int32_t n = a.counts[k];
  for (int i = lane; i < n; i += WAVE)
    if (base + i < a.M) a.free_pages[base + i] = a.staged[k * a.L + i];
  int32_t lo, ln;
  if (!row_lengths(a, k, &lo, &ln)) return;
  const int64_t uo = used_pages(lo, a.S), un = used_pages(ln, a.S);
  for (int64_t j = lane; j < uo; j += WAVE) {
    const int32_t po = a.table_old[k * a.L + j];
    const int32_t pn = j < un ? a.table_new[k * a.L + j] : -1;
    if (po != pn && po >= 0 && po < a.M) a.first[po] = 0;
  }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
constexpr size_t kPgAlign = SMCSD_WORKSPACE_ALIGN;
size_t pg_align(size_t x) { return (x + kPgAlign - 1) / kPgAlign * kPgAlign; }

struct PagesLayout {
  size_t a, b, counts, offsets, staged, base, total;
};

PagesLayout pages_layout(int64_t R, int64_t L, int64_t M) {
  PagesLayout l;
  l.a = 0;
  l.b = pg_align(l.a + 4 * (size_t)M);
  l.counts = pg_align(l.b + 4 * (size_t)M);
  l.offsets = pg_align(l.counts + 4 * (size_t)R);
  l.staged = pg_align(l.offsets + 4 * (size_t)R);
  l.base = pg_align(l.staged + 4 * (size_t)(R * L));
  l.total = pg_align(l.base + 4);
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
  hipLaunchKernelGGL(k_pages_append, dim3(1), dim3(PG_BLOCK), 0, s, a);
  return hipGetLastError() == hipSuccess ? SMCSD_OK : SMCSD_ERR_HIP;
}

int32_t smc_pages_resample(int32_t P, int32_t N, int32_t L, int32_t page_size, int64_t num_pages,
                           const int32_t* ancestors, const int32_t* page_table_old, const int32_t* page_table_new,
                           const int32_t* seq_len_in, int32_t* seq_len_out, int32_t* ref_count, int32_t* free_pages,
                           int32_t* free_count, uint32_t* status_flags, void* workspace, size_t workspace_bytes,
                           void* stream) {
  using namespace smcsd;
  const int64_t R = (int64_t)P * N;
  if (P < 0 || N < 1 || !pages_shape_ok(R, L, page_size, num_pages)) return SMCSD_ERR_INVALID_ARG;
  if (R == 0) return SMCSD_OK;
  if (!ancestors || !page_table_old || !page_table_new || !seq_len_in || !seq_len_out || !ref_count || !free_pages ||
      !free_count)
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
  a.M = num_pages;
  a.ancestors = ancestors;
  a.table_old = page_table_old;
  a.table_new = page_table_new;
  a.len_in = seq_len_in;
  a.len_out = seq_len_out;
  a.ref = ref_count;
  a.free_pages = free_pages;
  a.free_count = free_count;
  a.flags = status_flags;
  a.first = reinterpret_cast<uint32_t*>(ws + l.a);
  a.counts = reinterpret_cast<int32_t*>(ws + l.counts);
  a.offsets = reinterpret_cast<int32_t*>(ws + l.offsets);
  a.staged = reinterpret_cast<int32_t*>(ws + l.staged);
  a.base = reinterpret_cast<int32_t*>(ws + l.base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)((R + WAVES_PER_BLOCK - 1) / WAVES_PER_BLOCK);
  hipLaunchKernelGGL(k_pages_diff, dim3(grid), dim3(BLOCK), 0, s, a);
  if (hipGetLastError() != hipSuccess) return SMCSD_ERR_HIP;
  hipLaunchKernelGGL(k_pages_freed, dim3(grid), dim3(BLOCK), 0, s, a);
  if (hipGetLastError() != hipSuccess) return SMCSD_ERR_HIP;
  hipLaunchKernelGGL(k_pages_scan, dim3(1), dim3(PG_BLOCK), 0, s, a);
  if (hipGetLastError() != hipSuccess) return SMCSD_ERR_HIP;
  hipLaunchKernelGGL(k_pages_push, dim3(grid), dim3(BLOCK), 0, s, a);
  return hipGetLastError() == hipSuccess ? SMCSD_OK : SMCSD_ERR_HIP;
}

}  // extern "C"
