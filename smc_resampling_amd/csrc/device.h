// device.h -- device building blocks shared by the verify and SMC kernels.
//
// A "tile" is TILE = 2048 consecutive logits of one row, processed by one
// 64-lane wavefront.  Lane l holds 32 values in registers, loaded with 16-byte
// vector loads: chunk c (0..CHUNKS-1) covers elements
// [c*64*VEC, (c+1)*64*VEC) of the tile and lane l holds the VEC consecutive
// elements starting at c*64*VEC + l*VEC (VEC = 8 for bf16, 4 for fp32).
// Ascending token order inside a tile is therefore (chunk, lane, element).
//
// Softmax statistics use base-2 exponentials: with c = log2(e) / T,
// exp((z - m) / T) = 2^((z - m) * c).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smcsd {

constexpr int WAVE = 64;
constexpr int BLOCK = 256;  // threads per workgroup (4 wavefronts)
constexpr int WAVES_PER_BLOCK = BLOCK / WAVE;
constexpr int TILE = 2048;
constexpr int PER_LANE = TILE / WAVE;  // 32 values per lane

constexpr uint32_t FLAG_NONFINITE = 1, FLAG_ZERO_RESIDUAL = 2, FLAG_ZERO_WEIGHTS = 4,
                   FLAG_CDF_CLAMP = 8, FLAG_BAD_INPUT = 16, FLAG_WAIT_EXPIRED = 128;

// Index of the calling wavefront in its workgroup, as a value the compiler
// knows to be the same across the wavefront (so branches on it stay scalar).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE); }

// A 64-bit value the whole wavefront holds, as a value the compiler knows to be
// uniform.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for global memory operations still in flight (stores of
// outputs, loads issued ahead).  For code whose waves share nothing but LDS.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct Bf16 {
  using raw = uint16_t;
  static constexpr int VEC = 8;
  __device__ static float to_f32(raw v) { return __uint_as_float((uint32_t)v << 16); }
};
struct F32 {
  using raw = float;
  static constexpr int VEC = 4;
  __device__ static float to_f32(raw v) { return v; }
};

// ---------------------------------------------------------------------------
// wavefront reductions (DPP inside 16-lane rows, then the 4 row results)
// ---------------------------------------------------------------------------
constexpr int DPP_QUAD_1032 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_ROR4 = 0x124;      // row_ror:4
constexpr int DPP_ROR8 = 0x128;      // row_ror:8

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f32<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f32<DPP_ROR4>(v));
  v = fmaxf(v, dpp_f32<DPP_ROR8>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
               fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

// Maximum over the 64 lanes of values that are never NaN, through order-
// preserving integer keys: an unsigned max needs no NaN quieting and fuses
// with its DPP move, and the four row results combine in scalar registers.
__device__ __forceinline__ float wave_max_nonnan(float v) {
  const uint32_t b = __float_as_uint(v);
  uint32_t k = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, DPP_QUAD_1032, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, DPP_QUAD_2301, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, DPP_ROR4, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, DPP_ROR8, 0xF, 0xF, false));
  const uint32_t r = max(max((uint32_t)__builtin_amdgcn_readlane((int)k, 0), (uint32_t)__builtin_amdgcn_readlane((int)k, 16)),
                         max((uint32_t)__builtin_amdgcn_readlane((int)k, 32), (uint32_t)__builtin_amdgcn_readlane((int)k, 48)));
  return __uint_as_float(r ^ ((r & 0x80000000u) ? 0x80000000u : 0xFFFFFFFFu));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<DPP_QUAD_1032>(v);
  v += dpp_f32<DPP_QUAD_2301>(v);
  v += dpp_f32<DPP_ROR4>(v);
  v += dpp_f32<DPP_ROR8>(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

// 64-bit values move through DPP as two 32-bit halves
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, BANK_MASK, BOUND_ZERO);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, BANK_MASK, BOUND_ZERO);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ float dpp_f32m(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, BOUND_ZERO));
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ int64_t readlane_i64(int64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), lane);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// tagged words: values exchanged between the workgroups of one decision
// ---------------------------------------------------------------------------
// A value travels together with its tag in one 64-bit word (tag in the high
// half, the fp32 value's bits in the low half), stored and loaded with
// relaxed device-scope atomics.  Nothing else is communicated through the
// word's arrival, so no release or acquire is needed: a reader only relies
// on seeing, eventually, the one store that carries the tag it waits for.
// Tags are never 0, and the words start at 0 (an earlier kernel zeroes them).
__device__ __forceinline__ void tagged_put(uint64_t* w, uint32_t tag, float v) {
  __hip_atomic_store(w, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Ticks of the 100 MHz constant clock a reader waits for a word: 0.1 s, far
// beyond any exchange of workgroups that run together (about 1 us), so that
// a decision whose workgroups cannot all run (other work holding the device)
// still ends.  A test build sets 0, so that the waits run out at once.
#ifndef SMCSD_TAG_WAIT_TICKS
#define SMCSD_TAG_WAIT_TICKS 10000000
#endif
constexpr uint64_t TAG_WAIT_TICKS = SMCSD_TAG_WAIT_TICKS;

// Waits for word w to carry `tag` and returns its value in *v; false (and
// *v = 0) when the wait bound passes first.
__device__ __forceinline__ bool tagged_get(uint64_t* w, uint32_t tag, float* v) {
  const uint64_t t0 = wall_clock64();
  for (;;) {
    const uint64_t x = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(x >> 32) == tag) {
      *v = __uint_as_float((uint32_t)x);
      return true;
    }
    if (wall_clock64() - t0 > TAG_WAIT_TICKS) {
      *v = 0.0f;
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// OR of a small flag word over the 64 lanes (one ballot per bit).
__device__ __forceinline__ uint32_t wave_or_flags(uint32_t v) {
  uint32_t r = 0;
#pragma unroll
  for (int bit = 0; bit < 8; bit++)
    if (__ballot((v >> bit) & 1u)) r |= 1u << bit;
  return r;
}

// Sum and maximum over the 64 lanes in a fixed order (deterministic for a
// given lane assignment); every lane gets the result.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<DPP_QUAD_1032>(v);
  v += dpp_f64<DPP_QUAD_2301>(v);
  v += dpp_f64<DPP_ROR4>(v);
  v += dpp_f64<DPP_ROR8>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dpp_f64<DPP_QUAD_1032>(v));
  v = fmax(v, dpp_f64<DPP_QUAD_2301>(v));
  v = fmax(v, dpp_f64<DPP_ROR4>(v));
  v = fmax(v, dpp_f64<DPP_ROR8>(v));
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

// Inclusive prefix sums over the 64 lanes in ascending lane order, with DPP
// row shifts inside 16-lane rows, then the row totals carried across rows by
// row broadcasts (lanes a shift leaves without a source add 0).
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR3 = 0x113, DPP_ROW_SHR4 = 0x114,
              DPP_ROW_SHR8 = 0x118, DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

__device__ __forceinline__ float wave_incl_scan(float v, int /*lane*/) {
  float r = v + dpp_f32m<DPP_ROW_SHR1, 0xF, 0xF, true>(v);
  r += dpp_f32m<DPP_ROW_SHR2, 0xF, 0xF, true>(v);
  r += dpp_f32m<DPP_ROW_SHR3, 0xF, 0xF, true>(v);
  r += dpp_f32m<DPP_ROW_SHR4, 0xF, 0xE>(r);
  r += dpp_f32m<DPP_ROW_SHR8, 0xF, 0xC>(r);
  r += dpp_f32m<DPP_ROW_BCAST15, 0xA, 0xF>(r);
  r += dpp_f32m<DPP_ROW_BCAST31, 0xC, 0xF>(r);
  return r;
}

__device__ __forceinline__ double wave_incl_scan_f64(double v, int /*lane*/) {
  double r = v + dpp_f64<DPP_ROW_SHR1, 0xF, 0xF, true>(v);
  r += dpp_f64<DPP_ROW_SHR2, 0xF, 0xF, true>(v);
  r += dpp_f64<DPP_ROW_SHR3, 0xF, 0xF, true>(v);
  r += dpp_f64<DPP_ROW_SHR4, 0xF, 0xE>(r);
  r += dpp_f64<DPP_ROW_SHR8, 0xF, 0xC>(r);
  r += dpp_f64<DPP_ROW_BCAST15, 0xA, 0xF>(r);
  r += dpp_f64<DPP_ROW_BCAST31, 0xC, 0xF>(r);
  return r;
}

// ---------------------------------------------------------------------------
// tile loads: a tile stays packed in registers (bf16: 4 x 16 bytes per lane,
// fp32: 8 x 16 bytes) and is unpacked one chunk at a time
// ---------------------------------------------------------------------------
// Element index (within the tile) of value e of lane `lane`.
template <typename DT>
__device__ __forceinline__ int tile_elem(int lane, int e) {
  return (e / DT::VEC) * (WAVE * DT::VEC) + lane * DT::VEC + (e % DT::VEC);
}

// 16 bytes of raw logits in four 32-bit words (a native vector, so loads land
// in place).
using u32x4 = unsigned int __attribute__((ext_vector_type(4)));
using u32x2 = unsigned int __attribute__((ext_vector_type(2)));

template <typename DT>
struct Raw {
  static constexpr int CHUNKS = PER_LANE / DT::VEC;
  u32x4 q[CHUNKS];
};

// Buffer resource over the n bytes at p (a raw buffer: loads at byte offsets
// of n or more return 0 instead of touching memory).  p and n must be the
// same across the wavefront.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* p, uint32_t n) {
  constexpr int GFX9_RAW_BUFFER_WORD3 = 0x00020000;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)n, GFX9_RAW_BUFFER_WORD3);
}

// Load tile `tile` of `row` (V logits; row and tile the same across the
// wavefront) through a buffer resource that ends where the row does: an
// element past the row reads as 0 until mask_tail() turns it into -inf (only
// the last tile of a row reaches past V).  No load sits behind a branch (a
// conditional load would make the compiler wait for the data right away, which
// defeats loads kept in flight), and every lane's offsets are the same for
// every tile, so a tile costs its loads and a few scalar instructions.
// VECLOAD (one 16-byte load per chunk) requires a 16-byte aligned row base and
// V % DT::VEC == 0; otherwise each element is loaded on its own.  By default
// the loads are non-temporal (logits are streamed, not reused from cache:
// measured faster for the streaming and the decision kernels alike); POL = 0
// keeps them in cache for a kernel that reads the same tiles again.
template <typename DT, bool VECLOAD, int POL = 2>
__device__ __forceinline__ Raw<DT> load_raw(const typename DT::raw* __restrict__ row, int64_t V, int64_t tile,
                                            int lane) {
  using raw = typename DT::raw;
  Raw<DT> r;
  const int64_t t0 = tile * TILE;
  const __amdgpu_buffer_rsrc_t rs =
      buffer_over(reinterpret_cast<const void*>(uniform64(reinterpret_cast<int64_t>(row + t0))),
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)((V - t0) * (int64_t)sizeof(raw))));
  const int lane_bytes = lane * DT::VEC * (int)sizeof(raw);  // 16
  constexpr int pol = POL;                                    // cache policy
#pragma unroll
  for (int c = 0; c < Raw<DT>::CHUNKS; c++) {
    const int off = lane_bytes + c * WAVE * 16;
    if constexpr (VECLOAD) {
      r.q[c] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, pol);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        if constexpr (DT::VEC == 8) {
          const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 4 * k, 0, pol);
          const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 4 * k + 2, 0, pol);
          w[k] = lo | (hi << 16);
        } else {
          w[k] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 4 * k, 0, pol);
        }
      }
      r.q[c] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
  return r;
}

// Elements at or past V of tile `tile` become -inf; nothing happens for a tile
// that lies inside the row (the test is the same for the whole wavefront).
template <typename DT>
__device__ __forceinline__ void mask_tail(Raw<DT>& r, int64_t V, int64_t tile, int lane) {
  const int v = (int)V;
  const int base = (int)tile * TILE;
  if (base + TILE <= v) return;
#pragma unroll
  for (int c = 0; c < Raw<DT>::CHUNKS; c++) {
    const int off = base + c * (WAVE * DT::VEC) + lane * DT::VEC;
    uint32_t w[4] = {r.q[c].x, r.q[c].y, r.q[c].z, r.q[c].w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      if constexpr (DT::VEC == 8) {
        if (off + 2 * k >= v) w[k] = (w[k] & 0xFFFF0000u) | 0xFF80u;
        if (off + 2 * k + 1 >= v) w[k] = (w[k] & 0x0000FFFFu) | 0xFF800000u;
      } else {
        if (off + k >= v) w[k] = 0xFF800000u;
      }
    }
    r.q[c] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// load_raw then mask_tail: a tile ready to use (waits for its data).
template <typename DT, bool VECLOAD, int POL = 2>
__device__ __forceinline__ Raw<DT> load_tile(const typename DT::raw* __restrict__ row, int64_t V, int64_t tile,
                                             int lane) {
  Raw<DT> r = load_raw<DT, VECLOAD, POL>(row, V, tile, lane);
  mask_tail<DT>(r, V, tile, lane);
  return r;
}

// the VEC logits of chunk c, as fp32
template <typename DT>
__device__ __forceinline__ void unpack(const Raw<DT>& r, int c, float (&v)[DT::VEC]) {
  const u32x4 w = r.q[c];
  if constexpr (DT::VEC == 8) {
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xFFFF0000u);
    v[4] = __uint_as_float(w.z << 16);
    v[5] = __uint_as_float(w.z & 0xFFFF0000u);
    v[6] = __uint_as_float(w.w << 16);
    v[7] = __uint_as_float(w.w & 0xFFFF0000u);
  } else {
    v[0] = __uint_as_float(w.x);
    v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z);
    v[3] = __uint_as_float(w.w);
  }
}

// ---------------------------------------------------------------------------
// row statistics
// ---------------------------------------------------------------------------
struct RowStat {
  float M;    // offset of the row's z * c (log2 domain, c = log2(e) / T): at most
              // the row's largest z c, and within 64 of it
  double S;   // sum over the row of 2^(z c - M)
  double lS;  // natural log of S
  bool ok;    // M finite and S finite and >= 1 (up to rounding)
};

// natural-log probability of logit z under a row with statistics rs
__device__ __forceinline__ double log_prob(float z, const RowStat& rs, float c) {
  return ((double)z * (double)c - (double)rs.M) * 0.69314718055994530942 - rs.lS;
}

// ---------------------------------------------------------------------------
// ordered search inside a tile
// ---------------------------------------------------------------------------
// Finds the first element (ascending token order) whose inclusive prefix of
// the tile's weights exceeds `target`.  wfn(c, w) fills the DT::VEC weights of
// this lane's chunk c.  Returns the element index within the tile, or -1 when
// the whole tile's prefix stays <= target; *last_pos receives the last element
// with positive weight (or -1).  All 64 lanes must call it with the same target.
template <typename DT, typename WFN>
__device__ __forceinline__ int tile_search(WFN wfn, float target, int lane, int* last_pos) {
  constexpr int CHUNKS = PER_LANE / DT::VEC;
  float run = 0.0f;
  int found = -1;
  int lastp = -1;
#pragma unroll
  for (int c = 0; c < CHUNKS; c++) {
    float w[DT::VEC];
    wfn(c, w);
    float ls = 0.0f;
    int lk = -1;  // this lane's last positive value in the chunk
#pragma unroll
    for (int k = 0; k < DT::VEC; k++) {
      ls += w[k];
      if (w[k] > 0.0f) lk = k;
    }
    // last positive element so far: the highest lane holding one
    const uint64_t pos = __ballot(lk >= 0);
    if (pos) {
      const int hl = 63 - __builtin_clzll(pos);
      lastp = tile_elem<DT>(hl, c * DT::VEC + __builtin_amdgcn_readlane(lk, hl));
    }
    const float incl = wave_incl_scan(ls, lane);
    const uint64_t bal = __ballot(run + incl > target);
    if (bal) {
      const int src = __builtin_ctzll(bal);
      int idx = -1;
      float acc = run + (incl - ls);
#pragma unroll
      for (int k = 0; k < DT::VEC; k++) {
        acc += w[k];
        if (idx < 0 && acc > target) idx = k;
      }
      if (idx < 0) idx = lk;  // rounding between the two sums: the lane's last positive
      found = tile_elem<DT>(src, c * DT::VEC + __builtin_amdgcn_readlane(idx, src));
      break;
    }
    run += readlane_f32(incl, WAVE - 1);
  }
  *last_pos = lastp;
  return found;
}

}  // namespace smcsd
