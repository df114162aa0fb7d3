// launch.h -- internal interface between the C-ABI entry points (api.hip) and
// the kernel launchers (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smcsd.h"

namespace smcsd {

// What both operations stream.  Rows are taken group by group (a group is an
// SD sequence or an SMC particle: its target rows 0..K_b, then its draft rows
// 0..K_b-1); each row is cut into nseg segments of `seg` tiles; a unit is one
// (row, segment).
struct StepArgs {
  const void* target;
  const void* draft;
  const int32_t* offsets;  // CSR over draft rows, or null (fixed K)
  const int32_t* tokens;   // draft token of each draft row
  int64_t ngroups, rows_t, rows_d, V;
  int K;          // draft length (largest, for CSR input)
  int ntiles;     // tiles per row
  int seg;        // tiles per segment
  int nseg;       // segments per row
  int tp;         // 1: each group's bonus row also has tile partials in tpart
  int64_t units;  // rows * nseg
  float c;        // log2(e) / T
  float cb;       // scale of each group's bonus row: c, or beta * log2(e) / T for a power target
  float2* part;   // [units] segment partials (max of z c, sum of 2^(z c - max))
  float2* tpart;  // [ngroups * ntiles] tile partials of each group's bonus row
  uint32_t* flags;
  int flat;       // 1: every row is a group of its own, the target rows then the draft rows (K = 0)
  float2* part1;  // power target: [ngroups * nseg] segment partials of each group's bonus row at scale c
  uint64_t* xz;   // [xzn] words the streaming kernel zeroes for the decision kernel after it (or null)
  int64_t xzn;
};

struct SdArgs {
  StepArgs s;
  const float* uniforms;
  int32_t* num_accepted;
  int32_t* final_token;
  // Members per sequence (1, 2 or 4): the workgroups that share a sequence's
  // residual pass, each weighing every split-th tile, and exchanging tile
  // masses through xchg: [B][ntiles] tagged words, zeroed by the streaming
  // kernel of the same call.  Set by launch_sd.
  int split;
  uint64_t* xchg;
};

struct SmcArgs {
  StepArgs s;
  float beta;  // power target: draft tokens add beta log p - log q
  int power;   // beta != 1: the bonus token also adds log sum_y p_K(y)^beta
  int N, L;
  float ess_frac;
  const float* bonus_u;
  const float* resample_u;
  float* logw;     // in/out (each entry is read before its prompt's particles are rewritten)
  float* ws_logw;  // [P*N] reweighted log-weights
  const int32_t* pt_in;
  int32_t* pt_out;
  int32_t* bonus_token;
  int32_t* ancestors;
  float* ess;
  int32_t* resampled;
  // [P*N] tagged words of the reweighted log-weights (tag 1), zeroed by the
  // streaming kernel, through which each prompt's last particle workgroup
  // collects its prompt's log-weights and then does the prompt's work itself;
  // null: a separate prompt kernel (the whole grid does not fit at once).
  // Set by launch_smc.
  uint64_t* lwords;
};

// Token trees: one workgroup per tree decides by walking it (the streaming
// kernel runs in flat mode over the trees' target rows, then their draft rows).
struct TreeArgs {
  StepArgs s;
  const int32_t* node_off;   // [B+1] CSR over nodes (= target rows)
  const int32_t* draft_off;  // [B+1] CSR over draft rows (one per node with children)
  const int32_t* parent;     // [nodes] local parent index, -1 at the root
  const int32_t* tokens;     // [nodes] draft token of each node
  const float* uniforms;     // [nodes] acceptance uniforms; the root's slot: final draw
  int32_t* num_accepted;
  int32_t* last_node;
  int32_t* final_token;
  int B;
  // Members per tree (1, 2 or 4): the workgroups that share each rejection
  // pass of a tree, each weighing every split-th tile, and exchanging tile
  // masses through xchg: [B][2][ntiles] tagged words, zeroed by the streaming
  // kernel of the same call.  Set by launch_tree.
  int split;
  uint64_t* xchg;
};

// Segment length and streaming grid of a call.
struct Plan {
  int seg, nseg;
  bool tp;    // bonus-row tile partials (segments long enough that a re-read would cost)
  bool wide;  // k_stream_wide (bf16, one-tile segments)
  bool pw;    // power target: the bonus rows also at the plain scale
  int64_t units;
  int grid;
};

// Events that take the start and stop times of a call's two kernels (any may
// be null).
struct KernelTimers {
  hipEvent_t stream_start, stream_stop, tail_start, tail_stop;
};

hipError_t plan_stream(int64_t rows, int ntiles, bool bf16, bool vec, bool pw, Plan* p);
// Each launches the streaming kernel, then the tail kernel; with timers, the
// launches carry the events.
// Phase codes of the measurement build's timestamps (each names the phase that
// ends at its stamp; 0 marks a workgroup's start).
enum : unsigned {
  STAMP_SD_MERGED = 1,          // statistics merged, token logits gathered
  STAMP_SD_TESTED = 2,          // accept tests up to the first rejection
  STAMP_SD_BONUS_DRAWN = 3,     // every draft accepted: the bonus draw
  STAMP_SD_RESIDUAL_PASS = 4,   // a rejection: the residual pass over the row pair
  STAMP_SD_LOCATED = 5,         // the residual draw's tile located
  STAMP_SD_RESIDUAL_DRAWN = 6,  // the search inside that tile
  STAMP_SD_FALLBACK_DRAWN = 7,  // zero residual: the draw from p_n
  STAMP_TREE_MERGED = 10,       // parents read, statistics merged
  STAMP_TREE_GATHERED = 11,     // draft rows ranked, token logits gathered
  STAMP_TREE_ACCEPTED = 100,    // + r: a level whose child was accepted after r rejections
  STAMP_TREE_REJECTED = 200,    // + r: a level whose r children were all rejected
  STAMP_TREE_LEAF = 300,        // a leaf reached
  STAMP_TREE_DRAWN = 400,       // the final draw (at a leaf, or from the last residual)
  // -DSMCSD_PHASE_STAMPS=2 also splits each rejection pass of the tree walk
  // (then the level phases above end at the pass's last stamp):
  STAMP_TREE_PASS_START = 12,     // the child's test and its barrier, up to the pass
  STAMP_TREE_PASS_WEIGHED = 13,   // thread 0's wavefront has weighed its tiles (round trip, arithmetic)
  STAMP_TREE_PASS_GATHERED = 14,  // the other members' masses read, barrier passed
};
hipError_t phase_stamps(void* dst, size_t bytes, bool clear);

hipError_t launch_sd(const SdArgs& a, const Plan& p, bool bf16, bool vec, hipStream_t s, const KernelTimers& t);
hipError_t launch_smc(const SmcArgs& a, const Plan& p, bool bf16, bool vec, hipStream_t s, const KernelTimers& t);
hipError_t launch_tree(const TreeArgs& a, const Plan& p, bool bf16, bool vec, hipStream_t s, const KernelTimers& t);

}  // namespace smcsd
