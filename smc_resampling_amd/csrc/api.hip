// api.hip -- C-ABI entry points: argument validation, workspace layout and
// kernel launches.  No allocation, no synchronisation.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "device.h"
#include "launch.h"
#include "smcsd.h"

namespace {

constexpr size_t kAlign = SMCSD_WORKSPACE_ALIGN;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int ntiles_of(int64_t V) { return (int)((V + smcsd::TILE - 1) / smcsd::TILE); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// 16-byte vector loads need aligned row starts: aligned bases and V a
// multiple of the vector width.
bool vec_ok(int32_t dtype, int64_t V, const void* a, const void* b) {
  const int64_t per = dtype == SMCSD_BF16 ? 8 : 4;
  return V % per == 0 && aligned16(a) && (b == nullptr || aligned16(b));
}

// Workspace layouts: scratch that each call writes before it reads it, so a
// workspace needs no initial contents and serves calls of any shapes it is
// large enough for.  The segment partials (sized for one-tile segments, the
// most a call can use), the tile partials of each group's bonus row and, for
// SMC, the reweighted log-weights.

// sd_verify's layout also holds the words through which the workgroups
// sharing a sequence's residual pass exchange tile masses (one per tile, per
// sequence); draft_sample's draws need none.
struct SdLayout {
  size_t part, tpart, xchg, total;
};

SdLayout sd_layout(int32_t B, int64_t V, int64_t rows_d, bool exchange) {
  const int nt = ntiles_of(V);
  SdLayout l;
  l.part = 0;
  l.tpart = align_up(l.part + sizeof(float2) * (size_t)((2 * rows_d + B) * nt));
  l.xchg = align_up(l.tpart + sizeof(float2) * (size_t)((int64_t)B * nt));
  l.total = align_up(l.xchg + (exchange ? sizeof(uint64_t) * (size_t)((int64_t)B * nt) : 0));
  return l;
}

// Token trees: every target row (node) and draft row is a group of its own,
// so each has segment partials and, with multi-tile segments, tile partials;
// then the words through which the workgroups sharing a tree exchange tile
// masses (two banks of one word per tile, per tree).
struct TreeLayout {
  size_t part, tpart, xchg, total;
};

TreeLayout tree_layout(int32_t B, int64_t rows, int64_t V) {
  const int nt = ntiles_of(V);
  TreeLayout l;
  l.part = 0;
  l.tpart = align_up(l.part + sizeof(float2) * (size_t)(rows * nt));
  l.xchg = align_up(l.tpart + sizeof(float2) * (size_t)(rows * nt));
  l.total = align_up(l.xchg + sizeof(uint64_t) * (size_t)((int64_t)B * 2 * nt));
  return l;
}

struct SmcLayout {
  size_t ws_logw, part, tpart, lwords, total;
};

SmcLayout smc_layout(int32_t P, int32_t N, int32_t K, int64_t V) {
  const int nt = ntiles_of(V);
  const int64_t PN = (int64_t)P * N;
  SmcLayout l;
  l.ws_logw = 0;
  l.part = align_up(l.ws_logw + sizeof(float) * (size_t)PN);
  // the segment partials of every row, then (power target) those of each
  // particle's bonus row at the plain scale: 2K+2 rows per particle
  l.tpart = align_up(l.part + sizeof(float2) * (size_t)(PN * (2 * K + 2) * nt));
  // the tagged words of the reweighted log-weights (one per particle)
  l.lwords = align_up(l.tpart + sizeof(float2) * (size_t)(PN * nt));
  l.total = align_up(l.lwords + sizeof(uint64_t) * (size_t)PN);
  return l;
}

// Kernel timers of this thread's next call (a profiling aid; see
// smcsd_time_next_call).
thread_local smcsd::KernelTimers t_timers = {};

smcsd::KernelTimers take_timers() {
  const smcsd::KernelTimers t = t_timers;
  t_timers = {};
  return t;
}

bool temperature_ok(float T) { return isfinite(T) && T > 0.0f; }

void fill_step(smcsd::StepArgs* s, const smcsd::Plan& plan, const void* target, const void* draft,
               const int32_t* offsets, const int32_t* tokens, int64_t ngroups, int64_t rows_t, int64_t rows_d,
               int64_t V, int K, float T, char* ws, size_t part_off, size_t tpart_off, uint32_t* flags) {
  s->target = target;
  s->draft = draft;
  s->offsets = offsets;
  s->tokens = tokens;
  s->ngroups = ngroups;
  s->rows_t = rows_t;
  s->rows_d = rows_d;
  s->V = V;
  s->K = K;
  s->ntiles = ntiles_of(V);
  s->seg = plan.seg;
  s->nseg = plan.nseg;
  s->tp = plan.tp ? 1 : 0;
  s->units = plan.units;
  s->c = (float)(1.4426950408889634 / (double)T);
  s->cb = s->c;
  s->part = reinterpret_cast<float2*>(ws + part_off);
  s->part1 = nullptr;
  s->xz = nullptr;
  s->xzn = 0;
  s->tpart = reinterpret_cast<float2*>(ws + tpart_off);
  s->flags = flags;
  s->flat = 0;
}


}  // namespace

extern "C" {

int32_t smcsd_abi_version(void) { return SMCSD_ABI_VERSION; }

int32_t smcsd_phase_stamps(void* host_dst, size_t bytes, int32_t clear) {
  const hipError_t e = smcsd::phase_stamps(host_dst, bytes, clear != 0);
  return e == hipSuccess ? SMCSD_OK : e == hipErrorNotSupported ? SMCSD_ERR_UNSUPPORTED : SMCSD_ERR_HIP;
}

void smcsd_time_next_call(void* stream_start, void* stream_stop, void* tail_start, void* tail_stop) {
  t_timers = {static_cast<hipEvent_t>(stream_start), static_cast<hipEvent_t>(stream_stop),
              static_cast<hipEvent_t>(tail_start), static_cast<hipEvent_t>(tail_stop)};
}

const char* smcsd_status_string(int32_t s) {
  switch (s) {
    case SMCSD_OK: return "SMCSD_OK";
    case SMCSD_ERR_INVALID_ARG: return "SMCSD_ERR_INVALID_ARG: bad shape, pointer, temperature or aliasing";
    case SMCSD_ERR_UNSUPPORTED: return "SMCSD_ERR_UNSUPPORTED: valid but outside what the kernels handle";
    case SMCSD_ERR_WORKSPACE: return "SMCSD_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case SMCSD_ERR_HIP: return "SMCSD_ERR_HIP: the HIP runtime refused a launch";
    default: return "SMCSD_UNKNOWN_STATUS";
  }
}

size_t sd_verify_workspace_bytes(int32_t dtype, int32_t B, int32_t K, int32_t V,
                                 int64_t total_draft_rows) {
  (void)dtype;
  (void)K;
  if (B <= 0 || V <= 0 || total_draft_rows < 0) return 0;
  return sd_layout(B, V, total_draft_rows, true).total;
}

int32_t sd_verify(int32_t dtype, int32_t B, int32_t K, int32_t V, float temperature,
                  const void* target_logits, const void* draft_logits,
                  const int32_t* draft_tokens, const float* uniforms,
                  const int32_t* draft_offsets, int64_t total_draft_rows,
                  int32_t* num_accepted, int32_t* final_token, uint32_t* status_flags,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != SMCSD_F32 && dtype != SMCSD_BF16) return SMCSD_ERR_INVALID_ARG;
  if (B < 0 || K < 0 || V < 1 || !temperature_ok(temperature)) return SMCSD_ERR_INVALID_ARG;
  if (V > SMCSD_MAX_V) return SMCSD_ERR_UNSUPPORTED;
  if (K > SMCSD_MAX_K) return SMCSD_ERR_UNSUPPORTED;
  if (total_draft_rows < 0 || total_draft_rows > (int64_t)B * K) return SMCSD_ERR_INVALID_ARG;
  if (!draft_offsets && total_draft_rows != (int64_t)B * K) return SMCSD_ERR_INVALID_ARG;
  if (B == 0) return SMCSD_OK;
  if (!target_logits || !uniforms || !num_accepted || !final_token) return SMCSD_ERR_INVALID_ARG;
  if (total_draft_rows > 0 && (!draft_logits || !draft_tokens)) return SMCSD_ERR_INVALID_ARG;
  const SdLayout l = sd_layout(B, V, total_draft_rows, true);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace % kAlign) != 0)
    return SMCSD_ERR_WORKSPACE;
  const bool bf16 = dtype == SMCSD_BF16;
  const bool vec = vec_ok(dtype, V, target_logits, draft_logits);
  const int64_t rows = 2 * total_draft_rows + B;
  smcsd::Plan plan;
  if (const hipError_t pe = smcsd::plan_stream(rows, ntiles_of(V), bf16, vec, false, &plan); pe != hipSuccess)
    return pe == hipErrorNotSupported ? SMCSD_ERR_UNSUPPORTED : SMCSD_ERR_HIP;
  char* ws = static_cast<char*>(workspace);
  smcsd::SdArgs a;
  fill_step(&a.s, plan, target_logits, draft_logits, draft_offsets, draft_tokens, B, total_draft_rows + B,
            total_draft_rows, V, K, temperature, ws, l.part, l.tpart, status_flags);
  a.uniforms = uniforms;
  a.num_accepted = num_accepted;
  a.final_token = final_token;
  a.split = 1;
  a.xchg = reinterpret_cast<uint64_t*>(ws + l.xchg);
  return smcsd::launch_sd(a, plan, bf16, vec, static_cast<hipStream_t>(stream), take_timers()) == hipSuccess
             ? SMCSD_OK
             : SMCSD_ERR_HIP;
}

size_t draft_sample_workspace_bytes(int32_t dtype, int32_t R, int32_t V) {
  (void)dtype;
  if (R <= 0 || V <= 0) return 0;
  return sd_layout(R, V, 0, false).total;
}

// One draw per row: the verify step's final draw with no draft tokens (each
// row a sequence whose draft length is 0, so its "bonus" row is the row).
int32_t draft_sample(int32_t dtype, int32_t R, int32_t V, float temperature, const void* logits,
                     const float* uniforms, int32_t* tokens, uint32_t* status_flags, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (dtype != SMCSD_F32 && dtype != SMCSD_BF16) return SMCSD_ERR_INVALID_ARG;
  if (R < 0 || V < 1 || !temperature_ok(temperature)) return SMCSD_ERR_INVALID_ARG;
  if (V > SMCSD_MAX_V) return SMCSD_ERR_UNSUPPORTED;
  if (R == 0) return SMCSD_OK;
  if (!logits || !uniforms || !tokens) return SMCSD_ERR_INVALID_ARG;
  const SdLayout l = sd_layout(R, V, 0, false);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace % kAlign) != 0)
    return SMCSD_ERR_WORKSPACE;
  const bool bf16 = dtype == SMCSD_BF16;
  const bool vec = vec_ok(dtype, V, logits, nullptr);
  smcsd::Plan plan;
  if (const hipError_t pe = smcsd::plan_stream(R, ntiles_of(V), bf16, vec, false, &plan); pe != hipSuccess)
    return pe == hipErrorNotSupported ? SMCSD_ERR_UNSUPPORTED : SMCSD_ERR_HIP;
  char* ws = static_cast<char*>(workspace);
  smcsd::SdArgs a;
  fill_step(&a.s, plan, logits, nullptr, nullptr, nullptr, R, R, 0, V, 0, temperature, ws, l.part, l.tpart,
            status_flags);
  a.uniforms = uniforms;
  a.num_accepted = nullptr;
  a.final_token = tokens;
  a.split = 1;
  a.xchg = nullptr;
  return smcsd::launch_sd(a, plan, bf16, vec, static_cast<hipStream_t>(stream), take_timers()) == hipSuccess
             ? SMCSD_OK
             : SMCSD_ERR_HIP;
}

size_t tree_verify_workspace_bytes(int32_t dtype, int32_t B, int32_t V, int64_t num_nodes, int64_t num_draft_rows) {
  (void)dtype;
  if (B <= 0 || V <= 0 || num_nodes < B || num_draft_rows < 0) return 0;
  return tree_layout(B, num_nodes + num_draft_rows, V).total;
}

int32_t tree_verify(int32_t dtype, int32_t B, int32_t V, float temperature, const int32_t* node_offsets,
                    const int32_t* parent, const int32_t* tokens, int64_t num_nodes, const void* target_logits,
                    const int32_t* draft_offsets, int64_t num_draft_rows, const void* draft_logits,
                    const float* uniforms, int32_t* num_accepted, int32_t* last_node, int32_t* final_token,
                    uint32_t* status_flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != SMCSD_F32 && dtype != SMCSD_BF16) return SMCSD_ERR_INVALID_ARG;
  if (B < 0 || V < 1 || !temperature_ok(temperature)) return SMCSD_ERR_INVALID_ARG;
  if (V > SMCSD_MAX_V) return SMCSD_ERR_UNSUPPORTED;
  // every tree has a root and at most SMCSD_TREE_MAX_NODES nodes, fewer
  // nodes with children than nodes
  if (num_nodes < B || num_nodes > (int64_t)B * SMCSD_TREE_MAX_NODES) return SMCSD_ERR_INVALID_ARG;
  if (num_draft_rows < 0 || num_draft_rows > num_nodes - B) return SMCSD_ERR_INVALID_ARG;
  if (B == 0) return SMCSD_OK;
  if (!node_offsets || !parent || !tokens || !target_logits || !draft_offsets || !uniforms || !num_accepted ||
      !last_node || !final_token)
    return SMCSD_ERR_INVALID_ARG;
  if (num_draft_rows > 0 && !draft_logits) return SMCSD_ERR_INVALID_ARG;
  const int64_t rows = num_nodes + num_draft_rows;
  const TreeLayout l = tree_layout(B, rows, V);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace % kAlign) != 0)
    return SMCSD_ERR_WORKSPACE;
  const bool bf16 = dtype == SMCSD_BF16;
  const bool vec = vec_ok(dtype, V, target_logits, num_draft_rows > 0 ? draft_logits : nullptr);
  smcsd::Plan plan;
  if (const hipError_t pe = smcsd::plan_stream(rows, ntiles_of(V), bf16, vec, false, &plan); pe != hipSuccess)
    return pe == hipErrorNotSupported ? SMCSD_ERR_UNSUPPORTED : SMCSD_ERR_HIP;
  char* ws = static_cast<char*>(workspace);
  smcsd::TreeArgs a;
  // flat streaming: group g is target row g, then draft row g - num_nodes
  fill_step(&a.s, plan, target_logits, draft_logits, nullptr, nullptr, rows, num_nodes, num_draft_rows, V, 0,
            temperature, ws, l.part, l.tpart, status_flags);
  a.s.flat = 1;
  a.node_off = node_offsets;
  a.draft_off = draft_offsets;
  a.parent = parent;
  a.tokens = tokens;
  a.uniforms = uniforms;
  a.num_accepted = num_accepted;
  a.last_node = last_node;
  a.final_token = final_token;
  a.B = B;
  a.split = 1;
  a.xchg = reinterpret_cast<uint64_t*>(ws + l.xchg);
  return smcsd::launch_tree(a, plan, bf16, vec, static_cast<hipStream_t>(stream), take_timers()) == hipSuccess
             ? SMCSD_OK
             : SMCSD_ERR_HIP;
}

size_t smc_workspace_bytes(int32_t dtype, int32_t P, int32_t N, int32_t K, int32_t V) {
  (void)dtype;
  if (P <= 0 || N <= 0 || K < 0 || V <= 0) return 0;
  return smc_layout(P, N, K, V).total;
}

}  // extern "C"

namespace {

static int32_t smc_step(int32_t dtype, int32_t P, int32_t N, int32_t K, int32_t V, float temperature,
                        float beta, float ess_frac, const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const float* bonus_uniforms,
                        const float* resample_uniforms, float* log_weights, const int32_t* page_table_in,
                        int32_t* page_table_out, int32_t pages_per_particle, int32_t* bonus_token,
                        int32_t* ancestors, float* ess, int32_t* resampled, uint32_t* status_flags,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != SMCSD_F32 && dtype != SMCSD_BF16) return SMCSD_ERR_INVALID_ARG;
  if (P < 0 || N < 1 || K < 0 || V < 1 || pages_per_particle < 0) return SMCSD_ERR_INVALID_ARG;
  if (!temperature_ok(temperature) || !isfinite(ess_frac) || ess_frac < 0.0f)
    return SMCSD_ERR_INVALID_ARG;
  // the bonus row's scale beta * log2(e) / T must be a positive finite number
  const double cb = (double)beta * 1.4426950408889634 / (double)temperature;
  if (!isfinite(beta) || !(beta > 0.0f) || !isfinite((float)cb) || !((float)cb > 0.0f)) return SMCSD_ERR_INVALID_ARG;
  if (K > SMCSD_MAX_K || N > SMCSD_MAX_N || V > SMCSD_MAX_V)
    return SMCSD_ERR_UNSUPPORTED;
  if (P == 0) return SMCSD_OK;
  const int64_t PN = (int64_t)P * N;
  if (!target_logits || !bonus_uniforms || !resample_uniforms || !log_weights || !bonus_token ||
      !ancestors || !ess || !resampled)
    return SMCSD_ERR_INVALID_ARG;
  if (K > 0 && (!draft_logits || !draft_tokens)) return SMCSD_ERR_INVALID_ARG;
  if (page_table_in && pages_per_particle > 0) {
    if (!page_table_out) return SMCSD_ERR_INVALID_ARG;
    const char* a0 = reinterpret_cast<const char*>(page_table_in);
    const char* b0 = reinterpret_cast<const char*>(page_table_out);
    const size_t bytes = sizeof(int32_t) * (size_t)PN * (size_t)pages_per_particle;
    if (a0 < b0 + bytes && b0 < a0 + bytes) return SMCSD_ERR_INVALID_ARG;
  }
  const SmcLayout l = smc_layout(P, N, K, V);
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace % kAlign) != 0)
    return SMCSD_ERR_WORKSPACE;
  const bool bf16 = dtype == SMCSD_BF16;
  const bool vec = vec_ok(dtype, V, target_logits, K > 0 ? draft_logits : nullptr);
  // a power target (beta != 1) also reduces every bonus row at the plain scale
  const bool power = beta != 1.0f;
  smcsd::Plan plan;
  const int64_t rows = PN * (2 * K + 1);
  if (const hipError_t pe = smcsd::plan_stream(rows, ntiles_of(V), bf16, vec, power, &plan); pe != hipSuccess)
    return pe == hipErrorNotSupported ? SMCSD_ERR_UNSUPPORTED : SMCSD_ERR_HIP;
  char* ws = static_cast<char*>(workspace);
  smcsd::SmcArgs a;
  fill_step(&a.s, plan, target_logits, draft_logits, nullptr, draft_tokens, PN, PN * (K + 1), PN * K, V, K,
            temperature, ws, l.part, l.tpart, status_flags);
  a.s.cb = (float)cb;
  a.s.part1 = power ? a.s.part + rows * plan.nseg : nullptr;  // after the call's own partials
  a.beta = beta;
  a.power = power ? 1 : 0;
  a.N = N;
  a.L = pages_per_particle;
  a.ess_frac = ess_frac;
  a.bonus_u = bonus_uniforms;
  a.resample_u = resample_uniforms;
  a.logw = log_weights;
  a.ws_logw = reinterpret_cast<float*>(ws + l.ws_logw);
  a.lwords = reinterpret_cast<uint64_t*>(ws + l.lwords);
  a.pt_in = page_table_in;
  a.pt_out = page_table_out;
  a.bonus_token = bonus_token;
  a.ancestors = ancestors;
  a.ess = ess;
  a.resampled = resampled;
  return smcsd::launch_smc(a, plan, bf16, vec, static_cast<hipStream_t>(stream), take_timers()) == hipSuccess
             ? SMCSD_OK
             : SMCSD_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t smc_reweight_resample(int32_t dtype, int32_t P, int32_t N, int32_t K, int32_t V,
                              float temperature, float ess_frac, const void* target_logits,
                              const void* draft_logits, const int32_t* draft_tokens,
                              const float* bonus_uniforms, const float* resample_uniforms,
                              float* log_weights, const int32_t* page_table_in,
                              int32_t* page_table_out, int32_t pages_per_particle,
                              int32_t* bonus_token, int32_t* ancestors, float* ess,
                              int32_t* resampled, uint32_t* status_flags, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return smc_step(dtype, P, N, K, V, temperature, 1.0f, ess_frac, target_logits, draft_logits, draft_tokens,
                  bonus_uniforms, resample_uniforms, log_weights, page_table_in, page_table_out,
                  pages_per_particle, bonus_token, ancestors, ess, resampled, status_flags, workspace,
                  workspace_bytes, stream);
}

int32_t smc_reweight_resample_power(int32_t dtype, int32_t P, int32_t N, int32_t K, int32_t V,
                                    float temperature, float beta, float ess_frac,
                                    const void* target_logits, const void* draft_logits,
                                    const int32_t* draft_tokens, const float* bonus_uniforms,
                                    const float* resample_uniforms, float* log_weights,
                                    const int32_t* page_table_in, int32_t* page_table_out,
                                    int32_t pages_per_particle, int32_t* bonus_token,
                                    int32_t* ancestors, float* ess, int32_t* resampled,
                                    uint32_t* status_flags, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return smc_step(dtype, P, N, K, V, temperature, beta, ess_frac, target_logits, draft_logits, draft_tokens,
                  bonus_uniforms, resample_uniforms, log_weights, page_table_in, page_table_out,
                  pages_per_particle, bonus_token, ancestors, ess, resampled, status_flags, workspace,
                  workspace_bytes, stream);
}

}  // extern "C"
