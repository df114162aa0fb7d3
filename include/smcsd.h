/*
 * smcsd.h -- C ABI of the MI355X (gfx950) verify-and-sample library.
 *
 * The verify-and-sample step of speculative decoding:
 *
 *   sd_verify              standard speculative decoding: turn the target and
 *                          draft logits of B sequences into the number of
 *                          accepted draft tokens and one final token per
 *                          sequence.
 *   smc_reweight_resample  SMC speculative decoding: reweight N particles per
 *                          prompt by their target/draft ratio, draw each
 *                          particle's (K+1)-th token, compute the effective
 *                          sample size and, when it falls below the threshold,
 *                          resample systematically and permute the particles'
 *                          KV page-table rows.
 * and the steps around it:
 *   smc_reweight_resample_power  the same SMC step for a power target p^beta;
 *   smc_pages_append / smc_pages_resample  paged-KV bookkeeping (reference
 *                          counts, free list, copy-on-write) around it;
 *   draft_sample, pacer_lengths  the draft side: token draws from q and PACER
 *                          draft lengths;
 *   tree_verify            verification of token trees.
 *
 * Where the operations are defined (pages by title and section):
 *   "Faster LLM Inference via Sequential Monte Carlo"
 *       sec. 1 Das Problem: SD is rejection sampling; the block is dropped
 *            after the first mismatch.
 *       sec. 2 Methodik, steps 1-4 and "Vorteil": N particles each draft K
 *            tokens; the target scores them in one pass; particles are
 *            reweighted by the target/draft probability ratio; they are
 *            resampled when the effective sample size falls below a threshold;
 *            every step yields exactly K+1 tokens per particle.
 *       sec. 3 Schluesselbeitraege: resampling is a metadata update of a paged
 *            KV cache (pointer operations, no data movement).
 *   "PACER: Blockwise Pre-verification for Speculative Decoding with Adaptive
 *    Length", Methodik 1-3: draft lengths vary per sequence (ragged CSR input).
 *   "Cross-Family Speculative Decoding for Polish Language Models on Apple
 *    Silicon", sec. 1: the target verifies k draft tokens in one pass.
 * The pages print no formulas.  The acceptance min(1, p/q), the residual
 * max(0, p - q), Kish's effective sample size and systematic resampling are
 * the standard definitions of the steps the pages name.
 *
 * Conventions (all indices 0-based):
 *   p_j = softmax(z_target[j] / T), q_j = softmax(z_draft[j] / T); the same
 *   temperature T scales both.  Draft token j is accepted iff u_j < p_j(x_j) /
 *   q_j(x_j) (strict).  Inverse-CDF draws pick the smallest token id i whose
 *   inclusive prefix weight exceeds u * (total weight).
 *
 * Memory and ordering:
 *   Every pointer is HIP device memory owned by the caller (for example the
 *   storage of a torch tensor) unless stated otherwise.  The library never
 *   allocates, frees or synchronises; each call enqueues its kernels on
 *   `stream` (a hipStream_t; NULL is the default stream) and returns: one that
 *   streams every logit once and one that turns the row statistics into
 *   decisions (for smc_reweight_resample a third, one to eight workgroups per
 *   prompt, for the effective sample size, the resampling and the page tables, except
 *   on the calls described below).  Outputs are valid once the stream reaches
 *   that point.  What one kernel reads from other workgroups the kernel
 *   before it wrote, with two exceptions, both taken only when the whole grid
 *   fits on the device at once: the decision kernels of sd_verify and
 *   tree_verify may run each sequence or tree on up to four workgroups that
 *   exchange single tagged words (see tree_verify), and on a
 *   smc_reweight_resample call of at most 512 particles the workgroup of each
 *   prompt's last particle collects the prompt's new log-weights as tagged
 *   words and does the prompt's work itself (no third kernel).  No other
 *   workgroup ever waits for another, so the other calls complete however
 *   much of the device they get.  Calls on one workspace
 *   must not overlap (on one stream they never do).
 *
 * Workspace:
 *   Caller-owned device scratch of at least the size the *_workspace_bytes()
 *   query returns, aligned to SMCSD_WORKSPACE_ALIGN.  A call writes every
 *   workspace byte it reads, so a workspace needs no initial contents and one
 *   workspace serves any sequence of calls of the shapes it is large enough
 *   for (the paged-KV calls' workspace is the exception: see there).
 *
 * Logits are row-major and contiguous: row r starts at element r * V.  bf16
 * logits are raw 16-bit bfloat16 patterns.
 *
 * Errors:
 *   Argument errors are found on the host and returned before anything is
 *   enqueued.  A call whose logits span more than INT32_MAX tiles of 2048
 *   (8.8 TB of bf16, more than any device holds) returns
 *   SMCSD_ERR_UNSUPPORTED.  A launch failure returns SMCSD_ERR_HIP.  Conditions that
 *   depend on the data are OR-ed as SMCSD_FLAG_* bits into *status_flags
 *   (device memory, optional, never cleared by the library).  Uniforms must
 *   lie in [0, 1); this is not checked.
 */
#ifndef SMCSD_H
#define SMCSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMCSD_OK = 0,
  SMCSD_ERR_INVALID_ARG = 1, /* bad shape, pointer, temperature or aliasing      */
  SMCSD_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels handle       */
  SMCSD_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned      */
  SMCSD_ERR_HIP = 4          /* the HIP runtime refused a launch                */
} smcsd_status;

typedef enum { SMCSD_F32 = 0, SMCSD_BF16 = 1 } smcsd_dtype;

/* Bits OR-ed into *status_flags. */
enum {
  SMCSD_FLAG_NONFINITE = 1,     /* a row held NaN or +inf, or only -inf; outputs of that
                                   sequence / prompt are unspecified                   */
  SMCSD_FLAG_ZERO_RESIDUAL = 2, /* residual mass 0 at the rejected position; the final
                                   token was drawn from p_n with the same uniform      */
  SMCSD_FLAG_ZERO_WEIGHTS = 4,  /* every particle of a prompt had log-weight -inf; no
                                   resampling, ess = 0                                 */
  SMCSD_FLAG_CDF_CLAMP = 8,     /* rounding left no prefix above u * total; the last
                                   index with positive weight was taken               */
  SMCSD_FLAG_BAD_INPUT = 16,    /* a draft token outside [0, V) (that position is
                                   rejected) or malformed CSR offsets (the outputs of
                                   the sequences they describe are unspecified); for
                                   the page bookkeeping, a state it rejects           */
  SMCSD_FLAG_PAGES_FULL = 32,   /* smc_pages_append: a row would exceed its L pages;
                                   nothing changed                                    */
  SMCSD_FLAG_PAGES_EXHAUSTED = 64, /* smc_pages_append: fewer free pages than the step
                                   needs; nothing changed                             */
  SMCSD_FLAG_WAIT_EXPIRED = 128 /* sd_verify, tree_verify: the workgroups sharing a
                                   sequence or tree did not all run within 0.1 s of
                                   each other (other work held the device); its
                                   outputs are unspecified.  smc_reweight_resample:
                                   the same for a prompt's particles on a call whose
                                   prompt work runs in the particle kernel            */
};

#define SMCSD_ABI_VERSION 3
#define SMCSD_MAX_K 128    /* largest draft length per sequence / particle      */
#define SMCSD_MAX_N 1024   /* largest particle count per prompt                 */
#define SMCSD_MAX_V 524288 /* largest vocabulary                                 */
#define SMCSD_WORKSPACE_ALIGN 256
/* Size of the static scratch of smc_reweight_resample_noalloc (one per GPU). */
#define SMCSD_NOALLOC_SCRATCH_BYTES (32u << 20)
/* Layout of the phase timestamps of a measurement build (smcsd_phase_stamps). */
#define SMCSD_STAMP_WGS 4096
#define SMCSD_STAMP_EVENTS 16

/* ABI version of the loaded library (SMCSD_ABI_VERSION it was built with). */
int32_t smcsd_abi_version(void);

/* Static, human-readable name of a status code. */
const char* smcsd_status_string(int32_t status);

/*
 * Profiling aid for benchmarks: the next sd_verify, smc_reweight_resample,
 * draft_sample or tree_verify call made by the calling thread launches its
 * two kernels so that the given
 * events take the start and stop times of the kernels themselves:
 * stream_start / stream_stop for the logit-streaming kernel, tail_start /
 * tail_stop for the decision kernel.  hipEventElapsedTime of a pair is then
 * that kernel's execution time, without the dispatch gaps around it.  Each
 * argument is a hipEvent_t created by the caller with timing enabled, or
 * NULL.  The setting is per thread and used once; not for calls under
 * stream capture.
 */
void smcsd_time_next_call(void* stream_start, void* stream_stop, void* tail_start, void* tail_stop);

/*
 * Measurement aid: the plain-read ceiling of the streaming kernel's access
 * pattern.  Reads every byte of a[0 .. a_bytes) and b[0 .. b_bytes) once with
 * the loads the logit-streaming kernel uses (16-byte non-temporal loads, 4 KiB
 * per wavefront per step, three steps in flight, the grid the device holds at
 * once) and no arithmetic, so its duration at a call's logit bytes is the
 * time those bytes take to stream with nothing else to do.
 *   a, b          device buffers, 16-byte aligned (b may be NULL with
 *                 b_bytes = 0); byte counts even.
 *   sink          device uint32 [64]: written only when the folded words hit
 *                 one fixed value (keeps the loads); contents unspecified.
 *   start_event, stop_event  hipEvent_t (timing enabled) attached to the
 *                 kernel's own start and stop, or NULL.
 * Returns SMCSD_ERR_INVALID_ARG on a NULL buffer with a nonzero size, an odd
 * size or a misaligned buffer, SMCSD_ERR_HIP when the launch fails.  One
 * kernel on `stream`; nothing allocated.
 */
int32_t smcsd_read_ceiling(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* sink,
                           void* start_event, void* stop_event, void* stream);

/*
 * Measurement aid: phase timestamps of the decision kernels of sd_verify and
 * tree_verify, recorded only by a build with -DSMCSD_PHASE_STAMPS=1 (the
 * library's own build records nothing and returns SMCSD_ERR_UNSUPPORTED).
 * Thread 0 of decision workgroup g < SMCSD_STAMP_WGS (a sequence or a tree)
 * records at its k-th event (k < SMCSD_STAMP_EVENTS) the GPU's constant
 * 100 MHz clock and a code naming the phase that just ended (0: the
 * workgroup's start).  The stamps persist on the device, one set per process,
 * until cleared; later calls overwrite the workgroups they run.
 *   host_dst   NULL, or host memory receiving the first `bytes` bytes of the
 *              uint64 array [SMCSD_STAMP_WGS][SMCSD_STAMP_EVENTS][2] (clock,
 *              code); unwritten events read 0.
 *   clear      nonzero: zero every stamp after the copy.
 * Synchronous: call it when the timed calls have finished (after a device
 * synchronisation).  Returns SMCSD_ERR_HIP when a copy fails.
 */
int32_t smcsd_phase_stamps(void* host_dst, size_t bytes, int32_t clear);

/*
 * Workspace bytes sd_verify needs for these sizes (0 when B == 0).
 * total_draft_rows is B*K for fixed K, or offsets[B] for CSR input.
 */
size_t sd_verify_workspace_bytes(int32_t dtype, int32_t B, int32_t K, int32_t V,
                                 int64_t total_draft_rows);

/*
 * Standard SD verify of B sequences.
 *
 *   dtype            SMCSD_F32 or SMCSD_BF16 (both logit tensors).
 *   B, K, V          sequences, largest draft length, vocabulary size.
 *                    0 <= K <= SMCSD_MAX_K, 1 <= V <= SMCSD_MAX_V.
 *   temperature      T > 0 and finite.
 *   target_logits    [R_t, V], R_t = total_draft_rows + B.  Sequence b's K_b + 1
 *                    target rows start at row t0_b = d0_b + b.
 *   draft_logits     [total_draft_rows, V].  Sequence b's K_b draft rows start at
 *                    row d0_b.
 *   draft_tokens     int32 [total_draft_rows], the draft token of each draft row.
 *   uniforms         fp32 [R_t].  Sequence b uses uniforms[t0_b + j] for the
 *                    accept test at position j < K_b and uniforms[t0_b + K_b]
 *                    for its final token.
 *   draft_offsets    NULL: fixed K, d0_b = b*K, K_b = K.
 *                    Else int32 [B+1] CSR offsets over draft rows: d0_b =
 *                    offsets[b], K_b = offsets[b+1] - offsets[b] <= K,
 *                    offsets[0] = 0, offsets[B] = total_draft_rows.  Malformed
 *                    offsets set SMCSD_FLAG_BAD_INPUT (checked on the device).
 *   total_draft_rows B*K when draft_offsets is NULL.
 *   num_accepted     int32 [B] out: n_b, the number of leading accepted drafts,
 *                    0 <= n_b <= K_b.
 *   final_token      int32 [B] out: if n_b < K_b, the residual draw from
 *                    max(0, p_n - q_n) at the rejected position n = n_b; if
 *                    n_b = K_b, the bonus draw from p_{K_b}.  The sequence emits
 *                    its first n_b draft tokens followed by this token.
 *   status_flags     NULL or device uint32 [1]; SMCSD_FLAG_* bits are OR-ed in.
 *   workspace        device memory of at least sd_verify_workspace_bytes(),
 *                    aligned to SMCSD_WORKSPACE_ALIGN (any contents; see
 *                    Workspace above).
 *   stream           hipStream_t.
 * Execution: with few sequences (B <= 64 on a 256-CU device, rows of four or
 * more tiles of 2048 logits; up to 128 with two), the residual pass of each
 * sequence is shared by four (two) workgroups exchanging tile masses through
 * tagged words in the workspace, as tree_verify's passes; the decisions are
 * bit-identical to one workgroup's.
 */
int32_t sd_verify(int32_t dtype, int32_t B, int32_t K, int32_t V, float temperature,
                  const void* target_logits, const void* draft_logits,
                  const int32_t* draft_tokens, const float* uniforms,
                  const int32_t* draft_offsets, int64_t total_draft_rows,
                  int32_t* num_accepted, int32_t* final_token, uint32_t* status_flags,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes smc_reweight_resample needs for these sizes (0 when P*N == 0). */
size_t smc_workspace_bytes(int32_t dtype, int32_t P, int32_t N, int32_t K, int32_t V);

/*
 * One SMC-SD step for P prompts of N particles each.  Particle i = p*N + n owns
 * target rows i*(K+1) .. i*(K+1)+K and draft rows i*K .. i*K+K-1.
 *
 *   dtype, V, temperature   as in sd_verify; 1 <= N <= SMCSD_MAX_N,
 *                           0 <= K <= SMCSD_MAX_K.
 *   ess_frac                resample a prompt iff ESS < ess_frac * N; 0 <= ess_frac,
 *                           finite (0 never resamples).
 *   target_logits           [P*N*(K+1), V].
 *   draft_logits            [P*N*K, V].
 *   draft_tokens            int32 [P*N*K].
 *   bonus_uniforms          fp32 [P*N]: the uniform of each particle's (K+1)-th
 *                           token, drawn from p_{i,K}.
 *   resample_uniforms       fp32 [P]: the systematic-resampling uniform of each
 *                           prompt.
 *   log_weights             fp32 [P*N] in/out.  In: the particles' log-weights.
 *                           Out: 0 for every particle of a prompt that resampled,
 *                           else logw + sum_{j<K} (log p_ij(x_ij) - log q_ij(x_ij)),
 *                           accumulated in fp64 and rounded once to fp32.  The
 *                           (K+1)-th token adds 0: its proposal is the target.
 *   page_table_in           NULL or int32 [P*N, L] page ids per particle.
 *   page_table_out          int32 [P*N, L] out (ignored when page_table_in is NULL):
 *                           row k = row ancestors[k] of the same prompt.  Must not
 *                           overlap page_table_in.
 *   pages_per_particle      L >= 0.
 *   bonus_token             int32 [P*N] out, in particle order before resampling.
 *   ancestors               int32 [P*N] out: local index (0..N-1) of the particle
 *                           each slot descends from; the identity when the prompt
 *                           did not resample.  Sorted ascending per prompt.
 *   ess                     fp32 [P] out: Kish ESS (sum w)^2 / sum w^2 of the
 *                           reweighted particles, w = exp(logw' - max logw').
 *   resampled               int32 [P] out: 1 iff the prompt resampled.
 *   status_flags, workspace, workspace_bytes, stream   as in sd_verify.
 */
int32_t smc_reweight_resample(int32_t dtype, int32_t P, int32_t N, int32_t K, int32_t V,
                              float temperature, float ess_frac, const void* target_logits,
                              const void* draft_logits, const int32_t* draft_tokens,
                              const float* bonus_uniforms, const float* resample_uniforms,
                              float* log_weights, const int32_t* page_table_in,
                              int32_t* page_table_out, int32_t pages_per_particle,
                              int32_t* bonus_token, int32_t* ancestors, float* ess,
                              int32_t* resampled, uint32_t* status_flags, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * The same step for a power-sampling target (the flexibility of "Faster LLM
 * Inference via Sequential Monte Carlo", sec. 3: modified targets such as
 * power sampling, without retraining): the target of a particle's tokens is
 * proportional to the product of p_j(x_j)^beta over them, p at the given
 * temperature.  Arguments as in smc_reweight_resample, plus:
 *
 *   beta                    > 0, finite, with beta / temperature finite.
 *   log_weights             Out: logw + sum_{j<K} (beta * log p_ij(x_ij)
 *                           - log q_ij(x_ij)) + log Z_i (or 0 after
 *                           resampling), p and q at the given temperature, and
 *                           Z_i = sum_y p_{i,K}(y)^beta: the (K+1)-th token is
 *                           drawn from the normalised p_{i,K}^beta / Z_i, so
 *                           its importance weight is Z_i whatever token it is.
 *   bonus_token             drawn from softmax(beta * z_{i,K} / temperature).
 *
 * beta = 1 gives exactly smc_reweight_resample's results (Z = 1, nothing
 * added).  For beta != 1 the streaming kernel also reduces every bonus row at
 * the plain scale (one more exponential per logit of those rows).  Same
 * workspace size (smc_workspace_bytes) and error codes; an invalid beta is
 * SMCSD_ERR_INVALID_ARG.
 */
int32_t smc_reweight_resample_power(int32_t dtype, int32_t P, int32_t N, int32_t K, int32_t V,
                                    float temperature, float beta, float ess_frac,
                                    const void* target_logits, const void* draft_logits,
                                    const int32_t* draft_tokens, const float* bonus_uniforms,
                                    const float* resample_uniforms, float* log_weights,
                                    const int32_t* page_table_in, int32_t* page_table_out,
                                    int32_t pages_per_particle, int32_t* bonus_token,
                                    int32_t* ancestors, float* ess, int32_t* resampled,
                                    uint32_t* status_flags, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * smc_reweight_resample for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, results and errors as smc_reweight_resample,
 * without the workspace: the kernels use a static device array of
 * SMCSD_NOALLOC_SCRATCH_BYTES (32 MiB) instead, one per GPU, held until the
 * process ends.  The call allocates nothing (no hipMalloc, no library
 * allocation); the caller still passes every input and output.
 *   A call whose workspace would exceed the array (smc_workspace_bytes(dtype,
 *   P, N, K, V) > SMCSD_NOALLOC_SCRATCH_BYTES) returns SMCSD_ERR_UNSUPPORTED
 *   before anything is enqueued; the 32-prompt x 64-particle step at K = 8,
 *   V = 151936 needs 23.4 MB.
 *   The first call on a GPU looks up that GPU's array address (no allocation);
 *   it may already be made under graph capture.
 *   Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents (nothing in it has to start at zero): calls that overlap on one
 *   GPU (two streams, two threads) race.  Calls in order on one stream do not.
 */
int32_t smc_reweight_resample_noalloc(int32_t dtype, int32_t P, int32_t N, int32_t K, int32_t V,
                                      float temperature, float ess_frac, const void* target_logits,
                                      const void* draft_logits, const int32_t* draft_tokens,
                                      const float* bonus_uniforms, const float* resample_uniforms,
                                      float* log_weights, const int32_t* page_table_in,
                                      int32_t* page_table_out, int32_t pages_per_particle,
                                      int32_t* bonus_token, int32_t* ancestors, float* ess,
                                      int32_t* resampled, uint32_t* status_flags, void* stream);

/*
 * Paged-KV bookkeeping around SMC resampling: the metadata update that makes
 * resampling a pointer operation on a page-based KV cache ("Faster LLM
 * Inference via Sequential Monte Carlo", sec. 3), with the K+1 tokens every
 * step adds per particle (sec. 2).  All arrays are device memory owned by the
 * caller; calls on one stream run in order.
 *
 * State.  A pool of num_pages (M) pages of page_size (S) token slots.
 *   page_table   int32 [P*N, L]: particle r = p*N + n; its first
 *                ceil(seq_len[r] / S) entries are page ids in [0, M).
 *   seq_len      int32 [P*N]: tokens per particle, 0 <= len <= L*S.
 *   ref_count    int32 [M]: entries naming each page; it must equal the table
 *                (not checked).  A partially filled page is named only as the
 *                last used entry (tail) of rows, so its count is the number of
 *                rows whose tail it is (checked by smc_pages_append).
 *   free_pages   int32 [M], free_count int32 [1]: the pages with count 0, a
 *                stack whose top is free_pages[free_count - 1].
 * Both calls need a workspace of smc_pages_workspace_bytes(P, N, L, M),
 * SMCSD_WORKSPACE_ALIGN aligned, zero-filled before its first use; every call
 * leaves at zero what has to start there, so one workspace serves every call
 * of those sizes (not two calls at once).
 * Requirements: N >= 1, L >= 1, S >= 1, M >= 1, (P*N)*L and L*S and M below
 * 2^31; otherwise SMCSD_ERR_INVALID_ARG.
 */
size_t smc_pages_workspace_bytes(int32_t P, int32_t N, int32_t L, int64_t num_pages);

/*
 * Adds new_tokens (A = K+1) token slots to every particle, particles in index
 * order: a partially filled tail page that other rows also name is copied on
 * write (a fresh page from the top of the stack; the copy is listed; the row
 * names the fresh page, the old page's count drops by one) unless this row is
 * the last (highest index) of its sharers, which keeps it; then one fresh page
 * per further position the A tokens reach (count 1).
 *   slots        int32 [P*N, A] out: page * S + offset of each new token.
 *   cow_list     int32 [P*N, 3] out: (source page, destination page, tokens to
 *                copy = old len % S) per copy, in particle order; *cow_count
 *                (int32 [1]) out: their number.  The caller copies the KV data.
 * page_table, seq_len (len += A), ref_count and free_count are updated in
 * place; free_pages is only read.  A row that would exceed L pages
 * (SMCSD_FLAG_PAGES_FULL), too few free pages (SMCSD_FLAG_PAGES_EXHAUSTED) or a
 * rejected state (SMCSD_FLAG_BAD_INPUT) change nothing.
 */
int32_t smc_pages_append(int32_t P, int32_t N, int32_t L, int32_t page_size, int32_t new_tokens,
                         int64_t num_pages, int32_t* page_table, int32_t* seq_len, int32_t* ref_count,
                         const int32_t* free_pages, int32_t* free_count, int32_t* slots, int32_t* cow_list,
                         int32_t* cow_count, uint32_t* status_flags, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * The bookkeeping of a resampling step, after smc_reweight_resample.
 *   ancestors       int32 [P*N]: local ancestor (0..N-1) of each slot.
 *   page_table_old  the rows before resampling (page_table_in of the step);
 *                   the new rows are the ancestors' old rows (its
 *                   page_table_out: row r = old row p*N + ancestors[r]), which
 *                   is all the call assumes of them; it does not read them.
 *   seq_len_in      lengths before; seq_len_out (out, must not overlap it):
 *                   seq_len_out[r] = seq_len_in[p*N + ancestors[r]].
 * Every entry of a new row counts its page once more and every entry of an old
 * row once less, so a page's count changes by the sum of (copies - 1) over the
 * old rows naming it, copies = the slots whose ancestor the row is; the pages
 * that reach zero are pushed on the free stack in the order of their first
 * entry in the old rows (row, then position).  ref_count, free_pages and
 * free_count are updated in place.  An ancestor or length out of range, or a
 * page id out of range in a row that is dropped or copied, raises
 * SMCSD_FLAG_BAD_INPUT (the state is then unspecified).
 */
int32_t smc_pages_resample(int32_t P, int32_t N, int32_t L, int32_t page_size, int64_t num_pages,
                           const int32_t* ancestors, const int32_t* page_table_old, const int32_t* seq_len_in,
                           int32_t* seq_len_out, int32_t* ref_count, int32_t* free_pages, int32_t* free_count,
                           uint32_t* status_flags, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Draft side: the steps just before verification.
 * ------------------------------------------------------------------------ */

/*
 * One token per row drawn from the draft distribution ("Faster LLM Inference
 * via Sequential Monte Carlo", sec. 2 step 1: the draft model extends every
 * particle, or sequence, by one token per draft position).
 *   logits    [R, V] fp32 or bf16 (dtype as for sd_verify), row-major, device.
 *   uniforms  float [R] in [0, 1), device, one per row.
 *   tokens    int32 [R] out, device: the smallest token id whose inclusive
 *             prefix sum of softmax(z / T) exceeds uniforms[r] times the row
 *             total (strict comparison, ascending token id); if rounding
 *             leaves none, the last token of positive probability
 *             (SMCSD_FLAG_CDF_CLAMP).  This is the convention of every draw
 *             in this library: the call is sd_verify's final draw with no
 *             draft tokens, on the same kernels.
 * Workspace: draft_sample_workspace_bytes(dtype, R, V) bytes, aligned as for
 * sd_verify (the same workspace may serve both).  Errors and flags as for sd_verify (SMCSD_FLAG_NONFINITE for a
 * row that is not a distribution; its token is then unspecified).
 */
size_t draft_sample_workspace_bytes(int32_t dtype, int32_t R, int32_t V);
int32_t draft_sample(int32_t dtype, int32_t R, int32_t V, float temperature, const void* logits,
                     const float* uniforms, int32_t* tokens, uint32_t* status_flags, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * PACER draft lengths ("PACER: Blockwise Pre-verification for Speculative
 * Decoding with Adaptive Length", Methodik 1-3: drafting in blocks; after each
 * block the pre-verifier's mean estimated acceptance of its tokens is compared
 * with a threshold t; below it the drafting stops, otherwise t grows by the
 * factor rho and another block follows).
 *   scores   float [B, max_blocks * block], device: the estimated acceptance of
 *            each drafted token, block after block.  Scores after a
 *            sequence's stopping block are not read.
 *   lengths  int32 [B] out, device: K_b = block * m, m the first block whose
 *            mean (its scores summed in index order in double, divided by
 *            block) is below t (strictly), or max_blocks; t starts at t0 and
 *            is multiplied by rho (in double) after every block that goes on.
 *            A NaN mean never stops a sequence.
 *   offsets  int32 [B + 1] out, device: 0, then the running sums of lengths
 *            (the draft_offsets of a ragged sd_verify).
 * One workgroup; no workspace.  Requirements: B >= 0, block >= 1,
 * max_blocks >= 1, B * max_blocks * block <= 2^31 - 1, t0 and rho finite;
 * otherwise SMCSD_ERR_INVALID_ARG.
 */
int32_t pacer_lengths(int32_t B, int32_t block, int32_t max_blocks, double t0, double rho, const float* scores,
                      int32_t* lengths, int32_t* offsets, void* stream);

/* ------------------------------------------------------------------------
 * Tree verification.
 * ------------------------------------------------------------------------ */

#define SMCSD_TREE_MAX_NODES 256 /* largest token tree (nodes, root included) */

/*
 * Verify B token trees ("Faster LLM Inference via Sequential Monte Carlo",
 * sec. 4: SMC-SD is measured against tree-based speculative decoding; the
 * pages give no algorithm for verifying a tree, and this is multi-draft
 * speculative sampling, the textbook way to check several draft
 * continuations against one target distribution):
 *   at node u the running distribution r starts as p_u; the children of u
 *   are tried in increasing node index, child c (token x_c) accepted iff
 *   u_c < r(x_c) / q_u(x_c) (strict), and the walk moves to c; a rejection
 *   turns r into max(0, r - q_u) / Z, Z its total (if Z is 0, r stays and
 *   SMCSD_FLAG_ZERO_RESIDUAL is raised).  The walk stops at a leaf (final
 *   token drawn from p_leaf) or at a node whose children were all rejected
 *   (final token drawn from the last max(0, r - q_u)).  A chain of K+1 nodes
 *   is sd_verify with K draft tokens, decision for decision.
 * Execution: when few trees leave most of the device idle (B <= 64 trees of
 *   two or more tiles on a 256-CU device), the decision kernel runs each tree
 *   on up to four workgroups: each walks the whole tree, weighs every fourth
 *   tile of a rejection pass and reads the other tiles' masses from the other
 *   workgroups through tagged words in the workspace (one relaxed device-scope
 *   64-bit atomic per value; the streaming kernel of the same call zeroes
 *   them).  The decisions are bit-identical to a single workgroup's.  A
 *   workgroup waits at most 0.1 s for the others; past that it raises
 *   SMCSD_FLAG_WAIT_EXPIRED.
 * Layout (all device memory, caller-owned):
 *   node_offsets   int32 [B+1]: tree b owns nodes node_offsets[b] ..
 *                  node_offsets[b+1]-1 (1 <= M_b <= SMCSD_TREE_MAX_NODES),
 *                  node_offsets[0] = 0, node_offsets[B] = num_nodes.
 *   parent         int32 [num_nodes]: local index of each node's parent;
 *                  -1 for node 0 (the root, the last committed token), and
 *                  0 <= parent < n for every other node n.
 *   tokens         int32 [num_nodes]: the draft token of each node (the
 *                  root's entry is not read).
 *   target_logits  [num_nodes, V]: row node_offsets[b] + n holds the target's
 *                  logits after the path root .. n.
 *   draft_offsets  int32 [B+1]: tree b owns draft rows draft_offsets[b] ..
 *                  draft_offsets[b+1]-1, one per node with at least one
 *                  child, in node order (the draft logits its children were
 *                  drawn from); draft_offsets[B] = num_draft_rows.
 *   draft_logits   [num_draft_rows, V].
 *   uniforms       float [num_nodes]: entry node_offsets[b] + n (n >= 1) is
 *                  node n's acceptance uniform; the root's entry is the final
 *                  draw's uniform.
 *   num_accepted   int32 [B] out: depth of the node where the walk stopped
 *                  (the accepted tokens are those of the path root .. it).
 *   last_node      int32 [B] out: local index of that node.
 *   final_token    int32 [B] out: the token drawn there.
 * Workspace: tree_verify_workspace_bytes(...) bytes, as for sd_verify.
 * Errors: SMCSD_ERR_INVALID_ARG for bad sizes, pointers or temperature;
 * SMCSD_ERR_UNSUPPORTED for V > SMCSD_MAX_V.  A tree whose offsets, parents
 * or draft-row count disagree with the rules above raises
 * SMCSD_FLAG_BAD_INPUT and its outputs are unspecified; a token outside
 * [0, V) is a rejection and raises SMCSD_FLAG_BAD_INPUT; flags otherwise as
 * for sd_verify.
 */
size_t tree_verify_workspace_bytes(int32_t dtype, int32_t B, int32_t V, int64_t num_nodes, int64_t num_draft_rows);
int32_t tree_verify(int32_t dtype, int32_t B, int32_t V, float temperature, const int32_t* node_offsets,
                    const int32_t* parent, const int32_t* tokens, int64_t num_nodes, const void* target_logits,
                    const int32_t* draft_offsets, int64_t num_draft_rows, const void* draft_logits,
                    const float* uniforms, int32_t* num_accepted, int32_t* last_node, int32_t* final_token,
                    uint32_t* status_flags, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SMCSD_H */
