/*
 * oracle.c -- plain, slow, sequential fp64 CPU reference of the
 * verify-and-sample step of speculative decoding (SD) and of the
 * reweight / ESS / resample step of SMC speculative decoding (SMC-SD).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * reads this file.  Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or helper with the GPU path.
 *
 * Sources (pages by title and section):
 *   [SMC]   "Faster LLM Inference via Sequential Monte Carlo"
 *           sec. 1 (Das Problem): SD is rejection sampling and drops the rest of
 *           the block at the first mismatch;
 *           sec. 2 (Methodik), steps 1-4: draft K tokens per particle, score
 *           them with the target, reweight by the target/draft probability
 *           ratio, resample when the effective sample size falls below a
 *           threshold; every step yields exactly K+1 tokens per particle;
 *           sec. 3 (Schluesselbeitraege): resampling is a pointer / page-table
 *           metadata update of a paged KV cache.
 *   [XFAM]  "Cross-Family Speculative Decoding for Polish Language Models on
 *           Apple Silicon", sec. 1: the target verifies k draft tokens at once.
 *   [PACER] "PACER: Blockwise Pre-verification for Speculative Decoding with
 *           Adaptive Length", Methodik 1-3: per-sequence draft lengths vary.
 * The pages print no formulas.  Where they name a step without a formula the
 * textbook definition is used and named at that function: the SD acceptance
 * min(1, p/q) and residual max(0, p - q) (standard speculative sampling), the
 * Kish effective sample size, and systematic resampling.
 *
 * Conventions fixed here (each one is a reading of a silent point):
 *   - logits are read exactly as stored (fp32, or bf16 widened exactly);
 *   - a_i = z_i / T, M = max_i a_i, S = sum_i exp(a_i - M) summed in index
 *     order, log p(i) = a_i - M - log S;
 *   - accept draft token j iff u_j < p_j(x_j) / q_j(x_j) (strict; a tie
 *     rejects);
 *   - inverse CDF: smallest index i (ascending token id) whose inclusive
 *     prefix sum C_i exceeds u * Z, strictly; if rounding leaves no such i,
 *     the last index with positive weight (flag CDF_CLAMP);
 *   - zero residual mass at the rejected position: sample p_n instead with
 *     the same uniform (flag ZERO_RESIDUAL);
 *   - SD uniforms per sequence: K_b accept uniforms, then one final uniform;
 *   - SMC: the (K+1)-th token is drawn from the target row K; its proposal is
 *     the target itself, so it adds log p - log p = 0 to the log-weight;
 *   - ESS = (sum w)^2 / sum w^2 with w_i = exp(logw_i - max logw);
 *     resample iff ESS < ess_frac * N (strict);
 *   - systematic resampling: U_k = (u + k) / N, a_k = smallest i with
 *     C_i > U_k, C the normalised inclusive cumulative weight; after
 *     resampling every log-weight is 0;
 *   - page tables: row k of the output is row a_k of the input;
 *   - power target ([SMC] sec. 3, Flexibilitaet: the framework also targets
 *     modified distributions such as power sampling, without retraining): the
 *     target of a particle's tokens is proportional to the product of
 *     p_j(x_j)^beta over them.  A draft token (proposal q) adds
 *     beta * log p - log q to the log-weight.  The (K+1)-th token comes from
 *     the normalised softmax(beta * z / T) = p_K^beta / Z_beta, i.e.
 *     temperature T / beta, so its importance weight is
 *     p_K(y)^beta / (p_K(y)^beta / Z_beta) = Z_beta = sum_y p_K(y)^beta, the
 *     same for every y: it adds log Z_beta.  beta = 1 is the plain step above
 *     (Z_1 = 1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* status bits (same meaning as the library's device flags) */
#define ORACLE_FLAG_NONFINITE 1u
#define ORACLE_FLAG_ZERO_RESIDUAL 2u
#define ORACLE_FLAG_ZERO_WEIGHTS 4u
#define ORACLE_FLAG_CDF_CLAMP 8u

/* dtype codes: 0 = fp32, 1 = bf16 (raw 16-bit patterns) */
double oracle_logit(int dtype, const void* row, int64_t i) {
  if (dtype == 0) return (double)((const float*)row)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)row)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static const void* row_ptr(int dtype, const void* base, int64_t row, int64_t V) {
  size_t esz = dtype == 0 ? 4 : 2;
  return (const char*)base + (size_t)row * (size_t)V * esz;
}

/*
 * Temperature softmax statistics of one row [SMC sec. 2 step 3 needs
 * normalised target and draft probabilities; the temperature scales both].
 * Returns 1 when the row is not a distribution (NaN or +inf logit, or every
 * logit -inf), else 0.
 */
int oracle_row_stats(int dtype, const void* row, int64_t V, double T, double* M_out,
                     double* logS_out) {
  double M = -INFINITY;
  int bad = 0;
  for (int64_t i = 0; i < V; i++) {
    double z = oracle_logit(dtype, row, i);
    if (isnan(z) || z == INFINITY) bad = 1;
    double a = z / T;
    if (a > M) M = a;
  }
  if (M == -INFINITY) bad = 1;
  double S = 0.0;
  for (int64_t i = 0; i < V; i++) S += exp(oracle_logit(dtype, row, i) / T - M);
  *M_out = M;
  *logS_out = log(S);
  return bad;
}

/* log p(i) of a row whose statistics are (M, logS). */
static double logprob_with(int dtype, const void* row, int64_t i, double T, double M,
                           double logS) {
  return oracle_logit(dtype, row, i) / T - M - logS;
}

/* Convenience: log p(i) of a row, computing its statistics. */
double oracle_logprob(int dtype, const void* row, int64_t V, double T, int64_t i) {
  double M, logS;
  oracle_row_stats(dtype, row, V, T, &M, &logS);
  return logprob_with(dtype, row, i, T, M, logS);
}

/*
 * Inverse-CDF draw from non-negative weights w[0..n) with uniform u in [0,1).
 * Returns the index; *margin receives the distance, in units of u, from u to
 * the nearer edge of the chosen index's CDF interval (0 when clamped).
 */
static int64_t inverse_cdf(const double* w, int64_t n, double u, double* margin,
                           uint32_t* flags) {
  double Z = 0.0;
  for (int64_t i = 0; i < n; i++) Z += w[i];
  double target = u * Z;
  double C = 0.0;
  for (int64_t i = 0; i < n; i++) {
    double Cprev = C;
    C += w[i];
    if (C > target) {
      if (margin) {
        double lo = u - Cprev / Z, hi = C / Z - u;
        *margin = lo < hi ? lo : hi;
      }
      return i;
    }
  }
  *flags |= ORACLE_FLAG_CDF_CLAMP;
  if (margin) *margin = 0.0;
  for (int64_t i = n - 1; i >= 0; i--)
    if (w[i] > 0.0) return i;
  return n - 1;
}

/*
 * Weights of the distribution the final SD token is drawn from, for one
 * sequence whose first rejection is at position n (n == K_b: all accepted).
 *   residual  (n <  K_b): w_i = max(0, p_n(i) - q_n(i))   [standard SD]
 *   bonus     (n == K_b): w_i = p_{K_b}(i)                 [K+1-th token]
 *   fallback  (residual mass exactly 0): w_i = p_n(i), flag ZERO_RESIDUAL.
 */
static void final_weights(int dtype, const void* trow, const void* drow, int64_t V,
                          double T, double* w, uint32_t* flags) {
  double Mt, lSt;
  if (oracle_row_stats(dtype, trow, V, T, &Mt, &lSt)) *flags |= ORACLE_FLAG_NONFINITE;
  if (!drow) {
    for (int64_t i = 0; i < V; i++) w[i] = exp(logprob_with(dtype, trow, i, T, Mt, lSt));
    return;
  }
  double Md, lSd;
  if (oracle_row_stats(dtype, drow, V, T, &Md, &lSd)) *flags |= ORACLE_FLAG_NONFINITE;
  double Z = 0.0;
  for (int64_t i = 0; i < V; i++) {
    double p = exp(logprob_with(dtype, trow, i, T, Mt, lSt));
    double q = exp(logprob_with(dtype, drow, i, T, Md, lSd));
    w[i] = p - q > 0.0 ? p - q : 0.0;
    Z += w[i];
  }
  if (Z == 0.0) {
    *flags |= ORACLE_FLAG_ZERO_RESIDUAL;
    for (int64_t i = 0; i < V; i++) w[i] = exp(logprob_with(dtype, trow, i, T, Mt, lSt));
  }
}

/* Sequence b's draft-row base and draft length (fixed K or CSR offsets). */
static void seq_layout(int b, int K, const int32_t* offsets, int64_t* d0, int* Kb) {
  if (offsets) {
    *d0 = offsets[b];
    *Kb = offsets[b + 1] - offsets[b];
  } else {
    *d0 = (int64_t)b * K;
    *Kb = K;
  }
}

/*
 * Standard SD verify of B sequences [SMC sec. 1; XFAM sec. 1; PACER Methodik
 * for ragged lengths].  Sequence b has K_b draft rows starting at draft row
 * d0 = offsets[b] (or b*K) and K_b + 1 target rows starting at target row
 * d0 + b; its uniforms start at the same index d0 + b.
 *
 * accept_margin[d0 + j]: |u_j - min(1, rho_j)| for each evaluated position j,
 *                        -1 for positions after the first rejection.
 * sample_margin[b]:      margin of the final inverse-CDF draw.
 * Returns 0.
 */
int oracle_sd_verify(int dtype, int B, int K, int64_t V, double T, const void* target,
                     const void* draft, const int32_t* tokens, const float* uniforms,
                     const int32_t* offsets, int32_t* num_accepted, int32_t* final_token,
                     uint32_t* flags, double* accept_margin, double* sample_margin) {
  double* w = (double*)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
  uint32_t fl = 0;
  for (int b = 0; b < B; b++) {
    int64_t d0;
    int Kb;
    seq_layout(b, K, offsets, &d0, &Kb);
    int64_t t0 = d0 + b;
    int n = Kb;
    for (int j = 0; j < Kb; j++) {
      const void* trow = row_ptr(dtype, target, t0 + j, V);
      const void* drow = row_ptr(dtype, draft, d0 + j, V);
      int32_t x = tokens[d0 + j];
      double Mt, lSt, Md, lSd;
      if (oracle_row_stats(dtype, trow, V, T, &Mt, &lSt)) fl |= ORACLE_FLAG_NONFINITE;
      if (oracle_row_stats(dtype, drow, V, T, &Md, &lSd)) fl |= ORACLE_FLAG_NONFINITE;
      double lp = logprob_with(dtype, trow, x, T, Mt, lSt);
      double lq = logprob_with(dtype, drow, x, T, Md, lSd);
      double rho = exp(lp - lq);
      double u = (double)uniforms[t0 + j];
      if (accept_margin) accept_margin[d0 + j] = fabs(u - (rho < 1.0 ? rho : 1.0));
      if (!(u < rho)) {
        n = j;
        break;
      }
    }
    if (accept_margin)
      for (int j = n + 1; j < Kb; j++) accept_margin[d0 + j] = -1.0;
    num_accepted[b] = n;
    const void* trow = row_ptr(dtype, target, t0 + n, V);
    const void* drow = n < Kb ? row_ptr(dtype, draft, d0 + n, V) : NULL;
    final_weights(dtype, trow, drow, V, T, w, &fl);
    double m = 0.0;
    final_token[b] = (int32_t)inverse_cdf(w, V, (double)uniforms[t0 + Kb], &m, &fl);
    if (sample_margin) sample_margin[b] = m;
  }
  free(w);
  if (flags) *flags |= fl;
  return 0;
}

/*
 * Normalised CDF (C_i / Z, i = 0..V-1) of the distribution sequence b's final
 * token is drawn from, given its number of accepted tokens n.  Used by the
 * comparison to judge a differing token against the decision band.
 */
int oracle_sd_final_cdf(int dtype, int b, int K, int64_t V, double T, const void* target,
                        const void* draft, const int32_t* offsets, int n, double* cdf) {
  int64_t d0;
  int Kb;
  seq_layout(b, K, offsets, &d0, &Kb);
  uint32_t fl = 0;
  const void* trow = row_ptr(dtype, target, d0 + b + n, V);
  const void* drow = n < Kb ? row_ptr(dtype, draft, d0 + n, V) : NULL;
  final_weights(dtype, trow, drow, V, T, cdf, &fl);
  double Z = 0.0;
  for (int64_t i = 0; i < V; i++) Z += cdf[i];
  double C = 0.0;
  for (int64_t i = 0; i < V; i++) {
    C += cdf[i];
    cdf[i] = C / Z;
  }
  return (int)fl;
}

/*
 * One SMC-SD step for P prompts of N particles each [SMC sec. 2 steps 3-4 and
 * the K+1 tokens per step; sec. 3 pointer-only resampling].
 * Particle i = p*N + n owns target rows i*(K+1) .. i*(K+1)+K and draft rows
 * i*K .. i*K+K-1.
 *
 *   log-weight:   logw'_i = fp32(logw_i + sum_{j<K} (beta log p_ij(x_ij) - log q_ij(x_ij))
 *                                   + log sum_y p_{i,K}(y)^beta)
 *   bonus token:  inverse CDF of softmax(beta z_{i,K} / T) with bonus_u[i]
 *                 (beta = 1 for the plain step: p_{i,K}, and the last term is 0)
 *   ESS:          Kish, (sum w)^2 / sum w^2, w_i = exp(logw'_i - max)
 *   resample iff ESS < ess_frac * N: systematic with resample_u[p];
 *                 ancestors (local indices), logw_out = 0, page-table rows
 *                 gathered by ancestor; otherwise identity and logw_out = logw'.
 *
 * logw is updated in place.  pt_in / pt_out may be NULL (L ignored).
 * cum_weight[i] (optional) receives the normalised inclusive cumulative weight
 * C_i used by the systematic draw (or -1 when the prompt did not resample);
 * bonus_margin[i], ess_margin[p] = |ESS - ess_frac*N| / N and
 * resample_margin[p] = min_k distance of U_k to its interval edges (optional).
 * Returns 0.
 */
int oracle_smc_step_power(int dtype, int P, int N, int K, int64_t V, double T, double beta,
                          double ess_frac, const void* target, const void* draft,
                          const int32_t* tokens, const float* bonus_u, const float* resample_u,
                          float* logw, const int32_t* pt_in, int32_t* pt_out, int L,
                          int32_t* bonus, int32_t* ancestors, float* ess, int32_t* resampled,
                          uint32_t* flags, double* cum_weight, double* bonus_margin,
                          double* ess_margin, double* resample_margin) {
  double* w = (double*)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
  double* pw = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  double* C = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  float* lw = (float*)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
  uint32_t fl = 0;
  for (int p = 0; p < P; p++) {
    /* reweight each particle by the target/draft ratio of its K draft tokens */
    for (int n = 0; n < N; n++) {
      int64_t i = (int64_t)p * N + n;
      double delta = 0.0;
      for (int j = 0; j < K; j++) {
        const void* trow = row_ptr(dtype, target, i * (K + 1) + j, V);
        const void* drow = row_ptr(dtype, draft, i * K + j, V);
        int32_t x = tokens[i * K + j];
        double Mt, lSt, Md, lSd;
        if (oracle_row_stats(dtype, trow, V, T, &Mt, &lSt)) fl |= ORACLE_FLAG_NONFINITE;
        if (oracle_row_stats(dtype, drow, V, T, &Md, &lSd)) fl |= ORACLE_FLAG_NONFINITE;
        delta += beta * logprob_with(dtype, trow, x, T, Mt, lSt) - logprob_with(dtype, drow, x, T, Md, lSd);
      }
      /* the (K+1)-th token's weight Z_beta = sum_y p_K(y)^beta.  With
       * p_K(y) = exp(a_y - M - log S), a_y = z_y / T:
       *   Z_beta = exp(-beta log S) * sum_y exp(beta (a_y - M)),
       * so log Z_beta = log S_beta - beta log S, S_beta the second sum.  At
       * beta = 1, Z_1 = 1 (p_K sums to one) and nothing is added. */
      const void* brow = row_ptr(dtype, target, i * (K + 1) + K, V);
      if (beta != 1.0) {
        double Mk, lSk;
        if (oracle_row_stats(dtype, brow, V, T, &Mk, &lSk)) fl |= ORACLE_FLAG_NONFINITE;
        double Sb = 0.0;
        for (int64_t y = 0; y < V; y++) Sb += exp(beta * (oracle_logit(dtype, brow, y) / T - Mk));
        delta += log(Sb) - beta * lSk;
      }
      lw[n] = (float)((double)logw[i] + delta);
      if (isnan(lw[n]) || lw[n] == INFINITY) fl |= ORACLE_FLAG_NONFINITE;
      /* the (K+1)-th token, drawn from the target's row K (power: at T / beta) */
      final_weights(dtype, brow, NULL, V, T / beta, w, &fl);
      double m = 0.0;
      bonus[i] = (int32_t)inverse_cdf(w, V, (double)bonus_u[i], &m, &fl);
      if (bonus_margin) bonus_margin[i] = m;
    }
    /* effective sample size of the normalised weights */
    double M = -INFINITY;
    for (int n = 0; n < N; n++)
      if ((double)lw[n] > M) M = (double)lw[n];
    double Sw = 0.0, Sw2 = 0.0;
    int do_resample = 0;
    double E = 0.0;
    if (M == -INFINITY) {
      fl |= ORACLE_FLAG_ZERO_WEIGHTS;
    } else {
      for (int n = 0; n < N; n++) {
        pw[n] = exp((double)lw[n] - M);
        Sw += pw[n];
        Sw2 += pw[n] * pw[n];
      }
      E = Sw * Sw / Sw2;
      do_resample = E < ess_frac * N;
    }
    ess[p] = (float)E;
    if (ess_margin) ess_margin[p] = fabs(E - ess_frac * N) / N;
    resampled[p] = do_resample;
    double rmargin = INFINITY;
    if (do_resample) {
      double acc = 0.0;
      for (int n = 0; n < N; n++) {
        acc += pw[n];
        C[n] = acc / Sw;
      }
      for (int k = 0; k < N; k++) {
        double U = ((double)resample_u[p] + k) / N;
        int a = -1;
        for (int n = 0; n < N; n++)
          if (C[n] > U) {
            a = n;
            break;
          }
        if (a < 0) {
          fl |= ORACLE_FLAG_CDF_CLAMP;
          for (a = N - 1; a > 0 && pw[a] == 0.0; a--) {
          }
          rmargin = 0.0;
        } else {
          double lo = U - (a > 0 ? C[a - 1] : 0.0), hi = C[a] - U;
          double mm = lo < hi ? lo : hi;
          if (mm < rmargin) rmargin = mm;
        }
        ancestors[(int64_t)p * N + k] = a;
      }
    } else {
      for (int k = 0; k < N; k++) ancestors[(int64_t)p * N + k] = k;
    }
    if (resample_margin) resample_margin[p] = rmargin;
    for (int k = 0; k < N; k++) {
      int64_t i = (int64_t)p * N + k;
      if (cum_weight) cum_weight[i] = do_resample ? C[k] : -1.0;
      logw[i] = do_resample ? 0.0f : lw[k];
      if (pt_in && pt_out) {
        int64_t src = (int64_t)p * N + ancestors[i];
        for (int l = 0; l < L; l++) pt_out[i * L + l] = pt_in[src * L + l];
      }
    }
  }
  free(w);
  free(pw);
  free(C);
  free(lw);
  if (flags) *flags |= fl;
  return 0;
}

/* The plain SMC-SD step: the power step with beta = 1 (1 * x and T / 1 are
 * exact, so the arithmetic is the same). */
int oracle_smc_step(int dtype, int P, int N, int K, int64_t V, double T, double ess_frac,
                    const void* target, const void* draft, const int32_t* tokens,
                    const float* bonus_u, const float* resample_u, float* logw,
                    const int32_t* pt_in, int32_t* pt_out, int L, int32_t* bonus,
                    int32_t* ancestors, float* ess, int32_t* resampled, uint32_t* flags,
                    double* cum_weight, double* bonus_margin, double* ess_margin,
                    double* resample_margin) {
  return oracle_smc_step_power(dtype, P, N, K, V, T, 1.0, ess_frac, target, draft, tokens, bonus_u,
                               resample_u, logw, pt_in, pt_out, L, bonus, ancestors, ess, resampled,
                               flags, cum_weight, bonus_margin, ess_margin, resample_margin);
}

/* ---------------------------------------------------------------------------
 * Paged-KV bookkeeping around SMC resampling ([SMC] sec. 3: resampling is a
 * pointer / metadata update of a page-based KV cache, no data movement; sec. 2:
 * every step adds exactly K+1 tokens per particle).  The pages give no data
 * structure; the reading fixed here:
 *   - a pool of M pages of S token slots; particle r (r = p*N + n) has a
 *     page-table row of L entries and a length len[r]; its first
 *     ceil(len[r] / S) entries are page ids, the others -1;
 *   - ref[page] = number of page-table entries (of used positions) naming it;
 *     a page with ref 0 is free, and the free pages are a stack
 *     free_pages[0 .. free_count-1] (top = free_count-1);
 *   - the reference counts equal the entries naming each page (assumed, not
 *     checked), and a partially filled page is named only as the last used
 *     entry (the tail) of rows (what resampling produces): its count must equal
 *     the number of rows whose tail it is, else the state is rejected.
 * Append (A = K+1 new tokens per particle), particles in index order:
 *   if the tail page is partially filled and ref > 1, copy on write: pop a page,
 *   list the copy (source page, destination page, tokens to copy = len % S),
 *   ref[source] -= 1, ref[new] = 1, and the row names the new page; then pop one
 *   page (ref 1) per further position the A tokens reach; slot t of particle r
 *   is page * S + offset of position len + t; len += A.  Pops take the top of
 *   the stack.  If some row would exceed L pages, or the pops exceed the free
 *   pages, nothing changes (status 1 or 2).
 * Resample (ancestors a_k of each prompt, new rows already gathered):
 *   len_out[k] = len_in[a_k]; every entry of a new row adds 1 to its page's ref,
 *   every entry of an old row subtracts 1; the pages whose ref reaches 0 are
 *   pushed in the order of their first entry in the old rows (row, then
 *   position).
 * ------------------------------------------------------------------------- */
static int64_t used_pages(int32_t len, int S) { return ((int64_t)len + S - 1) / S; }

/* Returns 0, or 1 (a row would exceed L pages), 2 (not enough free pages),
 * 3 (the state breaks the sharing rule); on a non-zero return nothing changes. */
int oracle_pages_append(int R, int L, int S, int A, int64_t M, int32_t* table, int32_t* len,
                        int32_t* ref, int32_t* free_pages, int32_t* free_count, int32_t* slots,
                        int32_t* cow, int32_t* n_cow) {
  /* check the sharing rule: the count of a partially filled tail page equals
   * the number of rows whose tail it is (tail ids must be pages of the pool) */
  int32_t* tails = (int32_t*)calloc((size_t)(M > 0 ? M : 1), sizeof(int32_t));
  int bad = 0;
  for (int r = 0; r < R; r++) {
    if (len[r] < 0 || used_pages(len[r], S) > L) bad = 1;
    else if (len[r] % S) {
      int32_t pg = table[(int64_t)r * L + used_pages(len[r], S) - 1];
      if (pg < 0 || pg >= M) bad = 1;
      else tails[pg]++;
    }
  }
  for (int r = 0; r < R && !bad; r++) {
    if (len[r] % S) {
      int32_t pg = table[(int64_t)r * L + used_pages(len[r], S) - 1];
      if (tails[pg] != ref[pg]) bad = 1;
    }
  }
  free(tails);
  if (bad) return 3;
  /* dry run on a copy of the ref counts: capacity and pages needed */
  int32_t* rc = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1));
  memcpy(rc, ref, sizeof(int32_t) * (size_t)M);
  int64_t need = 0;
  for (int r = 0; r < R; r++) {
    int64_t u0 = used_pages(len[r], S), u1 = used_pages(len[r] + A, S);
    if (u1 > L) {
      free(rc);
      return 1;
    }
    if (len[r] % S) {
      int32_t tail = table[(int64_t)r * L + u0 - 1];
      if (rc[tail] > 1) {
        rc[tail]--;
        need++;
      }
    }
    need += u1 - u0;
  }
  free(rc);
  if (need > *free_count) return 2;
  /* apply */
  int32_t top = *free_count, nc = 0;
  for (int r = 0; r < R; r++) {
    int32_t* row = table + (int64_t)r * L;
    int64_t u0 = used_pages(len[r], S), u1 = used_pages(len[r] + A, S);
    if (len[r] % S) {
      int32_t tail = row[u0 - 1];
      if (ref[tail] > 1) {
        int32_t q = free_pages[--top];
        cow[3 * nc] = tail;
        cow[3 * nc + 1] = q;
        cow[3 * nc + 2] = len[r] % S;
        nc++;
        ref[tail]--;
        ref[q] = 1;
        row[u0 - 1] = q;
      }
    }
    for (int64_t j = u0; j < u1; j++) {
      int32_t q = free_pages[--top];
      ref[q] = 1;
      row[j] = q;
    }
    for (int t = 0; t < A; t++) {
      int64_t pos = (int64_t)len[r] + t;
      slots[(int64_t)r * A + t] = row[pos / S] * S + (int32_t)(pos % S);
    }
    len[r] += A;
  }
  *free_count = top;
  *n_cow = nc;
  return 0;
}

/* ancestors: local indices per prompt (P prompts of N).  table_old / len_in:
 * the rows before resampling; table_new: the gathered rows.  Returns 0, or 3
 * (an ancestor outside 0..N-1, a length outside 0..L*S or a page id outside
 * the pool), changing nothing. */
int oracle_pages_resample(int P, int N, int L, int S, int64_t M, const int32_t* ancestors,
                          const int32_t* table_old, const int32_t* table_new,
                          const int32_t* len_in, int32_t* len_out, int32_t* ref,
                          int32_t* free_pages, int32_t* free_count) {
  int64_t R = (int64_t)P * N;
  for (int64_t k = 0; k < R; k++) {
    if (ancestors[k] < 0 || ancestors[k] >= N) return 3;
    if (len_in[k] < 0 || used_pages(len_in[k], S) > L) return 3;
  }
  for (int64_t k = 0; k < R; k++) {
    int32_t ln = len_in[(k / N) * N + ancestors[k]];
    for (int64_t j = 0; j < used_pages(ln, S); j++)
      if (table_new[k * L + j] < 0 || table_new[k * L + j] >= M) return 3;
    for (int64_t j = 0; j < used_pages(len_in[k], S); j++)
      if (table_old[k * L + j] < 0 || table_old[k * L + j] >= M) return 3;
  }
  for (int64_t k = 0; k < R; k++) len_out[k] = len_in[(k / N) * N + ancestors[k]];
  for (int64_t k = 0; k < R; k++) {
    for (int64_t j = 0; j < used_pages(len_out[k], S); j++) ref[table_new[k * L + j]]++;
    for (int64_t j = 0; j < used_pages(len_in[k], S); j++) ref[table_old[k * L + j]]--;
  }
  unsigned char* pushed = (unsigned char*)calloc((size_t)(M > 0 ? M : 1), 1);
  int32_t top = *free_count;
  for (int64_t k = 0; k < R; k++) {
    for (int64_t j = 0; j < used_pages(len_in[k], S); j++) {
      int32_t pg = table_old[k * L + j];
      if (ref[pg] == 0 && !pushed[pg]) {
        pushed[pg] = 1;
        free_pages[top++] = pg;
      }
    }
  }
  free(pushed);
  *free_count = top;
  return 0;
}

/* ---------------------------------------------------------------------------
 * Draft side: the steps just before verification.
 *   [SMC] sec. 2 step 1: the draft model extends every particle (or sequence)
 *         by one token per draft position, a draw from the draft
 *         distribution q.
 *   [PACER] Methodik 1-3: drafting goes in blocks of b tokens; after each
 *         block a pre-verifier estimates the acceptance of its tokens, and the
 *         drafting stops when the block's mean estimate falls below a
 *         threshold t; otherwise t grows by a factor rho and another block is
 *         drafted.
 * ------------------------------------------------------------------------- */

/*
 * One token per row r of logits [R, V], drawn from softmax(z_r / T) by inverse
 * CDF with uniforms[r] (the conventions at the top of this file).  margin[r]
 * (optional): the draw's distance to the nearer edge of its CDF interval.
 * Returns the status bits (NONFINITE, CDF_CLAMP) of all rows.
 */
int oracle_draft_sample(int dtype, int64_t R, int64_t V, double T, const void* logits,
                        const float* uniforms, int32_t* tokens, double* margin) {
  double* w = (double*)malloc(sizeof(double) * (size_t)(V > 0 ? V : 1));
  uint32_t flags = 0;
  for (int64_t r = 0; r < R; r++) {
    final_weights(dtype, row_ptr(dtype, logits, r, V), NULL, V, T, w, &flags);
    tokens[r] = (int32_t)inverse_cdf(w, V, (double)uniforms[r], margin ? &margin[r] : NULL, &flags);
  }
  free(w);
  return (int)flags;
}

/*
 * PACER draft lengths of B sequences.  scores [B, max_blocks * block]: the
 * pre-verifier's estimated acceptance of each drafted token, block after
 * block.  Per sequence the threshold starts at t0; after block m (m = 1, 2,
 * ...) the block's mean score -- its scores summed in index order in double,
 * divided by block -- is compared with t: if it is below t (strictly), or m ==
 * max_blocks, the sequence stops with K_b = block * m tokens; otherwise
 * t = t * rho.  Scores after a sequence's stopping block are not read.
 * offsets[B + 1]: offsets[0] = 0, offsets[b + 1] = offsets[b] + K_b (the
 * packed draft rows of a ragged verify).
 */
void oracle_pacer_lengths(int B, int block, int max_blocks, double t0, double rho,
                          const float* scores, int32_t* lengths, int32_t* offsets) {
  offsets[0] = 0;
  for (int b = 0; b < B; b++) {
    const float* s = scores + (int64_t)b * max_blocks * block;
    double t = t0;
    int m = 1;
    for (;; m++) {
      double sum = 0.0;
      for (int k = 0; k < block; k++) sum += (double)s[(int64_t)(m - 1) * block + k];
      double mean = sum / block;
      if (mean < t || m == max_blocks) break;
      t = t * rho;
    }
    lengths[b] = block * m;
    offsets[b + 1] = offsets[b] + lengths[b];
  }
}

/* ---------------------------------------------------------------------------
 * Tree verification.  [SMC] sec. 4 (Ergebnisse) compares SMC-SD with
 * tree-based speculative decoding but gives no algorithm for verifying a
 * token tree.  Reading (multi-draft speculative sampling, the textbook way to
 * verify several draft continuations against one target distribution):
 *   - tree b has M_b = node_off[b+1] - node_off[b] nodes; node 0 is the root
 *     (the last committed token), every other node n has a parent
 *     parent[n] < n (local index) and a draft token x_n proposed as a child of
 *     its parent; children of a node are tried in increasing node index;
 *   - target row of node n: global row node_off[b] + n (the target's logits
 *     for the token after the path root..n); draft row of node n, for nodes
 *     with at least one child: draft_off[b] + (number of such nodes of tree b
 *     with a smaller index) (the draft logits the children were drawn from);
 *   - at node u the running distribution r starts as p_u; child c (token x)
 *     is accepted iff u_c < r(x) / q_u(x) (strict), and the walk moves to c;
 *     after a rejection, r becomes max(0, r - q_u) / Z with Z its total mass
 *     (if Z is 0, r stays, flag ZERO_RESIDUAL);
 *   - the walk stops at a leaf (final token from p_leaf) or at a node all of
 *     whose children were rejected (final token from the last residual
 *     max(0, r - q_u), drawn from the unnormalised weights as in plain SD);
 *   - uniforms[node_off[b] + n], n >= 1: acceptance uniform of node n;
 *     uniforms[node_off[b]] (the root's slot): the final draw's uniform.
 * A chain (every node has one child) is plain SD with K_b = M_b - 1.
 * ------------------------------------------------------------------------ */

/* Draft row of each node of tree b (-1 for leaves); returns the number of
 * nodes with children, or -1 when the parents are not a tree in this order. */
static int64_t tree_draft_rows(const int32_t* par, int M, int64_t d0, int64_t* drow) {
  for (int n = 0; n < M; n++) drow[n] = -1;
  for (int n = 1; n < M; n++) {
    if (par[n] < 0 || par[n] >= n) return -1;
    drow[par[n]] = 0;
  }
  if (M > 0 && par[0] != -1) return -1;
  int64_t k = 0;
  for (int n = 0; n < M; n++)
    if (drow[n] == 0) drow[n] = d0 + k++;
  return k;
}

/*
 * One rejection: w = max(0, r - q) elementwise, Z = its total (index order),
 * r <- w / Z.  When Z is 0 (r and q agree), r stays, w = r and ZERO_RESIDUAL
 * is raised.
 */
static void residual_step(double* r, const double* q, double* w, int64_t V, uint32_t* fl) {
  double Z = 0.0;
  for (int64_t i = 0; i < V; i++) {
    w[i] = r[i] - q[i] > 0.0 ? r[i] - q[i] : 0.0;
    Z += w[i];
  }
  if (Z > 0.0) {
    for (int64_t i = 0; i < V; i++) r[i] = w[i] / Z;
  } else {
    *fl |= ORACLE_FLAG_ZERO_RESIDUAL;
    for (int64_t i = 0; i < V; i++) w[i] = r[i];
  }
}

/*
 * The residual chain at node u: r starts as p_u (and q as q_u when u has a
 * draft row); then the first nrej children of u in order (nrej < 0: all of
 * them) are rejected, each turning r into max(0, r - q_u) / Z.  Leaves w = the
 * weights of the final draw if the walk stops at u after those rejections
 * (p_u before any; then the last rejection's max(0, r - q_u), or r when its
 * mass is 0) and r = the running distribution.
 */
static void tree_residual(int dtype, int64_t V, double T, const void* trow, const void* drow,
                          const int32_t* par, int M, int u, int nrej, double* r, double* q, double* w,
                          uint32_t* fl) {
  double Mt, lSt;
  if (oracle_row_stats(dtype, trow, V, T, &Mt, &lSt)) *fl |= ORACLE_FLAG_NONFINITE;
  for (int64_t i = 0; i < V; i++) r[i] = exp(logprob_with(dtype, trow, i, T, Mt, lSt));
  for (int64_t i = 0; i < V; i++) w[i] = r[i];
  if (!drow) return;
  double Md, lSd;
  if (oracle_row_stats(dtype, drow, V, T, &Md, &lSd)) *fl |= ORACLE_FLAG_NONFINITE;
  for (int64_t i = 0; i < V; i++) q[i] = exp(logprob_with(dtype, drow, i, T, Md, lSd));
  int done = 0;
  for (int c = u + 1; c < M && (nrej < 0 || done < nrej); c++) {
    if (par[c] != u) continue;
    residual_step(r, q, w, V, fl);
    done++;
  }
}

/*
 * Verify B token trees.  Outputs per tree: num_accepted (depth of the node
 * where the walk stopped), last_node (its local index) and final_token.
 * accept_margin[node_off[b] + n] (optional): |u_n - min(1, ratio)| for every
 * child n that was tested, -1 for the others (and the root);
 * sample_margin[b] (optional): margin of the final draw.
 * Returns 0, or -1 (nothing written for that tree) when a tree's parents are
 * not in tree order or its number of nodes with children differs from
 * draft_off[b+1] - draft_off[b].
 */
int oracle_tree_verify(int dtype, int B, int64_t V, double T, const int32_t* node_off,
                       const int32_t* draft_off, const int32_t* parent, const int32_t* tokens,
                       const void* target, const void* draft, const float* uniforms,
                       int32_t* num_accepted, int32_t* last_node, int32_t* final_token, uint32_t* flags,
                       double* accept_margin, double* sample_margin) {
  size_t nv = (size_t)(V > 0 ? V : 1);
  double* r = (double*)malloc(sizeof(double) * nv);
  double* q = (double*)malloc(sizeof(double) * nv);
  double* w = (double*)malloc(sizeof(double) * nv);
  uint32_t fl = 0;
  int ret = 0;
  for (int b = 0; b < B; b++) {
    int64_t n0 = node_off[b];
    int M = node_off[b + 1] - node_off[b];
    const int32_t* par = parent + n0;
    int64_t* drow = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    if (M < 1 || tree_draft_rows(par, M, draft_off[b], drow) != draft_off[b + 1] - draft_off[b]) {
      free(drow);
      ret = -1;
      continue;
    }
    if (accept_margin)
      for (int n = 0; n < M; n++) accept_margin[n0 + n] = -1.0;
    int u = 0, depth = 0;
    for (;;) {
      const void* trow = row_ptr(dtype, target, n0 + u, V);
      const void* dr = drow[u] >= 0 ? row_ptr(dtype, draft, drow[u], V) : NULL;
      /* start of the residual chain at u: r = p_u, q = q_u */
      tree_residual(dtype, V, T, trow, dr, par, M, u, 0, r, q, w, &fl);
      if (!dr) break; /* a leaf: the final token comes from p_u (w) */
      int next = -1;
      for (int c = u + 1; c < M; c++) {
        if (par[c] != u) continue;
        int32_t x = tokens[n0 + c];
        /* a token outside the vocabulary is rejected */
        double ratio = x >= 0 && x < V ? r[x] / q[x] : 0.0;
        double uc = (double)uniforms[n0 + c];
        if (accept_margin) accept_margin[n0 + c] = fabs(uc - (ratio < 1.0 ? ratio : 1.0));
        if (uc < ratio) {
          next = c;
          break;
        }
        residual_step(r, q, w, V, &fl);
      }
      if (next < 0) break; /* every child rejected: final token from w */
      u = next;
      depth++;
    }
    num_accepted[b] = depth;
    last_node[b] = u;
    double m = 0.0;
    final_token[b] = (int32_t)inverse_cdf(w, V, (double)uniforms[n0], &m, &fl);
    if (sample_margin) sample_margin[b] = m;
    free(drow);
  }
  free(r);
  free(q);
  free(w);
  if (flags) *flags |= fl;
  return ret;
}

/*
 * Normalised CDF of the distribution tree b's final token is drawn from when
 * the walk stops at node u (every child of u rejected, or u a leaf).  Used by
 * the comparison to judge a differing token against the decision band.
 * Returns the flags raised, or -1 for a malformed tree.
 */
int oracle_tree_final_cdf(int dtype, int b, int64_t V, double T, const int32_t* node_off,
                          const int32_t* draft_off, const int32_t* parent, const void* target,
                          const void* draft, int u, double* cdf) {
  int64_t n0 = node_off[b];
  int M = node_off[b + 1] - node_off[b];
  const int32_t* par = parent + n0;
  if (M < 1 || u < 0 || u >= M) return -1;
  int64_t* drow = (int64_t*)malloc(sizeof(int64_t) * (size_t)M);
  if (tree_draft_rows(par, M, draft_off[b], drow) != draft_off[b + 1] - draft_off[b]) {
    free(drow);
    return -1;
  }
  size_t nv = (size_t)(V > 0 ? V : 1);
  double* r = (double*)malloc(sizeof(double) * nv);
  double* q = (double*)malloc(sizeof(double) * nv);
  uint32_t fl = 0;
  const void* dr = drow[u] >= 0 ? row_ptr(dtype, draft, drow[u], V) : NULL;
  tree_residual(dtype, V, T, row_ptr(dtype, target, n0 + u, V), dr, par, M, u, -1, r, q, cdf, &fl);
  double Z = 0.0;
  for (int64_t i = 0; i < V; i++) Z += cdf[i];
  double C = 0.0;
  for (int64_t i = 0; i < V; i++) {
    C += cdf[i];
    cdf[i] = C / Z;
  }
  free(drow);
  free(r);
  free(q);
  return (int)fl;
}
