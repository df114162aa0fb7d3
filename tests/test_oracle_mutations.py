"""The pins have power: each plausible mistake planted in a copy of the oracle
(a dropped term, a wrong sign or index, a transposed operand, a flipped
comparison) must make at least one pin fail.  Mutants are built on the CPU in
a temporary directory; the real oracle is never modified."""
import os
import subprocess
import sys

import pytest

import oracle

MUTATIONS = [
    ("temperature_dropped", "return oracle_logit(dtype, row, i) / T - M - logS;",
     "return oracle_logit(dtype, row, i) - M - logS;"),
    ("sum_skips_first", "for (int64_t i = 0; i < V; i++) S += exp(", "for (int64_t i = 1; i < V; i++) S += exp("),
    ("log_of_sum_dropped", "*logS_out = log(S);", "*logS_out = S;"),
    ("accept_tie_accepts", "if (!(u < rho)) {", "if (!(u <= rho)) {"),
    ("ratio_inverted", "double rho = exp(lp - lq);", "double rho = exp(lq - lp);"),
    ("residual_is_p", "w[i] = p - q > 0.0 ? p - q : 0.0;", "w[i] = p;"),
    ("residual_transposed", "w[i] = p - q > 0.0 ? p - q : 0.0;", "w[i] = q - p > 0.0 ? q - p : 0.0;"),
    ("cdf_non_strict", "if (C > target) {", "if (C >= target) {"),
    ("no_first_reject_truncation", "n = j;\n        break;", "n = j;"),
    ("final_row_off_by_one", "const void* trow = row_ptr(dtype, target, t0 + n, V);",
     "const void* trow = row_ptr(dtype, target, t0 + (n > 0 ? n - 1 : 0), V);"),
    ("final_uniform_index", "(double)uniforms[t0 + Kb]", "(double)uniforms[t0 + n]"),
    ("target_base_without_b", "int64_t t0 = d0 + b;", "int64_t t0 = d0;"),
    ("ess_formula", "E = Sw * Sw / Sw2;", "E = Sw / Sw2;"),
    ("ess_threshold_non_strict", "do_resample = E < ess_frac * N;", "do_resample = E <= ess_frac * N;"),
    ("systematic_stride", "double U = ((double)resample_u[p] + k) / N;",
     "double U = ((double)resample_u[p] + k) / (N + 1);"),
    ("systematic_non_strict", "if (C[n] > U) {", "if (C[n] >= U) {"),
    ("logw_not_reset", "logw[i] = do_resample ? 0.0f : lw[k];", "logw[i] = lw[k];"),
    ("page_table_scatter", "pt_out[i * L + l] = pt_in[src * L + l];", "pt_out[src * L + l] = pt_in[i * L + l];"),
    ("increment_sign",
     "delta += beta * logprob_with(dtype, trow, x, T, Mt, lSt) - logprob_with(dtype, drow, x, T, Md, lSd);",
     "delta += beta * logprob_with(dtype, drow, x, T, Md, lSd) - logprob_with(dtype, trow, x, T, Mt, lSt);"),
    ("power_on_draft",
     "delta += beta * logprob_with(dtype, trow, x, T, Mt, lSt) - logprob_with(dtype, drow, x, T, Md, lSd);",
     "delta += logprob_with(dtype, trow, x, T, Mt, lSt) - beta * logprob_with(dtype, drow, x, T, Md, lSd);"),
    ("power_dropped_from_weight",
     "delta += beta * logprob_with(dtype, trow, x, T, Mt, lSt) - logprob_with(dtype, drow, x, T, Md, lSd);",
     "delta += logprob_with(dtype, trow, x, T, Mt, lSt) - logprob_with(dtype, drow, x, T, Md, lSd);"),
    ("power_bonus_temperature", "V, T / beta, w, &fl);", "V, T * beta, w, &fl);"),
    ("power_bonus_plain", "V, T / beta, w, &fl);", "V, T, w, &fl);"),
    ("power_bonus_weight_dropped", "        delta += log(Sb) - beta * lSk;\n", ""),
    ("power_bonus_weight_unscaled", "delta += log(Sb) - beta * lSk;", "delta += log(Sb) - lSk;"),
    ("power_bonus_weight_sign", "delta += log(Sb) - beta * lSk;", "delta -= log(Sb) - beta * lSk;"),
    ("power_bonus_weight_plain_scale", "Sb += exp(beta * (oracle_logit(dtype, brow, y) / T - Mk));",
     "Sb += exp(oracle_logit(dtype, brow, y) / T - Mk);"),
    ("zero_residual_fallback_uniform",
     "    *flags |= ORACLE_FLAG_ZERO_RESIDUAL;\n    for (int64_t i = 0; i < V; i++) w[i] = exp(logprob_with(dtype, trow, i, T, Mt, lSt));",
     "    *flags |= ORACLE_FLAG_ZERO_RESIDUAL;\n    for (int64_t i = 0; i < V; i++) w[i] = 1.0;"),
    ("cdf_clamp_to_first", "  for (int64_t i = n - 1; i >= 0; i--)\n    if (w[i] > 0.0) return i;\n  return n - 1;",
     "  return 0;"),
    ("cdf_clamp_to_end", "  for (int64_t i = n - 1; i >= 0; i--)\n    if (w[i] > 0.0) return i;\n  return n - 1;",
     "  return n - 1;"),
    ("systematic_clamp_to_first", "          for (a = N - 1; a > 0 && pw[a] == 0.0; a--) {\n          }", "          a = 0;"),
    ("systematic_clamp_to_end", "          for (a = N - 1; a > 0 && pw[a] == 0.0; a--) {\n          }",
     "          a = N - 1;"),
    ("old_weight_dropped", "lw[n] = (float)((double)logw[i] + delta);", "lw[n] = (float)delta;"),
    ("bonus_from_first_row", "row_ptr(dtype, target, i * (K + 1) + K, V)", "row_ptr(dtype, target, i * (K + 1), V)"),
    ("weights_not_exponentiated", "pw[n] = exp((double)lw[n] - M);", "pw[n] = (double)lw[n] - M;"),
    ("pages_no_copy_on_write", "      if (ref[tail] > 1) {\n        int32_t q = free_pages[--top];",
     "      if (0) {\n        int32_t q = free_pages[--top];"),
    ("pages_copy_keeps_ref", "        ref[tail]--;\n        ref[q] = 1;", "        ref[q] = 1;"),
    ("pages_slot_offset", "slots[(int64_t)r * A + t] = row[pos / S] * S + (int32_t)(pos % S);",
     "slots[(int64_t)r * A + t] = row[pos / S] * S + (int32_t)((pos + 1) % S);"),
    ("pages_len_not_advanced", "    len[r] += A;\n  }\n  *free_count = top;", "  }\n  *free_count = top;"),
    ("pages_old_rows_not_released",
     "for (int64_t j = 0; j < used_pages(len_in[k], S); j++) ref[table_old[k * L + j]]--;", ""),
    ("pages_length_not_gathered", "len_out[k] = len_in[(k / N) * N + ancestors[k]];", "len_out[k] = len_in[k];"),
    ("pages_freed_twice", "if (ref[pg] == 0 && !pushed[pg]) {", "if (ref[pg] == 0) {"),
    ("draft_sample_uniform_index", "(double)uniforms[r]", "(double)uniforms[0]"),
    ("draft_sample_row_index", "row_ptr(dtype, logits, r, V)", "row_ptr(dtype, logits, 0, V)"),
    ("pacer_not_strict", "if (mean < t || m == max_blocks) break;", "if (mean <= t || m == max_blocks) break;"),
    ("pacer_threshold_not_grown", "t = t * rho;", "t = t * 1.0;"),
    ("pacer_mean_not_divided", "double mean = sum / block;", "double mean = sum;"),
    ("pacer_stopping_block_dropped", "lengths[b] = block * m;", "lengths[b] = block * (m - 1);"),
    ("pacer_offsets_not_accumulated", "offsets[b + 1] = offsets[b] + lengths[b];", "offsets[b + 1] = lengths[b];"),
    ("pacer_block_offset", "sum += (double)s[(int64_t)(m - 1) * block + k];", "sum += (double)s[(int64_t)m * block + k];"),
    ("tree_residual_not_renormalised", "for (int64_t i = 0; i < V; i++) r[i] = w[i] / Z;",
     "for (int64_t i = 0; i < V; i++) r[i] = w[i];"),
    ("tree_residual_is_r", "w[i] = r[i] - q[i] > 0.0 ? r[i] - q[i] : 0.0;", "w[i] = r[i];"),
    ("tree_ratio_inverted", "double ratio = x >= 0 && x < V ? r[x] / q[x] : 0.0;",
     "double ratio = x >= 0 && x < V ? q[x] / r[x] : 0.0;"),
    ("tree_accept_non_strict", "if (uc < ratio) {", "if (uc <= ratio) {"),
    ("tree_keeps_testing_after_accept", "          next = c;\n          break;", "          next = c;"),
    ("tree_final_uniform_of_node", "(double)uniforms[n0], &m, &fl);", "(double)uniforms[n0 + u], &m, &fl);"),
    ("tree_draft_row_not_advanced", "if (drow[n] == 0) drow[n] = d0 + k++;", "if (drow[n] == 0) { drow[n] = d0; k++; }"),
    ("tree_depth_not_counted", "      u = next;\n      depth++;", "      u = next;"),
    ("tree_row_of_root", "const void* trow = row_ptr(dtype, target, n0 + u, V);",
     "const void* trow = row_ptr(dtype, target, n0, V);"),
    ("accept_margin_unclamped", "fabs(u - (rho < 1.0 ? rho : 1.0))", "fabs(u - rho)"),
    ("sample_margin_on_clamp", "  if (margin) *margin = 0.0;\n", "  if (margin) *margin = 1.0;\n"),
    ("resample_margin_on_clamp", "          rmargin = 0.0;\n", "          rmargin = 1.0;\n"),
    ("nonfinite_weight_unflagged", "      if (isnan(lw[n]) || lw[n] == INFINITY) fl |= ORACLE_FLAG_NONFINITE;\n", ""),
    ("zero_weights_unflagged", "      fl |= ORACLE_FLAG_ZERO_WEIGHTS;\n", ""),
    ("pages_empty_row_refused", "if (len[r] < 0 || used_pages(len[r], S) > L) bad = 1;",
     "if (len[r] <= 0 || used_pages(len[r], S) > L) bad = 1;"),
    ("pages_page_zero_refused", "if (pg < 0 || pg >= M) bad = 1;", "if (pg <= 0 || pg >= M) bad = 1;"),
    ("pages_resample_empty_row_refused", "if (len_in[k] < 0 || used_pages(len_in[k], S) > L) return 3;",
     "if (len_in[k] <= 0 || used_pages(len_in[k], S) > L) return 3;"),
    ("tree_bad_token_accepted", "double ratio = x >= 0 && x < V ? r[x] / q[x] : 0.0;",
     "double ratio = x >= 0 && x < V ? r[x] / q[x] : 1.0;"),
    ("tree_zero_residual_uniform", "    *fl |= ORACLE_FLAG_ZERO_RESIDUAL;\n    for (int64_t i = 0; i < V; i++) w[i] = r[i];",
     "    *fl |= ORACLE_FLAG_ZERO_RESIDUAL;\n    for (int64_t i = 0; i < V; i++) w[i] = 1.0;"),
    ("tree_accept_margin_unclamped", "fabs(uc - (ratio < 1.0 ? ratio : 1.0))", "fabs(uc - ratio)"),
    ("tree_self_parent_accepted", "if (par[n] < 0 || par[n] >= n) return -1;", "if (par[n] < 0 || par[n] > n) return -1;"),
    ("tree_single_node_refused", "if (M < 1 || u < 0 || u >= M) return -1;", "if (M <= 1 || u < 0 || u >= M) return -1;"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) == 1, f"mutation site for {name} not unique in oracle.c"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(old, new))
    so = str(tmp_path / f"lib{name}.so")
    oracle.build(str(src), so, strict=False)
    # the pins run in a child process: a mutant that corrupts memory on a valid
    # input (which is also a failure the pins expose) cannot take the test
    # runner down with it
    here = os.path.dirname(os.path.abspath(__file__))
    res = subprocess.run([sys.executable, os.path.join(here, "mutant_runner.py"), so], capture_output=True,
                         text=True, timeout=600)
    assert res.returncode != 0, f"mutant {name} survived every pin\n{res.stdout[-2000:]}{res.stderr[-2000:]}"
    os.remove(so)
