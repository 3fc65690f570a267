"""Planted mistakes: each test compiles a copy of the oracle with one plausible
error (a dropped term, a wrong index or divisor, a flipped tie rule, a missing
mask) and checks that at least one of the oracle's pins now fails.  This shows
the pins constrain the oracle; the mistakes live only in temporary copies,
on the CPU.
"""
import contextlib
import os
import shutil
import subprocess

import pytest

import oracle

import test_oracle_attention as T_att
import test_oracle_gate_select as T_gs
import test_oracle_ground_truth as T_gt
import test_oracle_policy as T_pol
import test_oracle_per_head as T_ph
import test_oracle_pipeline as T_pipe


@contextlib.contextmanager
def mutated_oracle(tmp_path, old: str, new: str, count: int = 1):
    src = open(oracle._SRC).read()
    assert src.count(old) == count, f"mutation anchor occurs {src.count(old)} times: {old!r}"
    (tmp_path / "seer_oracle.c").write_text(src.replace(old, new))
    shutil.copy(os.path.join(oracle._HERE, "seer_oracle.h"), tmp_path / "seer_oracle.h")
    lib_path = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", lib_path,
                    str(tmp_path / "seer_oracle.c"), "-lm"], check=True, capture_output=True)
    saved = oracle._load()
    oracle._lib = oracle._bind(lib_path)
    try:
        yield
    finally:
        oracle._lib = saved


def fails(*checks) -> bool:
    """True if at least one pin check raises (assertion or numeric mismatch)."""
    for fn in checks:
        try:
            fn()
        except (AssertionError, ValueError):
            return True
    return False


MUTATIONS = [
    ("tail not attended", "        in_t[t] = 1;\n\n    /* D6", "        (void)t;\n\n    /* D6",
     lambda: T_att.test_all_blocks_selected_equals_dense_attention(4, 64, 300, 64)),
    ("softmax scale dropped", "z[t] = scale * dot;", "z[t] = dot;",
     lambda: T_att.test_all_blocks_selected_equals_dense_attention(4, 64, 300, 64)),
    ("tie toward the higher index", "(S[ids[b]] > S[ids[a]])", "(S[ids[b]] >= S[ids[a]])",
     T_gs.test_selection_ties_go_to_lower_index_and_output_ascends),
    ("transposed query projection", "wq[(int64_t)r * d + e]", "wq[(int64_t)e * dg + r]",
     T_gs.test_gate_single_entry_projections_closed_form),
    ("pooling divisor off by one", "kpool[(int64_t)j * d + c] = sum / bs;",
     "kpool[(int64_t)j * d + c] = sum / (bs - 1);", T_gs.test_pool_constant_block_is_that_row),
    ("group sum instead of mean", "S[j] = mean / G;", "S[j] = mean;",
     T_gs.test_gate_identity_projections_score_group_mean_query),
    ("pooled block offset wrong", "for (int t = j * bs; t < (j + 1) * bs; ++t)\n                sum +=",
     "for (int t = j * bs + 1; t < (j + 1) * bs + 1; ++t)\n                sum +=",
     T_gs.test_pool_ramp_closed_form),
    ("keep count floors", "* keep_num + keep_den - 1) / keep_den;", "* keep_num) / keep_den + 1;",
     T_pipe.test_prefill_keep_counts_golden),
    ("block mass summed instead of averaged over heads", "mass[j] = sum / G;", "mass[j] = sum;",
     lambda: T_gt.test_block_mass_normalised_and_nonnegative(300, 64)),
    ("tail share dropped from the ground truth", "const int t0 = j * bs, t1 = j < nc ? (j + 1) * bs : L;",
     "const int t0 = j * bs, t1 = j < nc ? (j + 1) * bs : j * bs;",
     lambda: T_gt.test_equal_keys_give_token_count_shares(300, 64)),
    ("ratio count rounds down", "k = (int)(((int64_t)nc * num + den - 1) / den);",
     "k = (int)(((int64_t)nc * num) / den);", lambda: T_pol.test_ratio_counts_closed_form(512, 1, 10, 52)),
    ("threshold compared on the unnormalised weight", "if (exp(S[j] - m) / z >= tau)",
     "if (exp(S[j] - m) >= tau)", lambda: T_pol.test_threshold_keeps_the_blocks_above_tau(64, 0.02)),
    ("per-head variant selects from the group mean", "int n = so_select_blocks(sh + (int64_t)h * nc, nc, kmax, sel);",
     "int n = so_select_blocks(S, nc, kmax, sel);", T_ph.test_heads_differ_and_each_head_is_its_own_masked_attention),
    ("prefill ground truth averaged over the block size, not its rows",
     "row[tt / bs] += exp(z[tt] - m) / denom / (t1 - t0);", "row[tt / bs] += exp(z[tt] - m) / denom / bs;",
     lambda: T_gt.test_prefill_mass_equals_torch_causal_softmax(300, 64)),
    ("prefill causal mask dropped", "for (int tt = 0; tt <= t; ++tt)", "for (int tt = 0; tt < L; ++tt)",
     lambda: T_pipe.test_prefill_keep_all_is_causal_attention(512, 64)),
    ("query group of KV head g taken at g, not g * G", "const uint16_t *qg = q + b * sq_b + (int64_t)g * G * sq_h;",
     "const uint16_t *qg = q + b * sq_b + (int64_t)g * sq_h;", T_pipe.test_budget_covering_context_is_dense_gqa_attention),
    ("gate scale dropped", "            s *= gate_scale;\n", "            (void)gate_scale;\n",
     lambda: T_gs.test_gate_matches_reassociated_form(4, 64, 32)),
    ("lse in log2 units", "        lse[h] = m + log(denom);", "        lse[h] = m + log2(denom);",
     lambda: T_att.test_all_blocks_selected_equals_dense_attention(4, 64, 300, 64)),
    ("kept ids left in score order", "    qsort(idx, (size_t)n, sizeof(int32_t), by_index);",
     "    (void)by_index;", T_gs.test_selection_ties_go_to_lower_index_and_output_ascends),
    ("prefill row keeps the previous block instead of its diagonal", "        dst[n] = i;",
     "        dst[n] = i > 0 ? i - 1 : i;", lambda: T_pipe.test_prefill_rows_keep_diagonal_and_k_i_blocks((1, 10))),
    ("pooled cache of every KV head taken from head 0", "so_pool_k(k + b * sk_b + g * sk_h, sk_t,",
     "so_pool_k(k + b * sk_b, sk_t,", T_pipe.test_batched_step_composes_stage_functions),
    ("decode output of KV head g written at row g, not g * G",
     "out + ((int64_t)b * Hq + (int64_t)g * G) * d,", "out + ((int64_t)b * Hq + (int64_t)g) * d,",
     T_pipe.test_budget_covering_context_is_dense_gqa_attention),
    ("prefill partial block pooled over bs rows", "        dst[c] = sum / (t1 - t0);", "        dst[c] = sum / bs;",
     T_pipe.test_prefill_partial_last_block_pools_existing_rows),
    ("prefill gate pools Q for the key side", "        pool_block_rows(k, row_stride, L, d, bs, i, kbar);",
     "        pool_block_rows(q, row_stride, L, d, bs, i, kbar);", T_pipe.test_prefill_partial_last_block_pools_existing_rows),
    ("prefill gate projections transposed",
     "sa += so_bf16_to_f64(wq[(int64_t)r * d + e]) * qbar[e];\n                sc += so_bf16_to_f64(wk[(int64_t)r * d + e]) * kbar[e];",
     "sa += so_bf16_to_f64(wq[(int64_t)e * dg + r]) * qbar[e];\n                sc += so_bf16_to_f64(wk[(int64_t)e * dg + r]) * kbar[e];",
     T_pipe.test_prefill_gate_single_entry_projections_closed_form),
    ("prefill gate Wq and Wk swapped",
     "sa += so_bf16_to_f64(wq[(int64_t)r * d + e]) * qbar[e];\n                sc += so_bf16_to_f64(wk[(int64_t)r * d + e]) * kbar[e];",
     "sa += so_bf16_to_f64(wk[(int64_t)r * d + e]) * qbar[e];\n                sc += so_bf16_to_f64(wq[(int64_t)r * d + e]) * kbar[e];",
     T_pipe.test_prefill_gate_single_entry_projections_closed_form),
    ("prefill gate key projection uses the query's pooled vector",
     "sc += so_bf16_to_f64(wk[(int64_t)r * d + e]) * kbar[e];",
     "sc += so_bf16_to_f64(wk[(int64_t)r * d + e]) * qbar[e];",
     T_pipe.test_prefill_gate_single_entry_projections_closed_form),
    ("a kept block's last token left out", "for (int t = idx[i] * bs; t < (idx[i] + 1) * bs; ++t)",
     "for (int t = idx[i] * bs; t < (idx[i] + 1) * bs - 1; ++t)", lambda: T_att.test_sparse_equals_masked_dense(0)),
    ("decode output weighs the keys instead of the values",
     "oh[c] += wt * so_bf16_to_f64(v[(int64_t)t * kv_row_stride + c]);",
     "oh[c] += wt * so_bf16_to_f64(k[(int64_t)t * kv_row_stride + c]);",
     lambda: T_att.test_sparse_equals_masked_dense(0)),
    ("prefill softmax scale dropped",
     "            z[tt] = scale * dot;\n            if (z[tt] > m)\n                m = z[tt];\n        }\n        double *ot",
     "            z[tt] = dot;\n            if (z[tt] > m)\n                m = z[tt];\n        }\n        double *ot",
     lambda: T_pipe.test_prefill_keep_all_is_causal_attention(512, 64)),
    ("prefill output weighs the keys instead of the values",
     "ot[c] += wt * so_bf16_to_f64(v[(int64_t)tt * row_stride + c]);",
     "ot[c] += wt * so_bf16_to_f64(k[(int64_t)tt * row_stride + c]);",
     lambda: T_pipe.test_prefill_keep_all_is_causal_attention(512, 64)),
    ("prefill lse in log2 units", "lse[t - t_lo] = m + log(denom);", "lse[t - t_lo] = m + log2(denom);",
     T_pipe.test_prefill_attention_equals_masked_dense),
    ("prefill block mass not divided by the row's softmax sum",
     "row[tt / bs] += exp(z[tt] - m) / denom / (t1 - t0);", "row[tt / bs] += exp(z[tt] - m) / (t1 - t0);",
     lambda: T_gt.test_prefill_mass_equals_torch_causal_softmax(256, 64)),
]


@pytest.mark.parametrize("name,old,new,check", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, check):
    count = open(oracle._SRC).read().count(old)
    with mutated_oracle(tmp_path, old, new, count=count):
        assert fails(check), f"no pin caught: {name}"
    # and the unmodified oracle passes the same check
    check()
