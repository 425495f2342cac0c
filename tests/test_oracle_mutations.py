"""Plant one mistake at a time in a copy of the oracle (on the CPU) and check
that the pins catch it.  Each mutation is a plausible slip: a sign, a pairing,
a dropped term or scale, an off-by-one in the block rule, a reversed tie
break, a wrong head mapping, a swapped operand."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qsa_oracle.c")

MUTATIONS = {
    "rope_sign": ("yr[j] = f64_to_bf16(a[j] * c - b[j] * s);",
                  "yr[j] = f64_to_bf16(a[j] * c + b[j] * s);"),
    "rope_pairing": ("b[j] = bf16_to_f64(xr[j + half]);", "b[j] = bf16_to_f64(xr[j + 1]);"),
    "rope_frequency": ("pow(theta, -2.0 * (double)j / (double)rope_dim)",
                       "pow(theta, -1.0 * (double)j / (double)rope_dim)"),
    "compress_drops_token": ("for (int t = 0; t < r; ++t) s += bf16_to_f64",
                             "for (int t = 1; t < r; ++t) s += bf16_to_f64"),
    "compress_rms_eps": ("sqrt(ss / (double)Di + 1e-6)", "sqrt(ss + 1e-6)"),
    "score_scale_dropped": ("s[b] = mode == 0 ? acc * scale : acc;", "s[b] = acc;"),
    "score_relu_dropped": ("acc += dot > 0.0 ? dot : 0.0;", "acc += dot;"),
    "complete_block_off_by_one": ("return p < 0 ? 0 : (p + 1) / r;",
                                  "return p < 0 ? 0 : p / r;"),
    "tie_break_reversed": ("return a->b < c->b ? -1 : (a->b > c->b ? 1 : 0);",
                           "return a->b > c->b ? -1 : (a->b < c->b ? 1 : 0);"),
    "partial_block_dropped": ("for (int64_t j = nc * r; j <= p; ++j) tok[n++] = j;",
                              "for (int64_t j = nc * r; j < p; ++j) tok[n++] = j;"),
    "gqa_mapping": ("int g = h / group;", "int g = h % Hkv;"),
    "softmax_scale": ("double scale = 1.0 / sqrt((double)D);", "double scale = 1.0 / (double)D;"),
    "value_operand_swapped": ("const uint16_t *vr = V + ", "const uint16_t *vr = K + "),
    "lse_drops_max": ("lse[h] = m + log(sw);", "lse[h] = log(sw);"),
    "kbar_rope_sign": ("m2[j] = a * c - bb * s;", "m2[j] = a * c + bb * s;"),
    "kbar_rope_block_index": ("double p = (double)r * (double)(block0 + b);",
                              "double p = (double)(block0 + b);"),
    "kbar_gain_dropped": ("m[d] *= inv * g;", "m[d] *= inv;"),
    "kbar_rope_frequency": ("pow(theta, -(double)(2 * j) / (double)rope_dim)",
                            "pow(theta, -(double)j / (double)rope_dim)"),
    "distill_gqa_mapping": ("const int g = h / (H / Hkv);", "const int g = h % Hkv;"),
    "distill_softmax_scale": ("const double inv_sqrt_d = 1.0 / sqrt((double)D);",
                              "const double inv_sqrt_d = 1.0 / (double)D;"),
    "distill_mean_pool": ("if (a > mb) mb = a;", "mb += a / (double)r;"),
    "distill_kl_reversed": ("if (t > 0.0) kl += t * (log(t) - ls);",
                            "if (t > 0.0) kl += exp(ls) * (ls - log(t));"),
    "distill_partial_block_dropped": ("for (int64_t j = 0; j <= p; ++j) z += exp(l[j] - m);",
                                      "for (int64_t j = 0; j < nc * r; ++j) z += exp(l[j] - m);"),
    "distill_scores_not_softmaxed": ("double lse_s = ms + log(zs);", "double lse_s = 0.0;"),
    "sparse_kl_tail_out_of_softmax": ("for (int64_t j = 0; j < ntok; ++j) zh += exp(lg[j] - mh);",
                                      "for (int64_t j = 0; j < (int64_t)nsel * r; ++j) zh += exp(lg[j] - mh);"),
    "sparse_kl_mean_pool": ("mb = a > mb ? a : mb;", "mb += a / (double)r;"),
    "sparse_kl_last_head_only": ("Tb[i] += mb;", "Tb[i] = mb;"),
    "sparse_kl_gqa_mapping": ("const int kvh = h / (H / Hkv);", "const int kvh = h % Hkv;"),
    "sparse_kl_reversed": ("if (ti > 0.0) acc += ti * (log(ti) - lsi);",
                           "if (ti > 0.0) acc += exp(lsi) * (lsi - log(ti));"),
    "sparse_kl_score_by_rank": ("for (int k = 0; k < ns; ++k) s_sel[k] = s[bi[k]];",
                                "for (int k = 0; k < ns; ++k) s_sel[k] = s[k];"),
    "sparse_kl_student_not_normalised": ("const double s_lse = smax + log(ssum);",
                                         "const double s_lse = smax;"),
    "reuse_tail_from_own_block": ("int64_t from = qsa_oracle_num_complete(p_sel, r) * r;",
                                  "int64_t from = qsa_oracle_num_complete(p, r) * r;"),
    "reuse_tail_stops_short": ("for (int64_t j = from; j <= p; ++j) tok[n++] = j;",
                               "for (int64_t j = from; j < p; ++j) tok[n++] = j;"),
    # row drivers: a position or a row taken from the loop index instead of
    # the row's own index
    "sparse_attn_rows_position_by_index": ("int64_t p = pos0 + t;\n        int ns = nsel[i];",
                                           "int64_t p = pos0 + i;\n        int ns = nsel[i];"),
    "sparse_attn_rows_query_by_index": (
        "qsa_oracle_attend_row(Q + t * H * (int64_t)D, K, V, H, Hkv, D, tok, ntok,\n"
        "                              O + i * H * (int64_t)D, lse + i * H, &e);",
        "qsa_oracle_attend_row(Q + i * H * (int64_t)D, K, V, H, Hkv, D, tok, ntok,\n"
        "                              O + i * H * (int64_t)D, lse + i * H, &e);"),
    "qsa_rows_at_query_row_zero": (
        "qsa_oracle_attend_row(Q + i * H * (int64_t)D, K, V, H, Hkv, D, tok, ntok,\n"
        "                              O + i * H * (int64_t)D, lse + i * H, &wsum_err[i]);",
        "qsa_oracle_attend_row(Q, K, V, H, Hkv, D, tok, ntok,\n"
        "                              O + i * H * (int64_t)D, lse + i * H, &wsum_err[i]);"),
    "qsa_rows_at_indexer_row_zero": ("qsa_oracle_scores_row(qi + i * Hi * (int64_t)Di, kbar, nb, p,",
                                     "qsa_oracle_scores_row(qi, kbar, nb, p,"),
    "qsa_rows_at_position_of_row_zero": ("int64_t p = pos[i];", "int64_t p = pos[0];"),
    "qsa_rows_position_by_index": (
        "int64_t p = pos0 + t;\n        int64_t nc_full = qsa_oracle_num_complete(p, r);\n"
        "        double *s = (double *)malloc(sizeof(double) * (size_t)(nc_full > 0 ? nc_full : 1));\n"
        "        int64_t nc = qsa_oracle_scores_row(qi + t * Hi * (int64_t)Di, kbar, nb, p, Hi, Di, r,\n"
        "                                           mode, s);\n        int32_t *blk",
        "int64_t p = pos0 + i;\n        int64_t nc_full = qsa_oracle_num_complete(p, r);\n"
        "        double *s = (double *)malloc(sizeof(double) * (size_t)(nc_full > 0 ? nc_full : 1));\n"
        "        int64_t nc = qsa_oracle_scores_row(qi + t * Hi * (int64_t)Di, kbar, nb, p, Hi, Di, r,\n"
        "                                           mode, s);\n        int32_t *blk"),
    "select_rows_position_by_index": (
        "int64_t p = pos0 + t;\n        int64_t nc_full = qsa_oracle_num_complete(p, r);\n"
        "        double *s = (double *)malloc(sizeof(double) * (size_t)(nc_full > 0 ? nc_full : 1));\n"
        "        int64_t nc = qsa_oracle_scores_row(qi + t * Hi * (int64_t)Di, kbar, nb, p, Hi, Di, r,\n"
        "                                           mode, s);\n        if (s_out)",
        "int64_t p = pos0 + i;\n        int64_t nc_full = qsa_oracle_num_complete(p, r);\n"
        "        double *s = (double *)malloc(sizeof(double) * (size_t)(nc_full > 0 ? nc_full : 1));\n"
        "        int64_t nc = qsa_oracle_scores_row(qi + t * Hi * (int64_t)Di, kbar, nb, p, Hi, Di, r,\n"
        "                                           mode, s);\n        if (s_out)"),
    "dense_rows_position_by_index": (
        "int64_t p = pos0 + t;\n        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(p + 1));",
        "int64_t p = pos0 + i;\n        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(p + 1));"),
    "sparse_attn_rows_at_position_of_row_zero": ("const int64_t p_i = pos[i];",
                                                 "const int64_t p_i = pos[0];"),
    "sparse_attn_rows_at_query_row_zero": (
        "qsa_oracle_attend_row(Q + i * H * (int64_t)D, K, V, H, Hkv, D, tok, ntok,\n"
        "                              O + i * H * (int64_t)D, lse + i * H, &e);",
        "qsa_oracle_attend_row(Q, K, V, H, Hkv, D, tok, ntok,\n"
        "                              O + i * H * (int64_t)D, lse + i * H, &e);"),
    "sparse_attn_rows_at_selection_row_zero": (
        "qsa_oracle_token_set(sel + i * Kbudget, ns_i, p_i, r, tok);",
        "qsa_oracle_token_set(sel, ns_i, p_i, r, tok);"),
    # bf16 narrowing below the normal range
    "bf16_subnormal_quantum": ("if (e < -125) e = -125;", "if (e < -126) e = -126;"),
    "bf16_subnormal_unclamped": ("if (e < -125) e = -125;", "if (e < -1075) e = -1075;"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, mutant_dir):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    c_path = os.path.join(mutant_dir, f"{name}.c")
    so_path = os.path.join(mutant_dir, f"{name}.so")
    with open(c_path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-o",
                           so_path, c_path, "-lm"])
    env = dict(os.environ, QSA_ORACLE_LIB=so_path, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"
