/*
 * QSA layer oracle: a plain, slow CPU implementation in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the HIP library.
 *
 * What it follows (page = "On the Design of Qwen3.8 Next Architecture", the
 * papers.chlience.com reading notes, section 6 "GDN continuous compression and
 * QSA exact retrieval", unless stated otherwise):
 *   - keys are pooled over micro-blocks of r tokens (equation for k-bar_b;
 *     also the ai.info summary, "Methodology in Plain English");
 *   - the indexer scores each query against every fully formed micro-block
 *     (equation for I_ib);
 *   - at most K/r = 512 complete blocks are selected per query and the
 *     trailing, not yet complete causal block is always kept; the selected
 *     blocks expand to token indices for the core attention (same section);
 *   - head shapes: 24 query heads, 2 KV heads, head dim 256, RoPE on 64 dims;
 *     indexer 4 query heads, 1 shared key head, dim 128, ratio 4 (Model
 *     Summary table of the same page).
 * Readings where the pages are silent (each listed with its reason in the
 * design notes): NeoX rotate-half pairs (j, j+32) with angle p*theta^(-2j/64);
 * RoPE output and the pooled key rounded to bf16 (nearest even) as part of the
 * definition; MAXHEAD score max_h(q_h.kbar)/sqrt(128) as default and the
 * page's sum of ReLUs as a second mode; RMSNorm mode with unit gain and eps
 * 1e-6; ties broken by (score descending, block index ascending); query head h
 * reads KV head h / (H/Hkv); softmax scale 1/sqrt(D).
 *
 * bf16 values are passed as uint16 bit patterns.  Everything is computed in
 * double precision; bf16 inputs convert exactly.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------- bf16 helpers (exact widening, direct nearest-even narrowing) -- */

static double bf16_to_f64(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a finite double to bf16 (8 significant bits), ties to even, by
 * scaling the value to an integer significand and using rint(). */
static uint16_t f64_to_bf16(double x) {
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    frexp(x, &e);                    /* |x| = m * 2^e, m in [0.5, 1) */
    if (e < -125) e = -125;          /* bf16 subnormal range: fixed quantum */
    double q = ldexp(1.0, e - 8);    /* quantum of an 8-bit significand */
    double y = rint(x / q) * q;      /* exact scaling; rint = nearest even */
    float f = (float)y;              /* exact: y has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

uint16_t qsa_oracle_f64_to_bf16(double x) { return f64_to_bf16(x); }
double qsa_oracle_bf16_to_f64(uint16_t h) { return bf16_to_f64(h); }

/* ---------- O1: partial RoPE on attention Q/K ---------------------------- */
/* y[t][h][:] = x[t][h][:] with pairs (j, j+rope_dim/2), j < rope_dim/2,
 * rotated by the angle pos(t) * theta^(-2j/rope_dim); other dims copied.
 * pos(t) = pos ? pos[t] : pos0 + t.  Output rounded to bf16.  y may equal x. */
void qsa_oracle_rope(const uint16_t *x, uint16_t *y, int64_t T, int nheads, int head_dim,
                     int rope_dim, double theta, int64_t pos0, const int64_t *pos) {
    int half = rope_dim / 2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double p = (double)(pos ? pos[t] : pos0 + t);
        for (int h = 0; h < nheads; ++h) {
            const uint16_t *xr = x + (t * nheads + h) * (int64_t)head_dim;
            uint16_t *yr = y + (t * nheads + h) * (int64_t)head_dim;
            double *a = (double *)malloc(sizeof(double) * (size_t)(half > 0 ? 2 * half : 1));
            double *b = a + half;
            for (int j = 0; j < half; ++j) {
                a[j] = bf16_to_f64(xr[j]);
                b[j] = bf16_to_f64(xr[j + half]);
            }
            for (int j = 0; j < half; ++j) {
                double inv_freq = pow(theta, -2.0 * (double)j / (double)rope_dim);
                double ang = p * inv_freq;
                double c = cos(ang), s = sin(ang);
                yr[j] = f64_to_bf16(a[j] * c - b[j] * s);
                yr[j + half] = f64_to_bf16(b[j] * c + a[j] * s);
            }
            if (yr != xr)
                for (int d = rope_dim; d < head_dim; ++d) yr[d] = xr[d];
            free(a);
        }
    }
}

/* ---------- O2: key compression ------------------------------------------ */
/* kbar[b][:] for b < Tk/r (chlience section 6, the k-bar equation): m = the
 * mean of the r keys of block b (mode 0, average pooling), or in mode 1
 * RMSNorm(m) = m / sqrt(mean(m^2) + 1e-6), each dim times the gain gamma[d]
 * (gain NULL: unit gain).  With rope_dim > 0 the pooled key is then rotated
 * as in O1 over its first rope_dim dims, at the position of the block's first
 * token, r * (block0 + b) (the same section: pooling first, then partial
 * RoPE, so tokens at different phases are not averaged).  fp64 throughout,
 * one bf16 rounding at the end. */
void qsa_oracle_compress_ext(const uint16_t *k, int64_t Tk, int Di, int r, int mode,
                             const uint16_t *gain, int rope_dim, double theta, int64_t block0,
                             uint16_t *kbar) {
    int64_t nb = Tk / r;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        double *m = (double *)malloc(sizeof(double) * 2 * (size_t)Di);
        double *m2 = m + Di;
        for (int d = 0; d < Di; ++d) {
            double s = 0.0;
            for (int t = 0; t < r; ++t) s += bf16_to_f64(k[(b * r + t) * Di + d]);
            m[d] = s / (double)r;
        }
        if (mode == 1) {
            double ss = 0.0;
            for (int d = 0; d < Di; ++d) ss += m[d] * m[d];
            double inv = 1.0 / sqrt(ss / (double)Di + 1e-6);
            for (int d = 0; d < Di; ++d) {
                double g = gain ? bf16_to_f64(gain[d]) : 1.0;
                m[d] *= inv * g;
            }
        }
        if (rope_dim > 0) {
            int half = rope_dim / 2;
            double p = (double)r * (double)(block0 + b);
            for (int d = 0; d < Di; ++d) m2[d] = m[d];
            for (int j = 0; j < half; ++j) {
                double a = m[j], bb = m[j + half];
                double ang = p * pow(theta, -(double)(2 * j) / (double)rope_dim);
                double c = cos(ang), s = sin(ang);
                m2[j] = a * c - bb * s;
                m2[j + half] = bb * c + a * s;
            }
            for (int d = 0; d < Di; ++d) m[d] = m2[d];
        }
        for (int d = 0; d < Di; ++d) kbar[b * Di + d] = f64_to_bf16(m[d]);
        free(m);
    }
}

/* O2 without gain or rotation. */
void qsa_oracle_compress(const uint16_t *k, int64_t Tk, int Di, int r, int mode,
                         uint16_t *kbar) {
    qsa_oracle_compress_ext(k, Tk, Di, r, mode, NULL, 0, 0.0, 0, kbar);
}

/* ---------- O3: indexer scores of one query ------------------------------ */
/* Threads the OpenMP loops of this library use (1 without OpenMP). */
int qsa_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Number of complete micro-blocks visible to the query at position p. */
int64_t qsa_oracle_num_complete(int64_t p, int r) { return p < 0 ? 0 : (p + 1) / r; }

/* s[b], b < nc = min(num_complete(p), nb_avail).  mode 0: max over heads of
 * (q_h . kbar_b) / sqrt(Di); mode 1: sum over heads of max(0, q_h . kbar_b).
 * Returns nc. */
int64_t qsa_oracle_scores_row(const uint16_t *qi_row, const uint16_t *kbar, int64_t nb_avail,
                              int64_t p, int Hi, int Di, int r, int mode, double *s) {
    int64_t nc = qsa_oracle_num_complete(p, r);
    if (nc > nb_avail) nc = nb_avail;
    double *q = (double *)malloc(sizeof(double) * (size_t)Hi * (size_t)Di);
    for (int h = 0; h < Hi; ++h)
        for (int d = 0; d < Di; ++d) q[h * Di + d] = bf16_to_f64(qi_row[h * Di + d]);
    double scale = 1.0 / sqrt((double)Di);
    for (int64_t b = 0; b < nc; ++b) {
        const uint16_t *kr = kbar + b * Di;
        double acc = mode == 0 ? -INFINITY : 0.0;
        for (int h = 0; h < Hi; ++h) {
            double dot = 0.0;
            for (int d = 0; d < Di; ++d) dot += q[h * Di + d] * bf16_to_f64(kr[d]);
            if (mode == 0) {
                if (dot > acc) acc = dot;
            } else {
                acc += dot > 0.0 ? dot : 0.0;
            }
        }
        s[b] = mode == 0 ? acc * scale : acc;
    }
    free(q);
    return nc;
}

/* ---------- O4: top-K selection of one query ------------------------------ */
typedef struct { double s; int64_t b; } cand_t;

static int cand_cmp(const void *x, const void *y) {
    const cand_t *a = (const cand_t *)x, *c = (const cand_t *)y;
    if (a->s > c->s) return -1;
    if (a->s < c->s) return 1;
    return a->b < c->b ? -1 : (a->b > c->b ? 1 : 0);
}

static int i32_cmp(const void *x, const void *y) {
    int32_t a = *(const int32_t *)x, b = *(const int32_t *)y;
    return a < b ? -1 : (a > b ? 1 : 0);
}

/* Selects min(K, nc) blocks: all of them if nc <= K, else the first K in the
 * order (score descending, index ascending).  blk gets them ascending.
 * *sK, *sK1 = scores at ranks K and K+1 of that order (NAN when absent).
 * Returns the count. */
int qsa_oracle_topk_row(const double *s, int64_t nc, int K, int32_t *blk, double *sK,
                        double *sK1) {
    *sK = NAN;
    *sK1 = NAN;
    if (nc <= K) {
        for (int64_t b = 0; b < nc; ++b) blk[b] = (int32_t)b;
        if (nc > 0 && nc == K) {
            /* rank-K score still reported for the tie-band rule */
            double mn = INFINITY;
            for (int64_t b = 0; b < nc; ++b) if (s[b] < mn) mn = s[b];
            *sK = mn;
        }
        return (int)nc;
    }
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)nc);
    for (int64_t b = 0; b < nc; ++b) { c[b].s = s[b]; c[b].b = b; }
    qsort(c, (size_t)nc, sizeof(cand_t), cand_cmp);
    for (int i = 0; i < K; ++i) blk[i] = (int32_t)c[i].b;
    *sK = c[K - 1].s;
    *sK1 = c[K].s;
    free(c);
    qsort(blk, (size_t)K, sizeof(int32_t), i32_cmp);
    return K;
}

/* ---------- O5: token set ----------------------------------------------- */
/* Tokens of the selected blocks (ascending blocks -> ascending tokens),
 * followed by the query's incomplete trailing block r*nc .. p (kept always,
 * later tokens excluded).  Returns the count. */
int64_t qsa_oracle_token_set(const int32_t *blk, int nsel, int64_t p, int r, int64_t *tok) {
    int64_t n = 0;
    for (int i = 0; i < nsel; ++i)
        for (int t = 0; t < r; ++t) tok[n++] = (int64_t)blk[i] * r + t;
    int64_t nc = qsa_oracle_num_complete(p, r);
    for (int64_t j = nc * r; j <= p; ++j) tok[n++] = j;
    return n;
}

/* ---------- O5, index reuse: a later speculative query ------------------ */
/* chlience "5. 贡献全景与方法总览" item 5 (the MTP prediction steps reuse the
 * QSA top-k indices) and "Result 2" (decode with next_n = 4).  A query at
 * position p >= p_sel reuses the selection made for position p_sel: its
 * tokens are the selected blocks expanded, then every token from
 * r * nc(p_sel) through p (the incomplete block of p_sel and whatever
 * followed it).  For p = p_sel this is the token set above.  Returns the
 * number of tokens written to tok. */
int64_t qsa_oracle_token_set_reuse(const int32_t *blk, int nsel, int64_t p_sel, int64_t p, int r,
                                   int64_t *tok) {
    int64_t n = 0;
    for (int i = 0; i < nsel; ++i)
        for (int t = 0; t < r; ++t) tok[n++] = (int64_t)blk[i] * r + t;
    int64_t from = qsa_oracle_num_complete(p_sel, r) * r;
    for (int64_t j = from; j <= p; ++j) tok[n++] = j;
    return n;
}

/* ---------- O6: softmax attention of one query over a token set --------- */
/* q_row [H][D] (post-RoPE), K/V [*][Hkv][D]; for head h, KV head
 * g = h / (H/Hkv): logits l_j = q_h.k_{g,j} / sqrt(D); O_h = sum_j w_j v_{g,j}
 * / sum_j w_j with w_j = exp(l_j - max l); lse_h = max l + ln sum_j w_j.
 * *max_wsum_err = max over heads of |sum_j w_j/sum w - 1|. */
void qsa_oracle_attend_row(const uint16_t *q_row, const uint16_t *K, const uint16_t *V, int H,
                           int Hkv, int D, const int64_t *tok, int64_t ntok, double *O,
                           double *lse, double *max_wsum_err) {
    int group = H / Hkv;
    double scale = 1.0 / sqrt((double)D);
    double *l = (double *)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1));
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double err = 0.0;
    for (int h = 0; h < H; ++h) {
        int g = h / group;
        for (int d = 0; d < D; ++d) q[d] = bf16_to_f64(q_row[h * D + d]);
        double m = -INFINITY;
        for (int64_t j = 0; j < ntok; ++j) {
            const uint16_t *kr = K + (tok[j] * Hkv + g) * (int64_t)D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += q[d] * bf16_to_f64(kr[d]);
            l[j] = dot * scale;
            if (l[j] > m) m = l[j];
        }
        double sw = 0.0;
        for (int64_t j = 0; j < ntok; ++j) { l[j] = exp(l[j] - m); sw += l[j]; }
        double *o = O + (int64_t)h * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        double check = 0.0;
        for (int64_t j = 0; j < ntok; ++j) {
            double w = l[j] / sw;
            check += w;
            const uint16_t *vr = V + (tok[j] * Hkv + g) * (int64_t)D;
            for (int d = 0; d < D; ++d) o[d] += w * bf16_to_f64(vr[d]);
        }
        if (fabs(check - 1.0) > err) err = fabs(check - 1.0);
        lse[h] = m + log(sw);
    }
    if (max_wsum_err) *max_wsum_err = err;
    free(q);
    free(l);
}

/* ---------- QSA rows: O3 + O4 + O5 + O6 for a list of query rows -------- */
/* Inputs of one sequence, all already past RoPE / compression:
 *   Q [Tq][H][D] rows for positions pos0 + t; K, V [Tk][Hkv][D];
 *   qi [Tq][Hi][Di]; kbar [nb][Di].
 * For each rows[i] = t: O [n][H][D], lse [n][H], sel [n][K] (ascending, -1
 * padded), nsel [n], sK/sK1 [n] (rank-K, rank-K+1 scores), wsum_err [n]. */
void qsa_oracle_qsa_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                         const uint16_t *qi, const uint16_t *kbar, int64_t nb, int64_t pos0,
                         int H, int Hkv, int D, int Hi, int Di, int r, int Kbudget, int mode,
                         const int64_t *rows, int64_t n, double *O, double *lse, int32_t *sel,
                         int32_t *nsel, double *sK, double *sK1, double *wsum_err) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = rows[i];
        int64_t p = pos0 + t;
        int64_t nc_full = qsa_oracle_num_complete(p, r);
        double *s = (double *)malloc(sizeof(double) * (size_t)(nc_full > 0 ? nc_full : 1));
        int64_t nc = qsa_oracle_scores_row(qi + t * Hi * (int64_t)Di, kbar, nb, p, Hi, Di, r,
                                           mode, s);
        int32_t *blk = sel + i * Kbudget;
        for (int k = 0; k < Kbudget; ++k) blk[k] = -1;
        int ns = qsa_oracle_topk_row(s, nc, Kbudget, blk, &sK[i], &sK1[i]);
        nsel[i] = ns;
        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ns * r + r));
        int64_t ntok = qsa_oracle_token_set(blk, ns, p, r, tok);
        qsa_oracle_attend_row(Q + t * H * (int64_t)D, K, V, H, Hkv, D, tok, ntok,
                              O + i * H * (int64_t)D, lse + i * H, &wsum_err[i]);
        free(tok);
        free(s);
    }
}

/* Same as qsa_oracle_qsa_rows for compact inputs: row i of Q [n][H][D] and
 * of qi [n][Hi][Di] is the query at absolute position pos[i]. */
void qsa_oracle_qsa_rows_at(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                            const uint16_t *qi, const uint16_t *kbar, int64_t nb,
                            const int64_t *pos, int H, int Hkv, int D, int Hi, int Di, int r,
                            int Kbudget, int mode, int64_t n, double *O, double *lse,
                            int32_t *sel, int32_t *nsel, double *sK, double *sK1,
                            double *wsum_err) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t p = pos[i];
        int64_t nc_full = qsa_oracle_num_complete(p, r);
        double *s = (double *)malloc(sizeof(double) * (size_t)(nc_full > 0 ? nc_full : 1));
        int64_t nc = qsa_oracle_scores_row(qi + i * Hi * (int64_t)Di, kbar, nb, p, Hi, Di, r,
                                           mode, s);
        int32_t *blk = sel + i * Kbudget;
        for (int k = 0; k < Kbudget; ++k) blk[k] = -1;
        int ns = qsa_oracle_topk_row(s, nc, Kbudget, blk, &sK[i], &sK1[i]);
        nsel[i] = ns;
        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ns * r + r));
        int64_t ntok = qsa_oracle_token_set(blk, ns, p, r, tok);
        qsa_oracle_attend_row(Q + i * H * (int64_t)D, K, V, H, Hkv, D, tok, ntok,
                              O + i * H * (int64_t)D, lse + i * H, &wsum_err[i]);
        free(tok);
        free(s);
    }
}

/* Attention rows over a GIVEN selection (e.g. one produced elsewhere and
 * validated against the tie band): sel [n][Kbudget] ascending, nsel [n]. */
void qsa_oracle_sparse_attn_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                 int64_t pos0, int H, int Hkv, int D, int r, int Kbudget,
                                 const int64_t *rows, int64_t n, const int32_t *sel,
                                 const int32_t *nsel, double *O, double *lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = rows[i];
        int64_t p = pos0 + t;
        int ns = nsel[i];
        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ns * r + r));
        int64_t ntok = qsa_oracle_token_set(sel + i * Kbudget, ns, p, r, tok);
        double e;
        qsa_oracle_attend_row(Q + t * H * (int64_t)D, K, V, H, Hkv, D, tok, ntok,
                              O + i * H * (int64_t)D, lse + i * H, &e);
        free(tok);
    }
}

/* Same as qsa_oracle_sparse_attn_rows for compact inputs: row i of Q
 * [n][H][D] is the query at absolute position pos[i], with selection row i. */
void qsa_oracle_sparse_attn_rows_at(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                                    const int64_t *pos, int H, int Hkv, int D, int r,
                                    int Kbudget, int64_t n, const int32_t *sel,
                                    const int32_t *nsel, double *O, double *lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        const int64_t p_i = pos[i];
        const int ns_i = nsel[i];
        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ns_i * r + r));
        const int64_t ntok = qsa_oracle_token_set(sel + i * Kbudget, ns_i, p_i, r, tok);
        double e;
        qsa_oracle_attend_row(Q + i * H * (int64_t)D, K, V, H, Hkv, D, tok, ntok,
                              O + i * H * (int64_t)D, lse + i * H, &e);
        free(tok);
    }
}

/* Scores + selection only, for a list of rows: s_out [n][nb_out] (NAN past
 * nc), sel/nsel/sK/sK1 as in qsa_oracle_qsa_rows.  s_out may be NULL. */
void qsa_oracle_select_rows(const uint16_t *qi, const uint16_t *kbar, int64_t nb, int64_t pos0,
                            int Hi, int Di, int r, int Kbudget, int mode, const int64_t *rows,
                            int64_t n, double *s_out, int64_t nb_out, int32_t *sel,
                            int32_t *nsel, double *sK, double *sK1) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = rows[i];
        int64_t p = pos0 + t;
        int64_t nc_full = qsa_oracle_num_complete(p, r);
        double *s = (double *)malloc(sizeof(double) * (size_t)(nc_full > 0 ? nc_full : 1));
        int64_t nc = qsa_oracle_scores_row(qi + t * Hi * (int64_t)Di, kbar, nb, p, Hi, Di, r,
                                           mode, s);
        if (s_out) {
            for (int64_t b = 0; b < nb_out; ++b) s_out[i * nb_out + b] = b < nc ? s[b] : NAN;
        }
        int32_t *blk = sel + i * Kbudget;
        for (int k = 0; k < Kbudget; ++k) blk[k] = -1;
        nsel[i] = qsa_oracle_topk_row(s, nc, Kbudget, blk, &sK[i], &sK1[i]);
        free(s);
    }
}

/* ---------- O7: dense causal attention rows ------------------------------ */
/* Same as O6 with the token set 0..p, p = pos0 + t. */
void qsa_oracle_dense_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                           int64_t pos0, int H, int Hkv, int D, const int64_t *rows, int64_t n,
                           double *O, double *lse) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = rows[i];
        int64_t p = pos0 + t;
        int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(p + 1));
        for (int64_t j = 0; j <= p; ++j) tok[j] = j;
        double e;
        qsa_oracle_attend_row(Q + t * H * (int64_t)D, K, V, H, Hkv, D, tok, p + 1,
                              O + i * H * (int64_t)D, lse + i * H, &e);
        free(tok);
    }
}

/* ---------- O8: stage-1 indexer distillation, forward --------------------- */
/* chlience section 6: the first stage trains the indexer alone against a
 * teacher distribution made from full attention, max-pooled within each
 * micro-block, by minimising a KL divergence.  For the query at position p
 * (its Q row [H][D] and K [*][Hkv][D], both post-RoPE):
 *   A_hj = softmax over j = 0..p of q_h . k_{g(h), j} / sqrt(D)   dense attention
 *   M_hb = max over t < r of A_{h, r*b + t}, for b < nc(p)         block max-pool
 *   T_b  = sum_h M_hb / sum_b' sum_h M_hb'                          heads summed,
 *                                                                   L1-normalised
 *   S_b  = softmax over b < nc(p) of the indexer scores s_b (O3)
 *   KL   = sum_b T_b (ln T_b - ln S_b), with 0 ln 0 = 0.
 * Returns KL (0 when nc(p) = 0); T_out / logS_out (length nc) if not NULL. */
double qsa_oracle_distill_row(const uint16_t *q_row, const uint16_t *K, int H, int Hkv, int D,
                              int64_t p, int r, const double *s, double *T_out,
                              double *logS_out) {
    int64_t nc = qsa_oracle_num_complete(p, r);
    if (nc <= 0) return 0.0;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    double *l = (double *)malloc(sizeof(double) * (size_t)(p + 1));
    double *T = (double *)calloc((size_t)nc, sizeof(double));
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    for (int h = 0; h < H; ++h) {
        const int g = h / (H / Hkv);
        for (int d = 0; d < D; ++d) q[d] = bf16_to_f64(q_row[h * D + d]);
        double m = -INFINITY;
        for (int64_t j = 0; j <= p; ++j) {
            const uint16_t *kr = K + (j * Hkv + g) * (int64_t)D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += q[d] * bf16_to_f64(kr[d]);
            l[j] = dot * inv_sqrt_d;
            if (l[j] > m) m = l[j];
        }
        double z = 0.0;
        for (int64_t j = 0; j <= p; ++j) z += exp(l[j] - m);
        double lse = m + log(z);
        for (int64_t b = 0; b < nc; ++b) {
            double mb = 0.0;
            for (int t = 0; t < r; ++t) {
                double a = exp(l[b * r + t] - lse);
                if (a > mb) mb = a;
            }
            T[b] += mb;
        }
    }
    double zt = 0.0, ms = -INFINITY;
    for (int64_t b = 0; b < nc; ++b) {
        zt += T[b];
        if (s[b] > ms) ms = s[b];
    }
    double zs = 0.0;
    for (int64_t b = 0; b < nc; ++b) zs += exp(s[b] - ms);
    double lse_s = ms + log(zs);
    double kl = 0.0;
    for (int64_t b = 0; b < nc; ++b) {
        double t = T[b] / zt, ls = s[b] - lse_s;
        if (t > 0.0) kl += t * (log(t) - ls);
        if (T_out) T_out[b] = t;
        if (logS_out) logS_out[b] = ls;
    }
    free(q);
    free(l);
    free(T);
    return kl;
}

/* O8 for rows of one sequence: the query at pos0 + rows[i] uses Q row
 * rows[i], indexer row qi[rows[i]] and the pooled keys kbar[nb][Di]. */
void qsa_oracle_distill_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *qi,
                             const uint16_t *kbar, int64_t nb, int64_t pos0, int H, int Hkv,
                             int D, int Hi, int Di, int r, int mode, const int64_t *rows,
                             int64_t n, double *kl) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = rows[i];
        int64_t p = pos0 + t;
        int64_t nc_full = qsa_oracle_num_complete(p, r);
        double *s = (double *)malloc(sizeof(double) * (size_t)(nc_full > 0 ? nc_full : 1));
        qsa_oracle_scores_row(qi + t * Hi * (int64_t)Di, kbar, nb, p, Hi, Di, r, mode, s);
        kl[i] = qsa_oracle_distill_row(Q + t * H * (int64_t)D, K, H, Hkv, D, p, r, s, NULL, NULL);
        free(s);
    }
}

/* ---------- O9: distillation KL under the sparse pattern ------------------ */
/* ai.info "Industry relevance": a fused QSA kernel yields the sparse
 * attention outputs and the KL loss without storing intermediates; chlience
 * section 6: in the second stage backbone and indexer train together under
 * the sparse pattern.  Reading (the pages give no formula for this loss): the
 * teacher is the sparse attention the layer actually computes, i.e. for each
 * head the softmax over the query's token set (its nsel selected blocks and
 * its incomplete block, O5), max-pooled within each selected block, summed
 * over the heads and L1-normalised over the selected blocks; the student is
 * the softmax of the indexer scores over the same selected blocks; the loss
 * is KL(teacher || student) as in O8.  The incomplete block counts in each
 * head's softmax but is not a block of either distribution.
 *   blk[0..nsel) the selected blocks (ascending), s_sel[i] the score of blk[i].
 * With every complete block selected this is O8.  Returns KL (0 when nsel is
 * 0); T_out / logS_out (length nsel) if not NULL. */
double qsa_oracle_sparse_kl_row(const uint16_t *q_row, const uint16_t *K, int H, int Hkv, int D,
                                int64_t p, int r, const int32_t *blk, int nsel,
                                const double *s_sel, double *T_out, double *logS_out) {
    if (nsel <= 0) return 0.0;
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nsel * r + r));
    const int64_t ntok = qsa_oracle_token_set(blk, nsel, p, r, tok);
    double *lg = (double *)malloc(sizeof(double) * (size_t)ntok);
    double *Tb = (double *)calloc((size_t)nsel, sizeof(double));
    const double qk_scale = 1.0 / sqrt((double)D);
    for (int h = 0; h < H; ++h) {
        const int kvh = h / (H / Hkv);
        double mh = -INFINITY;
        for (int64_t j = 0; j < ntok; ++j) {
            const uint16_t *kr = K + (tok[j] * Hkv + kvh) * (int64_t)D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += bf16_to_f64(q_row[h * D + d]) * bf16_to_f64(kr[d]);
            lg[j] = dot * qk_scale;
            mh = lg[j] > mh ? lg[j] : mh;
        }
        double zh = 0.0;
        for (int64_t j = 0; j < ntok; ++j) zh += exp(lg[j] - mh);
        const double lse_h = mh + log(zh);
        /* tokens i*r .. i*r + r - 1 of the set are selected block i */
        for (int i = 0; i < nsel; ++i) {
            double mb = 0.0;
            for (int t = 0; t < r; ++t) {
                const double a = exp(lg[(int64_t)i * r + t] - lse_h);
                mb = a > mb ? a : mb;
            }
            Tb[i] += mb;
        }
    }
    double tsum = 0.0, smax = -INFINITY;
    for (int i = 0; i < nsel; ++i) {
        tsum += Tb[i];
        smax = s_sel[i] > smax ? s_sel[i] : smax;
    }
    double ssum = 0.0;
    for (int i = 0; i < nsel; ++i) ssum += exp(s_sel[i] - smax);
    const double s_lse = smax + log(ssum);
    double acc = 0.0;
    for (int i = 0; i < nsel; ++i) {
        const double ti = Tb[i] / tsum, lsi = s_sel[i] - s_lse;
        if (ti > 0.0) acc += ti * (log(ti) - lsi);
        if (T_out) T_out[i] = ti;
        if (logS_out) logS_out[i] = lsi;
    }
    free(tok);
    free(lg);
    free(Tb);
    return acc;
}

/* O9 for rows of one sequence over a GIVEN selection sel [n][Kbudget] /
 * nsel [n] (ascending blocks, as the attention rows above): the student's
 * scores are O3's for the query at pos0 + rows[i] (indexer row qi[rows[i]],
 * pooled keys kbar[nb][Di]), taken at the selected blocks. */
void qsa_oracle_sparse_kl_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *qi,
                               const uint16_t *kbar, int64_t nb, int64_t pos0, int H, int Hkv,
                               int D, int Hi, int Di, int r, int mode, int Kbudget,
                               const int64_t *rows, int64_t n, const int32_t *sel,
                               const int32_t *nsel, double *kl) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = rows[i];
        int64_t p = pos0 + t;
        int64_t nc_full = qsa_oracle_num_complete(p, r);
        double *s = (double *)malloc(sizeof(double) * (size_t)(nc_full > 0 ? nc_full : 1));
        qsa_oracle_scores_row(qi + t * Hi * (int64_t)Di, kbar, nb, p, Hi, Di, r, mode, s);
        const int ns = nsel[i];
        const int32_t *bi = sel + i * (int64_t)Kbudget;
        double *s_sel = (double *)malloc(sizeof(double) * (size_t)(ns > 0 ? ns : 1));
        for (int k = 0; k < ns; ++k) s_sel[k] = s[bi[k]];
        kl[i] = qsa_oracle_sparse_kl_row(Q + t * H * (int64_t)D, K, H, Hkv, D, p, r, bi, ns,
                                         s_sel, NULL, NULL);
        free(s_sel);
        free(s);
    }
}
