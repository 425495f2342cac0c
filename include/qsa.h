/*
 * qsa.h — C ABI of the MI355X (gfx950) Qwen Sparse Attention (QSA) layer.
 *
 * The layer is the one described on the papers.chlience.com reading notes of
 * "On the Design of Qwen3.8 Next Architecture" (section 6, "GDN continuous
 * compression and QSA exact retrieval"; Model Summary table) and summarised on
 * the ai.info page ("Methodology in Plain English", Key Contribution 3):
 *   keys are pooled over micro-blocks of r = 4 tokens; a multi-query indexer
 *   (4 query heads, one shared key head, dim 128) scores every fully formed
 *   block for each query; at most 512 blocks (2048 tokens) are kept per query
 *   together with the query's incomplete trailing block; softmax attention
 *   (24 query heads, 2 KV heads, dim 256, RoPE on 64 dims) runs over the
 *   kept tokens only.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are raw bit patterns (qsa_bf16), row-major, contiguous in
 *     the layouts given below, 16-byte aligned.  All tensor pointers are
 *     DEVICE pointers owned by the caller; the library never allocates,
 *     frees, synchronises or prints.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work; outputs are valid once the stream reaches that point.
 *     Inputs must not be modified before then.
 *   - Positions: in prefill form (`seq_len == NULL`) query t of every
 *     sequence sits at absolute position pos0 + t.  In decode form
 *     (`seq_len` = device int64 [B], 1 <= Tq <= 16 queries per sequence) the
 *     cache of sequence b holds seq_len[b] tokens and its query i sits at
 *     seq_len[b] - Tq + i.  Tq > 1 is speculative decoding with index reuse
 *     (chlience "5. 贡献全景与方法总览", item 5: the MTP prediction steps reuse
 *     the QSA top-k indices; "Result 2": decode with next_n = 4): the block
 *     selection is made once per sequence, for its first query (position
 *     p0 = seq_len[b] - Tq, indexer query q_idx[b][0]), and query i attends
 *     the selected blocks plus every token from r*nc(p0) up to its own
 *     position.  Tq = 1 is ordinary one-query decode.  Device-side
 *     lengths are not visible to the host: the kernels clamp them to the
 *     allocated sizes (a length above Lmax acts as Lmax, a length < 1 gives an
 *     empty context), so no access leaves the buffers.
 *   - A query at position p sees nc(p) = floor((p+1)/r) complete blocks; its
 *     incomplete block holds tokens r*nc(p) .. p ((p+1) mod r tokens).
 *   - Arguments are checked on the host before any HIP call; the first failed
 *     check's status is returned and nothing is enqueued.  QSA_ERR_LAUNCH is
 *     returned when a launch is rejected; faults inside kernels surface at the
 *     caller's next synchronisation.  Inputs are assumed finite.
 *   - Supported shapes: head_dim 256 with at most 16 query heads per KV head
 *     for attention; indexer 4 heads x 128; r = 4 wherever blocks are read by
 *     attention or the indexer.  Other shapes return QSA_ERR_UNSUPPORTED:
 *     there is no slow fallback.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t qsa_bf16;

typedef enum {
    QSA_OK = 0,
    QSA_ERR_NULL = 1,        /* a required pointer is NULL */
    QSA_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree */
    QSA_ERR_UNSUPPORTED = 3, /* a shape the tuned kernels do not cover */
    QSA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
    QSA_ERR_OVERFLOW = 5,    /* a block index would not fit in int32 */
    QSA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required */
    QSA_ERR_LAUNCH = 7,      /* the HIP runtime rejected a launch */
    QSA_ERR_DEVICE = 8,      /* the current device is not a gfx950 GPU */
    QSA_ERR_SCRATCH = 9      /* the call needs more than the static scratch holds */
} qsa_status;

/* Indexer head combination.
 * MAXHEAD: s = max over heads of <q_h, kbar_b> / sqrt(Di) (default).
 * RELUSUM: s = sum over heads of max(0, <q_h, kbar_b>) (the indexer equation
 *          I_ib of section 6 of the chlience notes). */
typedef enum { QSA_SCORE_MAXHEAD = 0, QSA_SCORE_RELUSUM = 1 } qsa_score_mode;

/* Pooled key.
 * MEAN:    kbar_b = mean of the r keys of block b (average pooling, ai.info
 *          "Methodology in Plain English"; default).
 * RMSNORM: kbar_b = RMSNorm(mean) with unit gain and eps 1e-6 (the k-bar
 *          equation of section 6 of the chlience notes).
 * Either result is rounded to bf16, nearest even. */
typedef enum { QSA_KBAR_MEAN = 0, QSA_KBAR_RMSNORM = 1 } qsa_kbar_mode;

/* Paged caches (chlience "Result 2": the report's kernel measurement uses a
 * paged GQA dense baseline).  The cache of sequence b is cut into pages of page_tokens
 * tokens; table[b * table_stride + i] is the pool index of its i-th page.
 * With a qsa_pages argument the cache tensors of a call are page pools:
 *   K, V:  [n_pages * page_tokens][Hkv][D]     (token rows)
 *   kbar:  [n_pages * page_tokens / r][Di]     (pooled-block rows)
 * so token t of sequence b is row table[b*table_stride + t / page_tokens] *
 * page_tokens + t mod page_tokens, and pooled block j is row
 * table[b*table_stride + j*r / page_tokens] * (page_tokens / r) +
 * j mod (page_tokens / r).  table is a DEVICE int32 array; page_tokens a
 * power of two in 16 .. 4096; table_stride must cover the longest cache of
 * the call.  The kernels read the pages of the tokens (blocks) their queries
 * see, and only those: their table entries must be valid pool indices.
 * A NULL qsa_pages pointer selects the contiguous layouts given per call. */
typedef struct {
    const int32_t *table;
    int64_t table_stride;
    int page_tokens;
} qsa_pages;

/* Human-readable name of a status code (static string). */
const char *qsa_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int qsa_version(void);

/* QSA_OK if the current HIP device is a gfx950 (MI355X-class) GPU. */
int qsa_check_device(void);

/* ---- A1: partial rotary embedding (Model Summary table: RoPE dimension 64).
 * y[t][h][:] = x[t][h][:] with each pair (j, j + rope_dim/2), j < rope_dim/2,
 * rotated counter-clockwise by the angle pos(t) * theta^(-2j/rope_dim)
 * (angles and products in fp64), the result rounded to bf16 (nearest even);
 * dims >= rope_dim are copied.  x, y: [T][nheads][head_dim]; y may equal x.
 * pos(t) = pos0 + t, or, when seq_len (device int64 [T / next_n]) is given,
 * seq_len[t / next_n] - next_n + t % next_n (decode form: next_n queries per
 * sequence, rows grouped by sequence); positions below 0 rotate as 0.
 * Supported: head_dim in {64,128,256,512}, even rope_dim <= min(head_dim, 128),
 * 1 <= next_n <= 16 (T % next_n == 0 in the decode form; ignored otherwise). */
int qsa_rope_bf16(const qsa_bf16 *x, qsa_bf16 *y, int64_t T, int nheads, int head_dim,
                  int rope_dim, double theta, int64_t pos0, const int64_t *seq_len, int next_n,
                  void *stream);

/* ---- A2: key compression (chlience section 6, k-bar equation).
 * For each sequence b < B and block j < Tk / r:
 *   kbar[b*kbar_seq_stride + j*Di + :] = pool(k[b*k_seq_stride + (j*r + t)*Di + :], t < r)
 * Sums are formed in fp64 in token order, so MEAN mode is exact before the
 * single bf16 rounding.  In RMSNORM mode the normalised key is multiplied by
 * the gain gain[0 .. Di-1] (bf16, NULL = unit gain).  With rope_dim > 0 the
 * pooled key is then rotated like qsa_rope_bf16 over its first rope_dim dims
 * (pairs (j, j + rope_dim/2), base theta) at the position of the block's first
 * token, r * (block0 + j): the same section pools first and applies partial
 * RoPE after, so tokens at different phases are never averaged (indexer
 * queries are then rotated at their own positions with qsa_rope_bf16).
 * Pooling, normalisation and rotation run in fp64 with one bf16 rounding.
 * Strides are in elements; Tk % r tokens at the end are ignored; block0 is
 * the index of the first pooled block (appending blocks to a cache).
 * Supported: Di in {64,128,256}, 1 <= r <= 16, rope_dim 0 or a power of two
 * in 16 .. min(Di, 128). */
int qsa_compress_keys(const qsa_bf16 *k, int B, int64_t Tk, int64_t k_seq_stride, int Di, int r,
                      int kbar_mode, const qsa_bf16 *gain, int rope_dim, double theta,
                      int64_t block0, qsa_bf16 *kbar, int64_t kbar_seq_stride,
                      const qsa_pages *pages, void *stream);

/* ---- A3: indexer block scores (chlience section 6, I_ib; ai.info
 * contribution 3: MQA indexer, 4 query heads and one shared key head).
 * q_idx: [B][Tq][Hi][Di]; kbar: [B][nb_max][Di]; scores: fp32 [B][Tq][ld]
 * (decode form: [B][ld], one row per sequence, for its first query).
 * scores[b][t][j] for j < nc = min(nc(p), nb_max) holds the block score of
 * query t against pooled block j.  Entries j >= nc may be left untouched or
 * set to -inf (callers read only j < nc).
 * Prefill form: positions pos0 + t; decode form: see conventions.
 * Supported: Hi = 4, Di = 128, r = 4, ld >= nb_max, ld % 4 == 0. */
int qsa_index_scores(const qsa_bf16 *q_idx, const qsa_bf16 *kbar, int B, int64_t Tq,
                     int64_t pos0, const int64_t *seq_len, int64_t nb_max, int Hi, int Di, int r,
                     int score_mode, float *scores, int64_t ld, const qsa_pages *pages,
                     void *stream);

/* ---- A4: per-query top-K block selection (chlience section 6: at most 512
 * complete blocks per query; djimit pillar 2: up to 512 full blocks).
 * If nc <= K all nc blocks are taken, else the K largest scores, ties broken
 * by lower block index (scores compare as fp32 values; -0 equals +0).
 * blk_idx: int32 [B][Tq][K], ascending, padded with -1;
 * n_sel: int32 [B][Tq] = min(K, nc).  scores as produced by qsa_index_scores.
 * Decode form: one selection per sequence (scores [B][ld], blk_idx [B][K],
 * n_sel [B]), for the sequence's first query.
 * Workspace: qsa_topk_workspace_bytes(B, Tq, nb_max, K) bytes, 16-byte
 * aligned: the per-segment candidate lists of rows longer than 32,768 blocks
 * (or of few long rows, as in decode).  It is 0 when every row fits one pass;
 * ws may then be NULL.  Contents need no initialisation and are scratch.
 * Supported: 1 <= K <= 2048, ld >= nb_max, ld % 4 == 0. */
size_t qsa_topk_workspace_bytes(int B, int64_t Tq, int64_t nb_max, int K);
int qsa_topk_blocks(const float *scores, int B, int64_t Tq, int64_t ld, int64_t pos0,
                    const int64_t *seq_len, int64_t nb_max, int r, int K, int32_t *blk_idx,
                    int32_t *n_sel, void *ws, size_t ws_bytes, void *stream);

/* ---- A3 + A4 in one call: exactly the result of qsa_index_scores followed
 * by qsa_topk_blocks (same scores bit for bit, same tie order).  The scores
 * live in the caller's workspace (qsa_select_workspace_bytes, 16-byte
 * aligned), one chunk of query rows at a time (at most 8 GiB of fp32 scores
 * per chunk, the largest score of every 16 blocks of each row, from which
 * the top-K of long rows takes its floor and skips the groups below it, and
 * the top-K candidate lists of the chunk), so the workspace stays bounded at
 * any Tq; the decode form keeps one row per sequence, and
 * for long rows also the maxima of every 64 blocks and the candidate lists
 * of a filter pass (about 12 bytes per block and sequence in all).
 * Supported: as the two calls, and nb_max < 2^27. */
size_t qsa_select_workspace_bytes(int B, int64_t Tq, int64_t nb_max, int K);
int qsa_select_blocks(const qsa_bf16 *q_idx, const qsa_bf16 *kbar, int B, int64_t Tq,
                      int64_t pos0, const int64_t *seq_len, int64_t nb_max, int Hi, int Di,
                      int r, int score_mode, int K, int32_t *blk_idx, int32_t *n_sel, void *ws,
                      size_t ws_bytes, const qsa_pages *pages, void *stream);

/* ---- A5 + A6: sparse attention, prefill (chlience section 6: the selected
 * blocks expand to token indices for the core attention; the incomplete
 * trailing block is always kept).  One sequence.
 * Q: [Tq][H][D] post-RoPE, queries at pos0 .. pos0+Tq-1;
 * K, V: [Tk][Hkv][D] post-RoPE keys, Tk >= pos0 + Tq;
 * blk_idx/n_sel as from qsa_topk_blocks (entries must be < nc of the row);
 * O: fp32 [Tq][H][D];  lse: fp32 [Tq][H] natural-log sum of exp of the
 * scaled logits, or NULL.  Query head h reads KV head h / (H / Hkv); logits
 * are q.k / sqrt(D).  Supported: D = 256, H % Hkv == 0, H / Hkv <= 16, r = 4,
 * Tq * Hkv < 2^26 (one 64-thread workgroup per query and KV head; larger
 * Tq: QSA_ERR_OVERFLOW, split the rows into several calls). */
int qsa_sparse_attn_prefill(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                            const int32_t *blk_idx, const int32_t *n_sel, int64_t Tq, int64_t Tk,
                            int64_t pos0, int H, int Hkv, int D, int r, int Kbudget, float *O,
                            float *lse, const qsa_pages *pages, void *stream);

/* ---- A1 + A5 + A6: the same sparse prefill attention with the queries'
 * partial RoPE (Model Summary table: RoPE dimension 64) applied as they are
 * loaded.  Q: [Tq][H][D] BEFORE RoPE; the result equals, bit for bit,
 * qsa_rope_bf16(Q -> Qr, Tq, H, D, rope_dim, theta, pos0) followed by
 * qsa_sparse_attn_prefill(Qr, ...), without writing or reading Qr (the
 * rotated queries are never stored).  Arguments otherwise as
 * qsa_sparse_attn_prefill.  Supported: rope_dim 64 or 128 (the NeoX pair
 * partners then sit in one lane's fragment), theta > 0. */
int qsa_sparse_attn_prefill_rope(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                                 const int32_t *blk_idx, const int32_t *n_sel, int64_t Tq,
                                 int64_t Tk, int64_t pos0, int H, int Hkv, int D, int r,
                                 int Kbudget, int rope_dim, double theta, float *O, float *lse,
                                 const qsa_pages *pages, void *stream);

/* ---- A7: sparse attention, decode: the Tq newest queries of each sequence
 * (Tq = 1, or next_n speculative queries sharing one selection; see the
 * position conventions).
 * q: [B][Tq][H][D] post-RoPE; Kc, Vc: [B][Lmax][Hkv][D]; seq_len: device
 * int64 [B]; blk_idx: [B][Kbudget] and n_sel: [B], the selection made for
 * position seq_len[b] - Tq (entries must be < nc of that position);
 * O: fp32 [B][Tq][H][D]; lse: fp32 [B][Tq][H] or NULL.  A query with no
 * visible token (position < 0) gets O = 0 and lse = -inf.
 * Workspace: qsa_decode_workspace_bytes (split partial results).
 * Supported: 1 <= Tq <= 16, and as the prefill call. */
size_t qsa_decode_workspace_bytes(int B, int Tq, int H, int Hkv, int D, int Kbudget);
int qsa_sparse_attn_decode(const qsa_bf16 *q, const qsa_bf16 *Kc, const qsa_bf16 *Vc,
                           const int64_t *seq_len, const int32_t *blk_idx, const int32_t *n_sel,
                           int B, int Tq, int64_t Lmax, int H, int Hkv, int D, int r,
                           int Kbudget, float *O, float *lse, void *ws, size_t ws_bytes,
                           const qsa_pages *pages, void *stream);

/* ---- A1 + A7: the same decode attention with the queries' partial RoPE
 * (Model Summary table: RoPE dimension 64) applied as they are loaded.
 * q: [B][Tq][H][D] BEFORE RoPE; the result equals, bit for bit,
 * qsa_rope_bf16 of q in its decode form (row b * Tq + i at position
 * seq_len[b] - Tq + i, at least 0) followed by qsa_sparse_attn_decode on the
 * rotated rows, without writing or reading them.  Arguments otherwise,
 * workspace and support as qsa_sparse_attn_decode; rope_dim 64 or 128,
 * theta > 0 (else QSA_ERR_SHAPE / QSA_ERR_UNSUPPORTED before any launch). */
int qsa_sparse_attn_decode_rope(const qsa_bf16 *q, const qsa_bf16 *Kc, const qsa_bf16 *Vc,
                                const int64_t *seq_len, const int32_t *blk_idx,
                                const int32_t *n_sel, int B, int Tq, int64_t Lmax, int H, int Hkv,
                                int D, int r, int Kbudget, int rope_dim, double theta, float *O,
                                float *lse, void *ws, size_t ws_bytes, const qsa_pages *pages,
                                void *stream);

/* ---- A7 without allocation: qsa_sparse_attn_decode for callers that cannot
 * allocate device memory or hand over a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * arguments and results are those of qsa_sparse_attn_decode without ws and
 * ws_bytes; the same kernels run, and the split records live instead in a
 * static device array of qsa_decode_noalloc_max_bytes() bytes (64 MiB) that
 * each GPU the library runs on holds until the process ends.  The call
 * allocates nothing.  A call whose records need more than that array
 * (qsa_decode_workspace_bytes > 64 MiB, e.g. more than about 1,900 sequences
 * at Tq = 1) returns QSA_ERR_SCRATCH and enqueues nothing.
 * Every call on one GPU shares that GPU's array, whatever its stream: calls
 * whose work overlaps on one GPU (on different streams, or from several host
 * threads) race on it and give undefined results; order them on one stream
 * or with events.  Each call writes every record it later reads, so no
 * contents carry over from an earlier call. */
size_t qsa_decode_noalloc_max_bytes(void);
int qsa_sparse_attn_decode_noalloc(const qsa_bf16 *q, const qsa_bf16 *Kc, const qsa_bf16 *Vc,
                                   const int64_t *seq_len, const int32_t *blk_idx,
                                   const int32_t *n_sel, int B, int Tq, int64_t Lmax, int H,
                                   int Hkv, int D, int r, int Kbudget, float *O, float *lse,
                                   const qsa_pages *pages, void *stream);

/* ---- A8: dense causal attention (the pages' baseline in the chlience
 * Result 2 kernel measurement).
 * Q: [B][Tq][H][D]; K, V: [B][Lmax][Hkv][D]; O: fp32 [B][Tq][H][D];
 * lse: fp32 [B][Tq][H] or NULL.  Prefill form: query t attends keys
 * 0 .. pos0 + t (pos0 + Tq <= Lmax), a flash-attention pass whose P.V
 * product runs in fp16 (P and V rounded to fp16: V must lie within the fp16
 * range, |v| < 65504; values below 2^-14 lose relative precision), fp32
 * logits, softmax and accumulation.  Decode form: the Tq <= 16 newest
 * queries of each sequence, query i attending keys 0 .. seq_len[b] - Tq + i,
 * with the split-K kernel of the sparse decode path.
 * Workspace: dense_attn_workspace_bytes: the decode form's need for Tq
 * queries per sequence (the prefill form needs none; ws may be NULL). */
size_t dense_attn_workspace_bytes(int B, int64_t Tq, int64_t Lmax, int H, int Hkv, int D);
int dense_attn(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V, int B, int64_t Tq,
               int64_t Lmax, int64_t pos0, const int64_t *seq_len, int H, int Hkv, int D,
               float *O, float *lse, void *ws, size_t ws_bytes, const qsa_pages *pages,
               void *stream);

/* ---- Stage-1 indexer distillation, forward (chlience section 6: the first
 * QSA training stage trains the indexer alone, its teacher being the full
 * attention distribution max-pooled inside each micro-block, with a KL
 * objective; ai.info "Industry relevance": a fused kernel yields the KL loss
 * without materialising intermediates).  One sequence, prefill form.  For the
 * query at p = pos0 + t with nc = nc(p) complete blocks:
 *   teacher T_b = sum over heads h of max over the r tokens j of block b of
 *                 exp(q_h.k_j / sqrt(D) - lse_h), then divided by its sum
 *                 over b (lse_h: log-sum-exp over all keys 0 .. p);
 *   student S_b = softmax over b < nc of the indexer scores (qsa_index_scores);
 *   kl[t]       = sum_b T_b (ln T_b - ln S_b)   (0 when nc = 0).
 * Q: [Tq][H][D] post-RoPE; K: [Tk][Hkv][D] post-RoPE, Tk >= pos0 + Tq;
 * lse: fp32 [Tq][H] from dense_attn over the same Q and K; q_idx:
 * [Tq][Hi][Di]; kbar: [Tk / r][Di] (the indexer inputs as for
 * qsa_index_scores); kl: fp32 [Tq].  The attention probabilities and the
 * per-block teacher never leave the kernel; the indexer scores of one chunk
 * of rows pass through the workspace (at most 8 GiB).
 * Workspace: qsa_distill_workspace_bytes (0 when Tk < r: ws may be NULL).
 * Supported: H = 24, Hkv = 2, D = 256, Hi = 4, Di = 128, r = 4. */
size_t qsa_distill_workspace_bytes(int64_t Tq, int64_t Tk);
int qsa_distill_kl(const qsa_bf16 *Q, const qsa_bf16 *K, const float *lse, const qsa_bf16 *q_idx,
                   const qsa_bf16 *kbar, int64_t Tq, int64_t Tk, int64_t pos0, int H, int Hkv,
                   int D, int Hi, int Di, int r, int score_mode, float *kl, void *ws,
                   size_t ws_bytes, void *stream);

/* ---- Sparse attention prefill fused with the distillation KL under the
 * sparse pattern (ai.info "Industry relevance": a fused QSA kernel yields the
 * sparse attention outputs and the KL loss without materialising
 * intermediates; chlience section 6: the second stage trains backbone and
 * indexer together under the sparse pattern).  The pages give no formula for
 * this loss; it is read as the stage-1 loss above with the dense attention
 * replaced by the sparse attention the layer computes.  For the query at
 * p = pos0 + t with its ns selected blocks (n_sel, clamped as in
 * qsa_sparse_attn_prefill):
 *   O, lse      exactly as qsa_sparse_attn_prefill;
 *   teacher T_b = for each selected block b, sum over heads h of the largest
 *                 probability A_hj over the r tokens j of the block, where
 *                 A_h is the softmax over the query's token set (selected
 *                 blocks and incomplete block: the lse above); divided by its
 *                 sum over the selected blocks;
 *   student S_b = softmax over the selected blocks of their indexer scores
 *                 (qsa_index_scores' values, recomputed in the kernel);
 *   kl[t]       = sum_b T_b (ln T_b - ln S_b)   (0 when ns = 0).
 * Q, K, V, blk_idx, n_sel, O, lse as for qsa_sparse_attn_prefill (contiguous
 * caches, one sequence, lse may be NULL); q_idx: [Tq][Hi][Di] the chunk's
 * indexer queries as given to the selection; kbar: [Tk / r][Di];
 * score_mode: the selection's; kl: fp32 [Tq].  Probabilities, block maxima
 * and scores stay on chip (LDS: 112 bytes per budget entry plus 16.5 KB per
 * query's workgroup).  No workspace.
 * Supported: H = 24, Hkv = 2, D = 256, Hi = 4, Di = 128, r = 4,
 * Kbudget <= 1024, Tq < 2^25. */
int qsa_sparse_attn_prefill_kl(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                               const qsa_bf16 *q_idx, const qsa_bf16 *kbar,
                               const int32_t *blk_idx, const int32_t *n_sel, int64_t Tq,
                               int64_t Tk, int64_t pos0, int H, int Hkv, int D, int Hi, int Di,
                               int r, int Kbudget, int score_mode, float *O, float *lse,
                               float *kl, void *stream);

/* ---- The same distillation KL and sparse attention in two launches, for
 * throughput (ai.info "Industry relevance" and chlience section 6 as above).
 * The first launch is the plain sparse prefill (one wave per query and KV
 * head, the KV heads on separate XCDs, all its waves resident at once),
 * which also writes, per query, the max logit of every (selected block,
 * head) and each head's log-sum-exp to the workspace; the second turns them
 * into the teacher's block masses and the KL, with the student scores
 * recomputed as in the one-kernel form.  O, lse and kl equal the one-kernel
 * form's bit for bit (same arithmetic in the same order).  rope_dim 0: Q is
 * post-RoPE; rope_dim 64 or 128: Q is before RoPE and is rotated on load
 * with base theta, as qsa_sparse_attn_prefill_rope.  Workspace:
 * qsa_sparse_attn_prefill_kl_staged_workspace_bytes(Tq, Kbudget) bytes,
 * 16-byte aligned, scratch (about 48 KB per query at Kbudget 512; callers
 * bound it by calling per chunk of rows); the bytes function returns 0 for
 * invalid arguments.  Other arguments and support as
 * qsa_sparse_attn_prefill_kl, except Kbudget <= 2048. */
size_t qsa_sparse_attn_prefill_kl_staged_workspace_bytes(int64_t Tq, int Kbudget);
int qsa_sparse_attn_prefill_kl_staged(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                                      const qsa_bf16 *q_idx, const qsa_bf16 *kbar,
                                      const int32_t *blk_idx, const int32_t *n_sel, int64_t Tq,
                                      int64_t Tk, int64_t pos0, int H, int Hkv, int D, int Hi,
                                      int Di, int r, int Kbudget, int score_mode, int rope_dim,
                                      double theta, float *O, float *lse, float *kl, void *ws,
                                      size_t ws_bytes, void *stream);

/* ---- Launch sizing of the sparse prefill (A6; the same kernels as
 * qsa_sparse_attn_prefill and, with with_kl, qsa_sparse_attn_prefill_kl;
 * paged: over page pools).  Returns the number of queries whose workgroups
 * (Hkv one-wave workgroups per query; with_kl: one workgroup per query) the
 * current device holds at once: the kernel's resident workgroups per CU
 * times the CUs, over Hkv for the plain forms (1,536 on MI355X for Hkv = 2
 * and budget 512).  Every query costs about the same at a full budget, so workgroups
 * run in rounds of this size; a caller that splits a long prefill into
 * launches of this many queries leaves no round partly empty.  Returns 0
 * for unsupported arguments (Hkv not 1, 2 or 4; Kbudget outside 1..2048;
 * with_kl with paged, Hkv != 2 or Kbudget > 1024) or when the runtime
 * cannot say.  Enqueues nothing. */
int qsa_sparse_attn_prefill_concurrency(int Hkv, int Kbudget, int with_kl, int paged);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
