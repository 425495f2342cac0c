// C ABI of libqsa: host-side argument checks, workspace sizing and dispatch
// to the HIP launchers.  Every check runs before the first HIP call, so a
// rejected call enqueues nothing (and can be tested without a GPU).
#include <math.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/qsa.h"
#include "qsa_internal.h"

using namespace qsa;

namespace {

constexpr int64_t kI32Max = 2147483647;
constexpr int kMaxBudget = 2048;
constexpr int kMaxKlBudget = 1024;  // block maxima of 24 heads in LDS
constexpr int kMaxNextN = 16;  // queries per sequence in the decode form

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_LAUNCH; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Rows of one prefill score chunk (the scores of a chunk, at most 8 GiB, live
// in the workspace; top-K reads them back before the next chunk is scored).
// Fewer, larger chunks leave fewer kernel tails idle: 4 GiB against 1 GiB
// measured 9% faster at a 1M-token context, 8 GiB against 4 GiB 0.2 ms less
// selection per 128K prefill; 8 GiB is small beside 288 GB.  Chunks are whole
// 128-query tiles of the indexer.
constexpr int64_t kScoreChunkBytes = int64_t(1) << 33;

int64_t select_chunk_rows(int64_t Tq, int64_t ld) {
    int64_t rows = kScoreChunkBytes / (ld * 4);
    rows = rows / 128 * 128;
    if (rows < 128) rows = 128;
    return rows < Tq ? rows : Tq;
}

int check_attn_shape(int H, int Hkv, int D, int r) {
    if (H <= 0 || Hkv <= 0 || D <= 0 || r <= 0) return QSA_ERR_SHAPE;
    if (H % Hkv != 0) return QSA_ERR_SHAPE;
    if (D != kHeadDim || r != kBlock) return QSA_ERR_UNSUPPORTED;
    if (H / Hkv > 16 || (Hkv != 1 && Hkv != 2 && Hkv != 4)) return QSA_ERR_UNSUPPORTED;
    return QSA_OK;
}

// A paged-cache argument: NULL, or a table covering `tokens` per sequence
// with a supported page size.
int check_pages(const qsa_pages *pg, int64_t tokens) {
    if (!pg) return QSA_OK;
    if (!pg->table) return QSA_ERR_NULL;
    const int P = pg->page_tokens;
    if (P < 16 || P > 4096 || (P & (P - 1))) return QSA_ERR_UNSUPPORTED;
    if (pg->table_stride < (tokens + P - 1) / P) return QSA_ERR_SHAPE;
    return QSA_OK;
}

int log2_int(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}

// Page tables over token rows (K, V) and over pooled-block rows (kbar).
PageTable token_pages(const qsa_pages *pg) {
    return pg ? PageTable{pg->table, pg->table_stride, log2_int(pg->page_tokens)}
              : PageTable{nullptr, 0, 0};
}

PageTable block_pages(const qsa_pages *pg) {
    return pg ? PageTable{pg->table, pg->table_stride, log2_int(pg->page_tokens / kBlock)}
              : PageTable{nullptr, 0, 0};
}

}  // namespace

extern "C" {

const char *qsa_status_string(int status) {
    switch (status) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_NULL: return "QSA_ERR_NULL: a required pointer is NULL";
    case QSA_ERR_SHAPE: return "QSA_ERR_SHAPE: a size is out of range or sizes disagree";
    case QSA_ERR_UNSUPPORTED: return "QSA_ERR_UNSUPPORTED: shape not covered by the tuned kernels";
    case QSA_ERR_ALIGN: return "QSA_ERR_ALIGN: tensor pointer not 16-byte aligned";
    case QSA_ERR_OVERFLOW: return "QSA_ERR_OVERFLOW: index range exceeds int32";
    case QSA_ERR_WORKSPACE: return "QSA_ERR_WORKSPACE: workspace missing or too small";
    case QSA_ERR_LAUNCH: return "QSA_ERR_LAUNCH: the HIP runtime rejected a launch";
    case QSA_ERR_DEVICE: return "QSA_ERR_DEVICE: current device is not a gfx950 GPU";
    case QSA_ERR_SCRATCH:
        return "QSA_ERR_SCRATCH: the call needs more than the library's static scratch holds";
    default: return "unknown qsa_status";
    }
}

int qsa_version(void) { return 100; }

int qsa_check_device(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QSA_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QSA_ERR_DEVICE;
    return strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? QSA_OK : QSA_ERR_DEVICE;
}

int qsa_rope_bf16(const qsa_bf16 *x, qsa_bf16 *y, int64_t T, int nheads, int head_dim,
                  int rope_dim, double theta, int64_t pos0, const int64_t *seq_len, int next_n,
                  void *stream) {
    if (!x || !y) return QSA_ERR_NULL;
    if (T < 0 || nheads <= 0 || head_dim <= 0 || rope_dim <= 0 || !(theta > 0.0) || pos0 < 0)
        return QSA_ERR_SHAPE;
    if (next_n < 1 || next_n > kMaxNextN) return QSA_ERR_SHAPE;
    if (seq_len && T % next_n != 0) return QSA_ERR_SHAPE;
    if (rope_dim > head_dim || (rope_dim & 1)) return QSA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
        return QSA_ERR_UNSUPPORTED;
    if (rope_dim > 128 || (rope_dim % 8) != 0) return QSA_ERR_UNSUPPORTED;
    if (T > kI32Max) return QSA_ERR_OVERFLOW;
    if (!aligned16(x) || !aligned16(y)) return QSA_ERR_ALIGN;
    double inv_freq[64];
    for (int j = 0; j < rope_dim / 2; ++j)
        inv_freq[j] = pow(theta, -2.0 * static_cast<double>(j) / static_cast<double>(rope_dim));
    return launch_status(launch_rope(x, y, T, nheads, head_dim, rope_dim, inv_freq, pos0,
                                     seq_len, next_n, as_stream(stream)));
}

int qsa_compress_keys(const qsa_bf16 *k, int B, int64_t Tk, int64_t k_seq_stride, int Di, int r,
                      int kbar_mode, const qsa_bf16 *gain, int rope_dim, double theta,
                      int64_t block0, qsa_bf16 *kbar, int64_t kbar_seq_stride,
                      const qsa_pages *pages, void *stream) {
    if (!k || !kbar) return QSA_ERR_NULL;
    if (B <= 0 || Tk < 0 || Di <= 0 || r <= 0 || block0 < 0) return QSA_ERR_SHAPE;
    if (kbar_mode != QSA_KBAR_MEAN && kbar_mode != QSA_KBAR_RMSNORM) return QSA_ERR_SHAPE;
    if (rope_dim < 0 || rope_dim > Di || (rope_dim > 0 && !(theta > 0.0))) return QSA_ERR_SHAPE;
    if (Di != 64 && Di != 128 && Di != 256) return QSA_ERR_UNSUPPORTED;
    if (r > 16) return QSA_ERR_UNSUPPORTED;
    if (rope_dim != 0 && (rope_dim < 16 || rope_dim > 128 || (rope_dim & (rope_dim - 1))))
        return QSA_ERR_UNSUPPORTED;
    if (gain && !aligned16(gain)) return QSA_ERR_ALIGN;
    const int64_t nb = Tk / r;
    if (B > 1 && (k_seq_stride < Tk * Di || (!pages && kbar_seq_stride < nb * Di)))
        return QSA_ERR_SHAPE;
    if (pages && r != kBlock) return QSA_ERR_UNSUPPORTED;
    int st = check_pages(pages, (block0 + nb) * r);
    if (st != QSA_OK) return st;
    if (k_seq_stride % 8 || kbar_seq_stride % 8) return QSA_ERR_ALIGN;
    if (static_cast<int64_t>(B) * nb * (Di / 8) / 256 > kI32Max) return QSA_ERR_OVERFLOW;
    if (!aligned16(k) || !aligned16(kbar)) return QSA_ERR_ALIGN;
    double inv_freq[64];
    for (int j = 0; j < rope_dim / 2; ++j)
        inv_freq[j] = pow(theta, -2.0 * static_cast<double>(j) / static_cast<double>(rope_dim));
    return launch_status(launch_compress(k, B, Tk, k_seq_stride, Di, r, kbar_mode, gain,
                                         rope_dim, rope_dim ? inv_freq : nullptr, block0, kbar,
                                         kbar_seq_stride, as_stream(stream),
                                         block_pages(pages)));
}

static int check_index_args(const qsa_bf16 *q_idx, const qsa_bf16 *kbar, int B, int64_t Tq,
                            int64_t pos0, const int64_t *seq_len, int64_t nb_max, int Hi, int Di,
                            int r, int score_mode) {
    if (!q_idx || !kbar) return QSA_ERR_NULL;
    if (B <= 0 || Tq < 0 || nb_max < 0 || pos0 < 0 || Hi <= 0 || Di <= 0 || r <= 0)
        return QSA_ERR_SHAPE;
    if (score_mode != QSA_SCORE_MAXHEAD && score_mode != QSA_SCORE_RELUSUM) return QSA_ERR_SHAPE;
    if (seq_len && (Tq < 1 || Tq > kMaxNextN)) return QSA_ERR_SHAPE;
    if (Hi != kIdxHeads || Di != kIdxDim || r != kBlock) return QSA_ERR_UNSUPPORTED;
    if (nb_max > kI32Max || B > 65535) return QSA_ERR_OVERFLOW;
    if ((Tq + 63) / 64 > kI32Max) return QSA_ERR_OVERFLOW;
    if (!aligned16(q_idx) || !aligned16(kbar)) return QSA_ERR_ALIGN;
    return QSA_OK;
}

int qsa_index_scores(const qsa_bf16 *q_idx, const qsa_bf16 *kbar, int B, int64_t Tq,
                     int64_t pos0, const int64_t *seq_len, int64_t nb_max, int Hi, int Di, int r,
                     int score_mode, float *scores, int64_t ld, const qsa_pages *pages,
                     void *stream) {
    int st = check_index_args(q_idx, kbar, B, Tq, pos0, seq_len, nb_max, Hi, Di, r, score_mode);
    if (st != QSA_OK) return st;
    if (!scores) return QSA_ERR_NULL;
    if (ld < nb_max || ld % 4 != 0) return QSA_ERR_SHAPE;
    if (!aligned16(scores)) return QSA_ERR_ALIGN;
    st = check_pages(pages, nb_max * r);
    if (st != QSA_OK) return st;
    return launch_status(launch_index_scores(q_idx, kbar, B, Tq, pos0, seq_len, nb_max,
                                             score_mode, scores, ld, as_stream(stream), nullptr,
                                             0, block_pages(pages)));
}

size_t qsa_topk_workspace_bytes(int B, int64_t Tq, int64_t nb_max, int K) {
    if (B <= 0 || Tq <= 0 || nb_max <= 0 || K <= 0) return 0;
    // prefill form: B * Tq rows; decode form (Tq <= 16): B rows
    const size_t pre = topk_plan(static_cast<int64_t>(B) * Tq, nb_max, K).ws_bytes;
    const size_t dec = Tq <= kMaxNextN ? topk_plan(B, nb_max, K).ws_bytes : 0;
    return pre > dec ? pre : dec;
}

int qsa_topk_blocks(const float *scores, int B, int64_t Tq, int64_t ld, int64_t pos0,
                    const int64_t *seq_len, int64_t nb_max, int r, int K, int32_t *blk_idx,
                    int32_t *n_sel, void *ws, size_t ws_bytes, void *stream) {
    if (!scores || !blk_idx || !n_sel) return QSA_ERR_NULL;
    if (B <= 0 || Tq < 0 || nb_max < 0 || pos0 < 0 || r <= 0 || K <= 0) return QSA_ERR_SHAPE;
    if (seq_len && (Tq < 1 || Tq > kMaxNextN)) return QSA_ERR_SHAPE;
    if (ld < nb_max || ld % 4 != 0) return QSA_ERR_SHAPE;
    if (K > kMaxBudget) return QSA_ERR_UNSUPPORTED;
    if (nb_max > kI32Max || static_cast<int64_t>(B) * Tq > kI32Max) return QSA_ERR_OVERFLOW;
    if (!aligned16(scores)) return QSA_ERR_ALIGN;
    if (Tq == 0) return QSA_OK;
    const size_t need = qsa_topk_workspace_bytes(B, Tq, nb_max, K);
    if (need > 0 && (!ws || ws_bytes < need)) return QSA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return QSA_ERR_ALIGN;
    return launch_status(launch_topk(scores, B, Tq, ld, pos0, seq_len, nb_max, r, K, blk_idx,
                                     n_sel, ws, as_stream(stream)));
}

// Workspace of qsa_select_blocks: the fp32 scores of one chunk of query rows
// (all rows in the decode form), then the top-K candidate lists of that chunk.
// Prefill chunks: the scores [chunk][ld] and their 16-block group maxima
// [chunk][gld] (gld = ld / 16 rounded up to whole 64-block tiles), then the
// top-K workspace.
static int64_t gmax_ld(int64_t ld) { return round_up(ld, 64) / 16; }

static void select_layout(int B, int64_t Tq, int64_t nb_max, int K, bool decode, int64_t *ld,
                          int64_t *chunk, size_t *score_bytes, size_t *topk_bytes) {
    *ld = round_up(nb_max > 0 ? nb_max : 1, 4);
    *chunk = decode ? 1 : select_chunk_rows(Tq, *ld);
    const int64_t rows = decode ? B : *chunk;
    *score_bytes = static_cast<size_t>(round_up(rows * *ld * 4, 256));
    if (!decode) *score_bytes += static_cast<size_t>(round_up(rows * gmax_ld(*ld) * 4, 256));
    *topk_bytes = topk_plan(rows, nb_max, K).ws_bytes;
    if (decode) {  // or the decode-form candidate lists, whichever is larger
        const size_t lb = dec_list_layout(rows, nb_max, K).ws_bytes;
        *topk_bytes = lb > *topk_bytes ? lb : *topk_bytes;
    }
}

size_t qsa_select_workspace_bytes(int B, int64_t Tq, int64_t nb_max, int K) {
    if (B <= 0 || Tq <= 0 || nb_max <= 0 || K <= 0) return 0;
    int64_t ld, chunk;
    size_t sb, tb;
    select_layout(B, Tq, nb_max, K, false, &ld, &chunk, &sb, &tb);
    size_t need = sb + tb;
    if (Tq <= kMaxNextN) {  // the decode form may need more
        select_layout(B, Tq, nb_max, K, true, &ld, &chunk, &sb, &tb);
        need = sb + tb > need ? sb + tb : need;
    }
    return need;
}

int qsa_select_blocks(const qsa_bf16 *q_idx, const qsa_bf16 *kbar, int B, int64_t Tq,
                      int64_t pos0, const int64_t *seq_len, int64_t nb_max, int Hi, int Di,
                      int r, int score_mode, int K, int32_t *blk_idx, int32_t *n_sel, void *ws,
                      size_t ws_bytes, const qsa_pages *pages, void *stream) {
    int st = check_index_args(q_idx, kbar, B, Tq, pos0, seq_len, nb_max, Hi, Di, r, score_mode);
    if (st != QSA_OK) return st;
    st = check_pages(pages, nb_max * r);
    if (st != QSA_OK) return st;
    const PageTable pg = block_pages(pages);
    if (!blk_idx || !n_sel) return QSA_ERR_NULL;
    if (K <= 0) return QSA_ERR_SHAPE;
    if (K > kMaxBudget) return QSA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(B) * Tq > kI32Max) return QSA_ERR_OVERFLOW;
    if (nb_max >= (int64_t(1) << 27)) return QSA_ERR_OVERFLOW;  // bounds the score chunk
    if (Tq == 0) return QSA_OK;
    const size_t need = qsa_select_workspace_bytes(B, Tq, nb_max, K);
    if (need > 0 && (!ws || ws_bytes < need)) return QSA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return QSA_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    int64_t ld, chunk;
    size_t sb, tb;
    select_layout(B, Tq, nb_max, K, seq_len != nullptr, &ld, &chunk, &sb, &tb);
    float *sc = static_cast<float *>(ws);
    void *tws = need > 0 ? static_cast<char *>(ws) + sb : nullptr;
    if (seq_len && dec_list_layout(B, nb_max, K).use) {
        // decode form, long rows: the scan also writes the group maxima the
        // top-K filter takes its floor from (start of the top-K workspace)
        const DecListLayout l = dec_list_layout(B, nb_max, K);
        hipError_t e = launch_index_scores(q_idx, kbar, B, Tq, pos0, seq_len, nb_max, score_mode,
                                           sc, ld, s, static_cast<uint32_t *>(tws), l.gld, pg);
        if (e != hipSuccess) return QSA_ERR_LAUNCH;
        return launch_status(launch_topk_dec_lists(sc, B, static_cast<int>(Tq), ld, seq_len,
                                                   nb_max, r, K, blk_idx, n_sel, tws, s));
    }
    if (seq_len || Tq == 1) {
        hipError_t e = launch_index_scores(q_idx, kbar, B, Tq, pos0, seq_len, nb_max, score_mode,
                                           sc, ld, s, nullptr, 0, pg);
        if (e != hipSuccess) return QSA_ERR_LAUNCH;
        return launch_status(launch_topk(sc, B, Tq, ld, pos0, seq_len, nb_max, r, K, blk_idx,
                                         n_sel, tws, s));
    }
    // the chunk's group maxima follow its scores
    const int64_t gld = gmax_ld(ld);
    uint32_t *gm = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) +
                                                round_up(chunk * ld * 4, 256));
    for (int b = 0; b < B; ++b) {
        const qsa_bf16 *qb = q_idx + static_cast<int64_t>(b) * Tq * (kIdxHeads * kIdxDim);
        // one sequence at a time: its own rows of the cache or of the page table
        const qsa_bf16 *kb = pg.table ? kbar : kbar + static_cast<int64_t>(b) * nb_max * kIdxDim;
        const PageTable pgb{pg.table ? pg.table + b * pg.stride : nullptr, pg.stride, pg.shift};
        const int64_t row0 = static_cast<int64_t>(b) * Tq;
        for (int64_t q0 = 0; q0 < Tq; q0 += chunk) {
            const int64_t len = Tq - q0 < chunk ? Tq - q0 : chunk;
            hipError_t e = launch_index_scores(qb + q0 * (kIdxHeads * kIdxDim), kb, 1, len,
                                               pos0 + q0, nullptr, nb_max, score_mode, sc, ld, s,
                                               gm, gld, pgb);
            if (e != hipSuccess) return QSA_ERR_LAUNCH;
            e = launch_topk(sc, 1, len, ld, pos0 + q0, nullptr, nb_max, r, K,
                            blk_idx + (row0 + q0) * K, n_sel + row0 + q0, tws, s, gm, gld);
            if (e != hipSuccess) return QSA_ERR_LAUNCH;
        }
    }
    return QSA_OK;
}

// RoPE arguments of the rotate-on-load entry points: rope_dim 64 or 128
// (the NeoX partners then sit in one lane's query fragment), theta > 0; the
// frequencies exactly as qsa_rope_bf16 forms them.
static int rope_args(int rope_dim, double theta, RopeArgs &ra) {
    ra = RopeArgs{};
    if (rope_dim <= 0 || !(theta > 0.0)) return QSA_ERR_SHAPE;
    if (rope_dim != 64 && rope_dim != 128) return QSA_ERR_UNSUPPORTED;
    ra.half = rope_dim / 2;
    for (int j = 0; j < ra.half; ++j)
        ra.inv_freq[j] = pow(theta, -2.0 * static_cast<double>(j) / static_cast<double>(rope_dim));
    return QSA_OK;
}

static int sparse_prefill(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                          const int32_t *blk_idx, const int32_t *n_sel, int64_t Tq, int64_t Tk,
                          int64_t pos0, int H, int Hkv, int D, int r, int Kbudget,
                          const RopeArgs &ra, float *O, float *lse, const qsa_pages *pages,
                          void *stream) {
    if (!Q || !K || !V || !blk_idx || !n_sel || !O) return QSA_ERR_NULL;
    if (Tq < 0 || Tk < 0 || pos0 < 0 || Kbudget <= 0) return QSA_ERR_SHAPE;
    int st = check_attn_shape(H, Hkv, D, r);
    if (st != QSA_OK) return st;
    if (Tk < pos0 + Tq) return QSA_ERR_SHAPE;
    if (Kbudget > kMaxBudget) return QSA_ERR_UNSUPPORTED;
    if (Tq > kI32Max || Tk / kBlock > kI32Max) return QSA_ERR_OVERFLOW;
    if (Tq * Hkv > kMaxPrefillWaves) return QSA_ERR_OVERFLOW;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return QSA_ERR_ALIGN;
    AttnArgs a{};
    a.Q = Q; a.K = K; a.V = V; a.blk_idx = blk_idx; a.n_sel = n_sel; a.seq_len = nullptr;
    a.O = O; a.lse = lse; a.part = nullptr;
    a.Tq = Tq; a.Lmax = Tk; a.pos0 = pos0; a.B = 1; a.H = H; a.Hkv = Hkv; a.Kbudget = Kbudget;
    st = check_pages(pages, Tk);
    if (st != QSA_OK) return st;
    const PageTable pt = token_pages(pages);
    a.ptable = pt.table; a.pstride = pt.stride; a.pshift = pt.shift;
    return launch_status(launch_sparse_prefill(a, ra, as_stream(stream)));
}

int qsa_sparse_attn_prefill(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                            const int32_t *blk_idx, const int32_t *n_sel, int64_t Tq, int64_t Tk,
                            int64_t pos0, int H, int Hkv, int D, int r, int Kbudget, float *O,
                            float *lse, const qsa_pages *pages, void *stream) {
    RopeArgs none{};
    return sparse_prefill(Q, K, V, blk_idx, n_sel, Tq, Tk, pos0, H, Hkv, D, r, Kbudget, none, O,
                          lse, pages, stream);
}

int qsa_sparse_attn_prefill_rope(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                                 const int32_t *blk_idx, const int32_t *n_sel, int64_t Tq,
                                 int64_t Tk, int64_t pos0, int H, int Hkv, int D, int r,
                                 int Kbudget, int rope_dim, double theta, float *O, float *lse,
                                 const qsa_pages *pages, void *stream) {
    RopeArgs ra;
    const int st = rope_args(rope_dim, theta, ra);
    if (st != QSA_OK) return st;
    return sparse_prefill(Q, K, V, blk_idx, n_sel, Tq, Tk, pos0, H, Hkv, D, r, Kbudget, ra, O, lse,
                          pages, stream);
}

// Split count and workspace bytes of the decode attention: one record per
// (sequence, KV head, column tile of 16 query-head pairs, split).  dense:
// the dense baseline's decode form (sel_entries = every block).
static size_t decode_ws(int B, int Tq, int H, int Hkv, int64_t sel_entries, int *nsplit,
                        bool dense = false) {
    const int nct = decode_col_tiles(Tq, H / Hkv);
    const int ns = decode_num_splits(B, Hkv, nct, decode_max_entries(Tq, sel_entries), dense);
    if (nsplit) *nsplit = ns;
    return decode_partial_floats(B, Hkv * nct, ns) * sizeof(float);
}

size_t qsa_decode_workspace_bytes(int B, int Tq, int H, int Hkv, int D, int Kbudget) {
    (void)D;
    if (B <= 0 || Tq < 1 || Tq > kMaxNextN || H <= 0 || Hkv <= 0 || H % Hkv || Kbudget <= 0)
        return 0;
    return decode_ws(B, Tq, H, Hkv, Kbudget, nullptr);
}

static int sparse_decode(const qsa_bf16 *q, const qsa_bf16 *Kc, const qsa_bf16 *Vc,
                         const int64_t *seq_len, const int32_t *blk_idx, const int32_t *n_sel,
                         int B, int Tq, int64_t Lmax, int H, int Hkv, int D, int r, int Kbudget,
                         const RopeArgs &ra, float *O, float *lse, void *ws, size_t ws_bytes,
                         const qsa_pages *pages, void *stream) {
    if (!q || !Kc || !Vc || !seq_len || !blk_idx || !n_sel || !O) return QSA_ERR_NULL;
    if (B <= 0 || Lmax < 0 || Kbudget <= 0) return QSA_ERR_SHAPE;
    if (Tq < 1 || Tq > kMaxNextN) return QSA_ERR_SHAPE;
    int st = check_attn_shape(H, Hkv, D, r);
    if (st != QSA_OK) return st;
    if (Kbudget > kMaxBudget) return QSA_ERR_UNSUPPORTED;
    if (B > 65535 || Lmax / kBlock > kI32Max) return QSA_ERR_OVERFLOW;
    if (!aligned16(q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(O)) return QSA_ERR_ALIGN;
    int nsplit = 0;
    const size_t need = decode_ws(B, Tq, H, Hkv, Kbudget, &nsplit);
    if (!ws || ws_bytes < need) return QSA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QSA_ERR_ALIGN;
    AttnArgs a{};
    a.Q = q; a.K = Kc; a.V = Vc; a.blk_idx = blk_idx; a.n_sel = n_sel; a.seq_len = seq_len;
    a.O = O; a.lse = lse; a.part = static_cast<float *>(ws);
    a.Tq = Tq; a.Lmax = Lmax; a.pos0 = 0; a.B = B; a.H = H; a.Hkv = Hkv; a.Kbudget = Kbudget;
    st = check_pages(pages, Lmax);
    if (st != QSA_OK) return st;
    const PageTable pt = token_pages(pages);
    a.ptable = pt.table; a.pstride = pt.stride; a.pshift = pt.shift;
    return launch_status(launch_attn_decode(a, ra, nsplit, as_stream(stream)));
}

int qsa_sparse_attn_decode(const qsa_bf16 *q, const qsa_bf16 *Kc, const qsa_bf16 *Vc,
                           const int64_t *seq_len, const int32_t *blk_idx, const int32_t *n_sel,
                           int B, int Tq, int64_t Lmax, int H, int Hkv, int D, int r, int Kbudget,
                           float *O, float *lse, void *ws, size_t ws_bytes,
                           const qsa_pages *pages, void *stream) {
    RopeArgs none{};
    return sparse_decode(q, Kc, Vc, seq_len, blk_idx, n_sel, B, Tq, Lmax, H, Hkv, D, r, Kbudget,
                         none, O, lse, ws, ws_bytes, pages, stream);
}

int qsa_sparse_attn_decode_rope(const qsa_bf16 *q, const qsa_bf16 *Kc, const qsa_bf16 *Vc,
                                const int64_t *seq_len, const int32_t *blk_idx,
                                const int32_t *n_sel, int B, int Tq, int64_t Lmax, int H, int Hkv,
                                int D, int r, int Kbudget, int rope_dim, double theta, float *O,
                                float *lse, void *ws, size_t ws_bytes, const qsa_pages *pages,
                                void *stream) {
    RopeArgs ra;
    const int st = rope_args(rope_dim, theta, ra);
    if (st != QSA_OK) return st;
    return sparse_decode(q, Kc, Vc, seq_len, blk_idx, n_sel, B, Tq, Lmax, H, Hkv, D, r, Kbudget,
                         ra, O, lse, ws, ws_bytes, pages, stream);
}

size_t qsa_decode_noalloc_max_bytes(void) { return kDecodeScratchBytes; }

int qsa_sparse_attn_decode_noalloc(const qsa_bf16 *q, const qsa_bf16 *Kc, const qsa_bf16 *Vc,
                                   const int64_t *seq_len, const int32_t *blk_idx,
                                   const int32_t *n_sel, int B, int Tq, int64_t Lmax, int H,
                                   int Hkv, int D, int r, int Kbudget, float *O, float *lse,
                                   const qsa_pages *pages, void *stream) {
    if (!q || !Kc || !Vc || !seq_len || !blk_idx || !n_sel || !O) return QSA_ERR_NULL;
    if (B <= 0 || Lmax < 0 || Kbudget <= 0) return QSA_ERR_SHAPE;
    if (Tq < 1 || Tq > kMaxNextN) return QSA_ERR_SHAPE;
    int st = check_attn_shape(H, Hkv, D, r);
    if (st != QSA_OK) return st;
    if (Kbudget > kMaxBudget) return QSA_ERR_UNSUPPORTED;
    if (B > 65535 || Lmax / kBlock > kI32Max) return QSA_ERR_OVERFLOW;
    if (!aligned16(q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(O)) return QSA_ERR_ALIGN;
    st = check_pages(pages, Lmax);
    if (st != QSA_OK) return st;
    int nsplit = 0;
    const size_t need = decode_ws(B, Tq, H, Hkv, Kbudget, &nsplit);
    if (need > kDecodeScratchBytes) return QSA_ERR_SCRATCH;
    float *part = nullptr;
    if (decode_scratch(need, &part) != hipSuccess) return QSA_ERR_LAUNCH;
    AttnArgs a{};
    a.Q = q; a.K = Kc; a.V = Vc; a.blk_idx = blk_idx; a.n_sel = n_sel; a.seq_len = seq_len;
    a.O = O; a.lse = lse; a.part = part;
    a.Tq = Tq; a.Lmax = Lmax; a.pos0 = 0; a.B = B; a.H = H; a.Hkv = Hkv; a.Kbudget = Kbudget;
    const PageTable pt = token_pages(pages);
    a.ptable = pt.table; a.pstride = pt.stride; a.pshift = pt.shift;
    RopeArgs none{};
    return launch_status(launch_attn_decode(a, none, nsplit, as_stream(stream)));
}

size_t dense_attn_workspace_bytes(int B, int64_t Tq, int64_t Lmax, int H, int Hkv, int D) {
    (void)D;
    if (B <= 0 || H <= 0 || Hkv <= 0 || H % Hkv || Lmax <= 0) return 0;
    // what the decode form needs (Tq <= 16); the prefill form needs none
    if (Tq < 1 || Tq > kMaxNextN) return 0;
    return decode_ws(B, static_cast<int>(Tq), H, Hkv, Lmax / kBlock, nullptr, true);
}

int dense_attn(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V, int B, int64_t Tq,
               int64_t Lmax, int64_t pos0, const int64_t *seq_len, int H, int Hkv, int D,
               float *O, float *lse, void *ws, size_t ws_bytes, const qsa_pages *pages,
               void *stream) {
    if (!Q || !K || !V || !O) return QSA_ERR_NULL;
    if (B <= 0 || Tq < 0 || Lmax < 0 || pos0 < 0) return QSA_ERR_SHAPE;
    int st = check_attn_shape(H, Hkv, D, kBlock);
    if (st != QSA_OK) return st;
    if (seq_len && (Tq < 1 || Tq > kMaxNextN)) return QSA_ERR_SHAPE;
    if (!seq_len && pos0 + Tq > Lmax) return QSA_ERR_SHAPE;
    if (B > 65535 || Tq > kI32Max || Lmax / kBlock > kI32Max) return QSA_ERR_OVERFLOW;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return QSA_ERR_ALIGN;
    AttnArgs a{};
    a.Q = Q; a.K = K; a.V = V; a.blk_idx = nullptr; a.n_sel = nullptr; a.seq_len = seq_len;
    a.O = O; a.lse = lse; a.part = static_cast<float *>(ws);
    a.Tq = Tq; a.Lmax = Lmax; a.pos0 = pos0; a.B = B; a.H = H; a.Hkv = Hkv; a.Kbudget = 0;
    st = check_pages(pages, Lmax);
    if (st != QSA_OK) return st;
    const PageTable pt = token_pages(pages);
    a.ptable = pt.table; a.pstride = pt.stride; a.pshift = pt.shift;
    hipStream_t s = as_stream(stream);
    if (seq_len) {
        int nsplit = 0;
        const size_t need =
            decode_ws(B, static_cast<int>(Tq), H, Hkv, Lmax / kBlock, &nsplit, true);
        if (!ws || ws_bytes < need) return QSA_ERR_WORKSPACE;
        if (!aligned16(ws)) return QSA_ERR_ALIGN;
        RopeArgs none{};
        return launch_status(launch_attn_decode(a, none, nsplit, s));
    }
    return launch_status(launch_dense_prefill(a, s));
}

// Distillation: the indexer scores of one chunk of query rows live in the
// workspace (at most 8 GiB); the fused kernel reads them back.
static void distill_layout(int64_t Tq, int64_t nb_max, int64_t *ld, int64_t *chunk) {
    *ld = round_up(nb_max > 0 ? nb_max : 1, 4);
    *chunk = select_chunk_rows(Tq, *ld);
}

size_t qsa_distill_workspace_bytes(int64_t Tq, int64_t Tk) {
    if (Tq <= 0 || Tk < kBlock) return 0;
    int64_t ld, chunk;
    distill_layout(Tq, Tk / kBlock, &ld, &chunk);
    return static_cast<size_t>(chunk * ld * 4);
}

int qsa_distill_kl(const qsa_bf16 *Q, const qsa_bf16 *K, const float *lse, const qsa_bf16 *q_idx,
                   const qsa_bf16 *kbar, int64_t Tq, int64_t Tk, int64_t pos0, int H, int Hkv,
                   int D, int Hi, int Di, int r, int score_mode, float *kl, void *ws,
                   size_t ws_bytes, void *stream) {
    if (!Q || !K || !lse || !kl) return QSA_ERR_NULL;
    if (Tq < 0 || Tk < 0 || pos0 < 0 || pos0 + Tq > Tk) return QSA_ERR_SHAPE;
    int st = check_attn_shape(H, Hkv, D, r);
    if (st != QSA_OK) return st;
    if (H != 24 || Hkv != 2) return QSA_ERR_UNSUPPORTED;  // one workgroup: 16 queries x 24 heads
    const int64_t nb_max = Tk / kBlock;
    st = check_index_args(q_idx, kbar, 1, Tq, pos0, nullptr, nb_max, Hi, Di, r, score_mode);
    if (st != QSA_OK) return st;
    if (nb_max >= (int64_t(1) << 27) || Tq > kI32Max) return QSA_ERR_OVERFLOW;
    if (!aligned16(Q) || !aligned16(K)) return QSA_ERR_ALIGN;
    if (Tq == 0) return QSA_OK;
    const size_t need = qsa_distill_workspace_bytes(Tq, Tk);
    if (need > 0 && (!ws || ws_bytes < need)) return QSA_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return QSA_ERR_ALIGN;
    hipStream_t s = as_stream(stream);
    int64_t ld, chunk;
    distill_layout(Tq, nb_max, &ld, &chunk);
    float *sc = static_cast<float *>(ws);
    for (int64_t q0 = 0; q0 < Tq; q0 += chunk) {
        const int64_t len = Tq - q0 < chunk ? Tq - q0 : chunk;
        hipError_t e = launch_index_scores(q_idx + q0 * (kIdxHeads * kIdxDim), kbar, 1, len,
                                           pos0 + q0, nullptr, nb_max, score_mode, sc, ld, s);
        if (e != hipSuccess) return QSA_ERR_LAUNCH;
        e = launch_distill(Q + q0 * H * kHeadDim, lse + q0 * H, K, sc, len, pos0 + q0, Tk, ld,
                           kl + q0, s);
        if (e != hipSuccess) return QSA_ERR_LAUNCH;
    }
    return QSA_OK;
}

int qsa_sparse_attn_prefill_concurrency(int Hkv, int Kbudget, int with_kl, int paged) {
    if ((Hkv != 1 && Hkv != 2 && Hkv != 4) || Kbudget <= 0 || Kbudget > kMaxBudget) return 0;
    if (with_kl && (paged || Hkv != 2 || Kbudget > kMaxKlBudget)) return 0;
    return sparse_prefill_concurrency(Hkv, Kbudget, with_kl != 0, paged != 0);
}

// Checks shared by the two KL forms; fills a on success.
static int kl_prefill_args(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                           const qsa_bf16 *q_idx, const qsa_bf16 *kbar, const int32_t *blk_idx,
                           const int32_t *n_sel, int64_t Tq, int64_t Tk, int64_t pos0, int H,
                           int Hkv, int D, int Hi, int Di, int r, int Kbudget, int max_budget,
                           int score_mode, float *O, float *lse, float *kl, AttnArgs &a) {
    if (!Q || !K || !V || !blk_idx || !n_sel || !O || !kl) return QSA_ERR_NULL;
    if (Tq < 0 || Tk < 0 || pos0 < 0 || Kbudget <= 0) return QSA_ERR_SHAPE;
    int st = check_attn_shape(H, Hkv, D, r);
    if (st != QSA_OK) return st;
    if (Tk < pos0 + Tq) return QSA_ERR_SHAPE;
    if (H != 24 || Hkv != 2 || Kbudget > max_budget) return QSA_ERR_UNSUPPORTED;
    const int64_t nb_max = Tk / kBlock;
    st = check_index_args(q_idx, kbar, 1, Tq, pos0, nullptr, nb_max > 0 ? nb_max : 1, Hi, Di, r,
                          score_mode);
    if (st != QSA_OK) return st;
    if (Tq > kI32Max || nb_max > kI32Max) return QSA_ERR_OVERFLOW;
    if (Tq * Hkv > kMaxPrefillWaves) return QSA_ERR_OVERFLOW;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return QSA_ERR_ALIGN;
    a = AttnArgs{};
    a.Q = Q; a.K = K; a.V = V; a.blk_idx = blk_idx; a.n_sel = n_sel; a.seq_len = nullptr;
    a.O = O; a.lse = lse; a.part = nullptr;
    a.Tq = Tq; a.Lmax = Tk; a.pos0 = pos0; a.B = 1; a.H = H; a.Hkv = Hkv; a.Kbudget = Kbudget;
    a.q_idx = q_idx; a.kbar = kbar; a.kl = kl; a.score_mode = score_mode;
    return QSA_OK;
}

int qsa_sparse_attn_prefill_kl(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                               const qsa_bf16 *q_idx, const qsa_bf16 *kbar,
                               const int32_t *blk_idx, const int32_t *n_sel, int64_t Tq,
                               int64_t Tk, int64_t pos0, int H, int Hkv, int D, int Hi, int Di,
                               int r, int Kbudget, int score_mode, float *O, float *lse,
                               float *kl, void *stream) {
    AttnArgs a;
    const int st = kl_prefill_args(Q, K, V, q_idx, kbar, blk_idx, n_sel, Tq, Tk, pos0, H, Hkv, D,
                                   Hi, Di, r, Kbudget, kMaxKlBudget, score_mode, O, lse, kl, a);
    if (st != QSA_OK) return st;
    return launch_status(launch_sparse_prefill_kl(a, as_stream(stream)));
}

size_t qsa_sparse_attn_prefill_kl_staged_workspace_bytes(int64_t Tq, int Kbudget) {
    if (Tq < 0 || Tq > kI32Max || Kbudget <= 0 || Kbudget > kMaxBudget) return 0;
    return sparse_prefill_kl_staged_floats(Tq, Kbudget) * sizeof(float);
}

int qsa_sparse_attn_prefill_kl_staged(const qsa_bf16 *Q, const qsa_bf16 *K, const qsa_bf16 *V,
                                      const qsa_bf16 *q_idx, const qsa_bf16 *kbar,
                                      const int32_t *blk_idx, const int32_t *n_sel, int64_t Tq,
                                      int64_t Tk, int64_t pos0, int H, int Hkv, int D, int Hi,
                                      int Di, int r, int Kbudget, int score_mode, int rope_dim,
                                      double theta, float *O, float *lse, float *kl, void *ws,
                                      size_t ws_bytes, void *stream) {
    AttnArgs a;
    int st = kl_prefill_args(Q, K, V, q_idx, kbar, blk_idx, n_sel, Tq, Tk, pos0, H, Hkv, D, Hi,
                             Di, r, Kbudget, kMaxBudget, score_mode, O, lse, kl, a);
    if (st != QSA_OK) return st;
    RopeArgs ra{};
    if (rope_dim != 0) {
        st = rope_args(rope_dim, theta, ra);
        if (st != QSA_OK) return st;
    }
    const size_t need = sparse_prefill_kl_staged_floats(Tq, Kbudget) * sizeof(float);
    if (need > 0 && (!ws || ws_bytes < need)) return QSA_ERR_WORKSPACE;
    if (ws && !aligned16(ws)) return QSA_ERR_ALIGN;
    a.bmax = static_cast<float *>(ws);
    a.lse2 = a.bmax + static_cast<size_t>(Tq) * 2 * Kbudget * 12;
    return launch_status(launch_sparse_prefill_kl_staged(a, ra, as_stream(stream)));
}

}  // extern "C"
