// Internal declarations shared by the HIP translation units of libqsa.
// Launchers are called by qsa_api.cpp after host-side argument checks; they
// only enqueue kernels and return the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// ---------------------------------------------------------------- types --
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
// waves of one prefill attention launch (Tq * Hkv): a dispatch holds fewer
// than 2^32 threads
constexpr int64_t kMaxPrefillWaves = (int64_t(1) << 26) - 1;

// Tuned shapes.
constexpr int kHeadDim = 256;   // attention head dim
constexpr int kIdxHeads = 4;    // indexer query heads
constexpr int kIdxDim = 128;    // indexer head dim
constexpr int kBlock = 4;       // micro-block size r

// ------------------------------------------------------- device helpers --
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round a finite double to bf16 (nearest, ties to even) by integer
// manipulation of its bits.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
    uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    uint32_t sign = static_cast<uint32_t>(u >> 63) << 15;
    int e = static_cast<int>((u >> 52) & 0x7FF) - 1023;
    if (x == 0.0) return static_cast<uint16_t>(sign);
    if (e < -126) {
        // bf16 subnormal range: quantum 2^-133
        double n = rint(fabs(x) * 0x1p133);
        return static_cast<uint16_t>(sign | static_cast<uint32_t>(n));
    }
    uint64_t mant = u & ((1ull << 52) - 1);
    uint32_t top = (static_cast<uint32_t>(e + 127) << 7) | static_cast<uint32_t>(mant >> 45);
    uint64_t rem = mant & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    if (rem > half || (rem == half && (top & 1u))) top += 1;
    return static_cast<uint16_t>(sign | top);
}

// Partial RoPE of one NeoX pair (a at dim j, b at dim j + rope_dim / 2)
// with the angle's cosine c and sine s: fp64 products, no contraction, one
// RNE rounding per output.  Every kernel that rotates uses this, so their
// results agree bit for bit.
__device__ __forceinline__ void rope_pair(uint16_t a_bits, uint16_t b_bits, double c, double s,
                                          uint16_t &o0, uint16_t &o1) {
#pragma clang fp contract(off)
    const double a = static_cast<double>(bf16_bits_to_f32(a_bits));
    const double b = static_cast<double>(bf16_bits_to_f32(b_bits));
    const double ac = a * c, bs = b * s, bc = b * c, as = a * s;
    o0 = f64_to_bf16_rne(ac - bs);
    o1 = f64_to_bf16_rne(bc + as);
}

// Angle of dim pair j at position p: the cosine and sine of p * inv_freq[j]
// in fp64.
__device__ __forceinline__ void rope_angle(int64_t p, double inv_freq, double &c, double &s) {
#pragma clang fp contract(off)
    const double ang = static_cast<double>(p) * inv_freq;
    sincos(ang, &s, &c);
}

// Partial RoPE applied to the queries on load (sparse prefill and decode):
// half = the rotated pairs per head (0: none), inv_freq[j] =
// theta^(-2j / rope_dim) formed on the host as for the RoPE kernel.
struct RopeArgs {
    int half;
    double inv_freq[64];
};

// Complete blocks visible to a query at position p: floor((p+1)/r).
__host__ __device__ __forceinline__ int64_t num_complete_blocks(int64_t p, int r) {
    return p < 0 ? 0 : (p + 1) / r;
}

// Order-preserving map of a finite fp32 to uint32 (larger float -> larger
// key); -0.0 maps to the key of +0.0 so that equal values compare equal.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup barrier that publishes LDS data: the wave's own LDS operations
// are waited for (lgkmcnt(0)) before s_barrier.  The compiler's barrier can
// omit that wait, e.g. for LDS stores at the end of a loop body followed by
// the barrier at the top of the next iteration; other waves could then read
// rows still being written, which was observed when other kernels' LDS DMA
// loaded the CU.
__device__ __forceinline__ void block_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __syncthreads();
}

// Indexer head combination of one query's four head dot products (held by one
// lane as rows 4*g4 .. 4*g4+3 of a 16x16 MFMA tile).  MODE 0: max over heads
// scaled by 1/sqrt(128); MODE 1: sum of ReLUs.  Shared by every kernel that
// scores blocks, so their scores agree bit for bit.
template <int MODE>
__device__ __forceinline__ float combine_heads(f32x4 acc) {
    if (MODE == 0) {
        const float m = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
        return m * 0.08838834764831845f;
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += acc[i] > 0.f ? acc[i] : 0.f;
    return s;
}

// Page table of paged caches: row i of sequence b lives at row
// (table[b * stride + (i >> shift)] << shift) + i mod 2^shift of the pool.
// Rows are tokens (K/V, shift = log2 of the page's tokens) or pooled blocks
// (kbar, shift = log2 of the page's blocks).  table == nullptr: contiguous
// per-sequence caches.
struct PageTable {
    const int32_t *table;
    int64_t stride;
    int shift;
};

// ------------------------------------------------------------ launchers --
// Decode form (seq_len given): T = B * nq rows, row t at position
// seq_len[t / nq] - nq + t % nq.
hipError_t launch_rope(const uint16_t *x, uint16_t *y, int64_t T, int nheads, int head_dim,
                       int rope_dim, const double *inv_freq, int64_t pos0,
                       const int64_t *seq_len, int nq, hipStream_t s);

// gain: RMSNorm gain (mode 1) or nullptr; rope_dim > 0 (a power of two)
// rotates the pooled keys at positions r * (block0 + block) with inv_freq.
// pg.table set: kbar is a page pool of pooled blocks; block block0 + j of
// sequence b goes to its page row.
hipError_t launch_compress(const uint16_t *k, int B, int64_t Tk, int64_t k_seq_stride, int Di,
                           int r, int mode, const uint16_t *gain, int rope_dim,
                           const double *inv_freq, int64_t block0, uint16_t *kbar,
                           int64_t kbar_seq_stride, hipStream_t s,
                           PageTable pg = PageTable{nullptr, 0, 0});

// Decode form (seq_len given): when gmax is set, also writes the largest
// score key of every group of 64 consecutive blocks, gmax[b * gld + g] for
// the groups holding complete blocks.  Prefill form: groups of 16 blocks,
// gmax[t * gld + g] for every 64-block tile a query's row covers (gld a
// multiple of 4).
// pg.table set: kbar is a page pool of pooled blocks (pg.shift = log2 of the
// blocks per page); only blocks a query sees are read.
hipError_t launch_index_scores(const uint16_t *q_idx, const uint16_t *kbar, int B, int64_t Tq,
                               int64_t pos0, const int64_t *seq_len, int64_t nb_max, int mode,
                               float *scores, int64_t ld, hipStream_t s,
                               uint32_t *gmax = nullptr, int64_t gld = 0,
                               PageTable pg = PageTable{nullptr, 0, 0});

// Top-K passes for rows of up to nmax candidates: either one streaming pass
// per row, or npass reduction passes (segment lengths seg[i], entries[i]
// candidates per row after pass i) then one final pass.  ws_bytes of
// workspace hold the candidate lists.
struct TopkPlan {
    bool stream;    // one streaming pass per row, no workspace
    int stream_nt;  // its workgroup size
    int npass;
    int64_t seg[4];
    int64_t entries[4];
    int64_t final_entries;
    int64_t ld[2];
    size_t ws_bytes;
};
TopkPlan topk_plan(int64_t rows, int64_t nmax, int K);

// Decode form (seq_len given): B rows, row b made for position
// seq_len[b] - Tq (the first of the sequence's Tq newest queries).
// gmax (prefill form, optional): the 16-block group maxima of the score rows
// (launch_index_scores); the streaming plan then takes its floor from them
// and reads only the groups at or above it.
hipError_t launch_topk(const float *scores, int B, int64_t Tq, int64_t ld, int64_t pos0,
                       const int64_t *seq_len, int64_t nb_max, int r, int K, int32_t *blk_idx,
                       int32_t *n_sel, void *ws, hipStream_t s,
                       const uint32_t *gmax = nullptr, int64_t gld = 0);

// Decode-form top-K for few long rows (one query per sequence): a filter
// pass over 4,096-key segments against a floor from the scan's group maxima,
// then one exact pass per row over the candidates.  Workspace: the group
// maxima [rows][gld] (written by the scan), then the candidate keys and
// indices [rows][lld] and the per-segment counts [rows][cld].
struct DecListLayout {
    bool use;  // false: the general plan applies
    int64_t gld, lld, cld;
    size_t ws_bytes;
};
DecListLayout dec_list_layout(int64_t rows, int64_t nb_max, int K);
hipError_t launch_topk_dec_lists(const float *scores, int B, int nq, int64_t ld,
                                 const int64_t *seq_len, int64_t nb_max, int r, int K,
                                 int32_t *blk_idx, int32_t *n_sel, void *ws, hipStream_t s);

// Sparse / dense attention over 4-token blocks (see attention.hip).
struct AttnArgs {
    const uint16_t *Q;       // [B][Tq][H][D]
    const uint16_t *K;       // [B][Lmax][Hkv][D]
    const uint16_t *V;
    const int32_t *blk_idx;  // prefill [Tq][Kbudget], decode [B][Kbudget] (one selection
                             // per sequence), or nullptr (dense: every complete block)
    const int32_t *n_sel;    // [Tq] / [B] or nullptr
    const int64_t *seq_len;  // decode form: [B], the Tq queries of sequence b at
                             // seq_len[b] - Tq .. seq_len[b] - 1; prefill form: nullptr
    float *O;                // [B][Tq][H][D]
    float *lse;              // [B][Tq][H] or nullptr
    float *part;             // split partials (decode), or nullptr
    int64_t Tq, Lmax, pos0;
    int B, H, Hkv, Kbudget;
    // Paged caches (ptable set): K, V are page pools [pages * 2^pshift][Hkv][D]
    // and token t of sequence b is row (ptable[b * pstride + (t >> pshift)]
    // << pshift) + t mod 2^pshift.
    const int32_t *ptable;
    int64_t pstride;
    int pshift;
    // Fused distillation KL (prefill, contiguous): the chunk's indexer queries
    // [Tq][4][128], the pooled keys [nb][128], the score mode and kl [Tq].
    const uint16_t *q_idx;
    const uint16_t *kbar;
    float *kl;
    int score_mode;
    // Staged KL form: the plain prefill kernel also writes each selected
    // block's max logit per head, bmax [Tq][Hkv][Kbudget][H / Hkv] (log2
    // units), and each head's log2-unit log-sum-exp, lse2 [Tq][H]; a second
    // kernel turns them into the KL.  nullptr otherwise.
    float *bmax;
    float *lse2;
};

// Row of token t in a page pool (tab: the sequence's page-table row).
__device__ __forceinline__ int64_t page_row(const int32_t *tab, int sh, int64_t t) {
    return (static_cast<int64_t>(tab[t >> sh]) << sh) | (t & ((int64_t(1) << sh) - 1));
}

// ra.half = 0: Q as given; 32 or 64: Q rotated on load (partial RoPE over
// 2 * ra.half dims at positions pos0 + t).
hipError_t launch_sparse_prefill(const AttnArgs &a, const RopeArgs &ra, hipStream_t s);
// Sparse prefill plus the distillation KL of every query (H = 24, Hkv = 2);
// dynamic LDS bytes it takes at a budget.
hipError_t launch_sparse_prefill_kl(const AttnArgs &a, hipStream_t s);
// Staged KL form: the plain prefill kernel writing a.bmax and a.lse2, then
// the KL epilogue kernel (contiguous caches, Hkv = 2, H = 24).
hipError_t launch_sparse_prefill_kl_staged(const AttnArgs &a, const RopeArgs &ra, hipStream_t s);
// floats of its workspace: bmax [Tq][2][Kbudget][12], then lse2 [Tq][24]
size_t sparse_prefill_kl_staged_floats(int64_t Tq, int Kbudget);
size_t sparse_prefill_kl_lds(int Kbudget);
// Workgroups (one per query) of the sparse prefill (kl: fused with the KL;
// paged: over page pools) resident at once on the current device: its
// resident workgroups per CU times the CUs; 0 when the runtime cannot say.
int sparse_prefill_concurrency(int Hkv, int Kbudget, bool kl, bool paged);
// Decode: split-K workgroups per (split, KV head, column tile, sequence); a
// column tile holds 16 (query, head) pairs of one KV head.
int decode_col_tiles(int Tq, int group);
int64_t decode_max_entries(int Tq, int64_t Kbudget_or_blocks);
size_t decode_partial_floats(int B, int Hkv, int nsplit);
// dense: the dense baseline (every block), which with several column tiles
// runs the tiles kernel (each stage read once for all tiles)
bool decode_uses_tiles(int nct, bool dense);
int decode_num_splits(int B, int Hkv, int nct, int64_t max_entries, bool dense);
// ra.half > 0: the queries are rotated as they are loaded (angles at the
// decode positions seq_len - Tq + query).
hipError_t launch_attn_decode(const AttnArgs &a, const RopeArgs &ra, int nsplit, hipStream_t s);
// The no-allocation decode: its split records live in a static device array
// of kDecodeScratchBytes per GPU.  decode_scratch gives the array's address
// on the current device (looked up once per device), or an error when need
// exceeds the array.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t decode_scratch(size_t need, float **ptr);
hipError_t launch_dense_prefill(const AttnArgs &a, hipStream_t s);

// Stage-1 distillation KL of a chunk of rows (see distill.hip): Q [rows][24][256]
// and lse [rows][24] of the chunk, K [Tk][2][256], scores [rows][ld]; kl: [rows].
hipError_t launch_distill(const uint16_t *Q, const float *lse, const uint16_t *K,
                          const float *scores, int64_t rows, int64_t pos0, int64_t Tk,
                          int64_t ld, float *kl, hipStream_t s);

}  // namespace qsa
