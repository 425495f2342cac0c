// A5-A8: softmax attention over 4-token micro-blocks (chlience section 6:
// selected blocks expand to token indices; the query's incomplete block is
// always kept, later tokens masked).  One per-wave routine serves the sparse
// prefill, the split-K decode and the dense decode (every complete block);
// the dense prefill is the flash kernel of flash_prefill.hip.
//
// Work unit: a stage of 4 entries (16 tokens) of one KV head.  An entry is a
// selected block (4 tokens) or the trailing partial block ((p+1) mod 4
// tokens).  Per stage a wave
//   - loads K rows straight into MFMA A fragments (registers), and V rows by
//     LDS DMA (global_load_lds_dwordx4) into an 8 KB tile whose 16-byte
//     chunks are XOR-swizzled per row, so no VGPR holds V in flight;
//   - computes S^T[16 tok, 16 heads] = K . Q^T with v_mfma_f32_16x16x32_bf16;
//   - runs the online softmax per head in fp32 (log2 domain);
//   - accumulates O^T[256, 16] += V^T . P^T with v_mfma_f32_16x16x16_bf16,
//     reading V^T columns from LDS (the transpose the PV product needs), and
//     P split as P_hi + P_lo (two bf16 terms, about 16 significant bits) so V
//     stays exact bf16.
// Up to 16 query heads share one KV head in the MFMA columns (12 here).
//
// MFMA layouts (lane l, n = l%16, g4 = l/16):
//   A[m][k]: lane holds row m = n and the k-slots of group g4
//   B[k][j]: lane holds column j = n and the same k-slots
//   D[m][j]: lane holds rows 4*g4 .. 4*g4+3 of column n
// S^T row 4*e + i is entry e (0..3) token i, so a lane's accumulator holds one
// whole block for one head: exactly the k-slots (tokens 4*g4 .. 4*g4+3) it
// supplies as the B operand P^T of the 16x16x16 PV product.
#include <mutex>

#include "qsa_internal.h"

namespace qsa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kScaleLog2 = 0.09016844005556021f;  // log2(e) / sqrt(256)
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kStageEntries = 4;             // 4 blocks = 16 tokens per stage
constexpr int kVStageBytes = 16 * 512;       // 16 tokens x 256 bf16
constexpr int kRecFloats = 4096 + 128;       // O^T (lane-major) + m + l of one wave
constexpr int kMaxListLds = 2048 + 16;  // budget entries plus the tail (paged lists)

__device__ __forceinline__ void lds_fence() {
    // LDS ops of one wave complete in order; this keeps the compiler from
    // moving LDS accesses across the point and drains outstanding ones.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// Entry e of a query's list: first token and number of tokens.  Entries
// below ns are selected complete blocks; the rest cover the tail, tokens
// 4*nc .. 4*nc + tail - 1 after the selection's visible blocks (the query's
// incomplete block, and for later speculative queries sharing the selection
// also the tokens up to their own positions).
// MULTI: several queries share the list (the tail may span entries and each
// column masks it at its own position); otherwise the tail is one entry of
// (p+1) mod 4 tokens, all visible.
// PMODE: 0 contiguous cache; 1 paged, lst holds the page-pool block of every
// entry (selected blocks and tail); 2 paged without a list (dense): a
// stage's 16 tokens lie in one page (pages hold a power of two of at least
// 16 tokens), whose pool page pg (read from the page table ptab, shift psh)
// the caller sets before the stage.
template <bool MULTI, int PMODE = 0>
struct EntryList {
    const int32_t *lst;  // LDS copy of the selected blocks (sparse), or nullptr (dense)
    int lst_off;         // index of lst[0] in the query's list
    int ns;              // number of complete-block entries
    int tail;            // tail tokens after block nc - 1
    int64_t nc;          // complete blocks visible to the selecting query
    const int32_t *ptab = nullptr;
    int psh = 0;
    int64_t pg = 0;  // PMODE 2: the pool page of the current stage
    __device__ __forceinline__ int count(int e) const {
        if (!MULTI) return e < ns ? 4 : (e == ns ? tail : 0);
        return e < ns ? 4 : max(0, min(4, tail - 4 * (e - ns)));
    }
    __device__ __forceinline__ int64_t base(int e) const {
        if (PMODE == 1) return 4 * static_cast<int64_t>(lst[e - lst_off]);
        int64_t t;
        if (e < ns)
            t = 4 * static_cast<int64_t>(lst ? lst[e - lst_off] : e);
        else
            t = MULTI ? 4 * (nc + e - ns) : 4 * nc;
        return PMODE == 2 ? (pg << psh) | (t & ((int64_t(1) << psh) - 1)) : t;
    }
    // token i of entry e, or the safe row p past the entry's count, with no
    // control flow: the list is read at a clamped index (contiguous
    // single-query lists with an LDS list)
    __device__ __forceinline__ int64_t token_or(int e, int i, int64_t p) const {
        static_assert(!MULTI && PMODE == 0, "contiguous single-query lists only");
        const int64_t b = 4 * static_cast<int64_t>(lst[e < ns ? e : 0]);
        const int64_t t = (e < ns ? b : 4 * nc) + i;
        return i < count(e) ? t : p;
    }
    // tokens of entry e visible to a query at position pq (selected blocks
    // precede every query sharing the selection)
    __device__ __forceinline__ int visible(int e, int64_t pq) const {
        const int c = count(e);
        if (!MULTI || e < ns) return c;
        const int64_t v = pq - 4 * (nc + e - ns) + 1;
        return v < 0 ? 0 : (v < c ? static_cast<int>(v) : c);
    }
};

struct WaveState {
    f32x4 o[16];  // O^T: d-tile dt holds rows d = 16*dt + 4*g4 + i of column (head) n
    float m;      // running max (log2 units) of head n
    float l;      // this lane's share of the weight sum of head n
};

__device__ __forceinline__ void state_init(WaveState &st) {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
}

__device__ __forceinline__ int row_swizzle(int tt) { return 2 * ((tt >> 2) & 3); }

// Stage helpers.  Entries e0 .. e0+3 of one KV head; Kg/Vg point at token 0
// of the head (row stride rs elements); p is a safe row for masked tokens.
// The V tile of a stage is 16 rows of 512 B whose 16-byte chunks sit at
// position c ^ row_swizzle(row): LDS bytes 1024*j + 16*lane hold row
// tt = 2j + lane/32, chunk (lane%32) ^ row_swizzle(tt).

// V rows into the tile by LDS DMA (instruction j fills bytes 1024*j ...).
template <bool MULTI, int PMODE>
__device__ __forceinline__ void stage_v_dma(const EntryList<MULTI, PMODE> &L, int e0, int64_t p,
                                            const uint16_t *__restrict__ Vg, int64_t rs,
                                            unsigned char *vlds, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int tt = 2 * j + h;
        const int e = e0 + (tt >> 2), i = tt & 3;
        const bool ok = i < L.count(e);
        const int64_t tok = ok ? L.base(e) + i : p;
        const int c = (lane & 31) ^ row_swizzle(tt);
        const uint16_t *src = Vg + tok * rs + 8 * c;
        // (C-style casts: the builtin takes explicit global / LDS address spaces)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)(vlds + 1024 * j),
                                         16, 0, 0);
    }
}

// The same 8 chunks of V into registers (written to the tile later), and K
// as stage_k below, both addressed without control flow (token_or), so that
// the loads issue unconditionally and their registers need no merging.
__device__ __forceinline__ void stage_v_regs(const EntryList<false, 0> &L, int e0, int64_t p,
                                             const uint16_t *__restrict__ Vg, int64_t rs,
                                             bf16x8 (&vr)[8], int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int tt = 2 * j + h;
        const int64_t tok = L.token_or(e0 + (tt >> 2), tt & 3, p);
        const int c = (lane & 31) ^ row_swizzle(tt);
        vr[j] = *reinterpret_cast<const bf16x8 *>(Vg + tok * rs + 8 * c);
    }
}

__device__ __forceinline__ void stage_k_regs(const EntryList<false, 0> &L, int e0, int64_t p,
                                             const uint16_t *__restrict__ Kg, int64_t rs,
                                             bf16x8 (&kf)[8], int lane) {
    const int n = lane & 15, g4 = lane >> 4;
    const uint16_t *src = Kg + L.token_or(e0 + (n >> 2), n & 3, p) * rs + 8 * g4;
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = *reinterpret_cast<const bf16x8 *>(src + 32 * s);
}

__device__ __forceinline__ void stage_v_store(const bf16x8 (&vr)[8], unsigned char *vlds,
                                              int lane) {
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<bf16x8 *>(vlds + 1024 * j + 16 * lane) = vr[j];
}

// K: A fragment row m = n is entry e0 + n/4, token n%4; k-slots of group g4
// at step s are dims 32*s + 8*g4 .. +7.
template <bool MULTI, int PMODE>
__device__ __forceinline__ void stage_k(const EntryList<MULTI, PMODE> &L, int e0, int64_t p,
                                        const uint16_t *__restrict__ Kg, int64_t rs,
                                        uint4 (&kf)[8], int lane) {
    const int n = lane & 15, g4 = lane >> 4;
    const int e = e0 + (n >> 2), i = n & 3;
    const bool ok = i < L.count(e);
    const int64_t tok = ok ? L.base(e) + i : p;
    const uint16_t *src = Kg + tok * rs + 8 * g4;
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = *reinterpret_cast<const uint4 *>(src + 32 * s);
}

// Logits, online softmax and the PV product of one stage whose K fragments
// are in kf; pq is the position of the query in this lane's column.  DMA_V:
// the V tile is still arriving by LDS DMA (wait for it before the PV reads);
// otherwise the caller has written it and fenced.  Returns the largest scaled
// logit (log2 units) among the lane's own tokens: entry e0 + g4 for column n
// (-inf where none is visible).  With lmx, lanes with lmo >= 0 also store
// lmv (the previous stage's max) at lmx[lmo].
template <bool DMA_V, bool MULTI, int PMODE>
__device__ __forceinline__ float stage_finish(const EntryList<MULTI, PMODE> &L, int e0,
                                              int64_t pq, f32x4 sacc, WaveState &st,
                                              const unsigned char *vlds, int lane,
                                              float *lmx = nullptr, int lmo = -1,
                                              float lmv = 0.f);

template <bool DMA_V, bool MULTI, int PMODE>
__device__ __forceinline__ float stage_compute(const EntryList<MULTI, PMODE> &L, int e0,
                                               int64_t pq, const bf16x8 (&kf)[8],
                                               const bf16x8 (&qT)[8], WaveState &st,
                                               const unsigned char *vlds, int lane,
                                               float *lmx = nullptr, int lmo = -1,
                                               float lmv = 0.f) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) sacc = mfma_bf16_16x16x32(kf[s], qT[s], sacc);
    return stage_finish<DMA_V>(L, e0, pq, sacc, st, vlds, lane, lmx, lmo, lmv);
}

// The logits S^T (16 tokens x 16 columns) in sacc: masking, online softmax
// and the PV product of the stage.
template <bool DMA_V, bool MULTI, int PMODE>
__device__ __forceinline__ float stage_finish(const EntryList<MULTI, PMODE> &L, int e0,
                                              int64_t pq, f32x4 sacc, WaveState &st,
                                              const unsigned char *vlds, int lane,
                                              float *lmx, int lmo, float lmv) {
    const int n = lane & 15, g4 = lane >> 4;
    // lane (column n, group g4) holds entry e0 + g4, tokens 0..3
    const int cnt = L.visible(e0 + g4, pq);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = i < cnt ? sacc[i] * kScaleLog2 : -INFINITY;
    const float lm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    float cm = fmaxf(lm, __shfl_xor(lm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));
    const float m_new = fmaxf(st.m, cm);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(st.m - m_use);
    s16x4 phi, plo;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float pv = exp2f(sv[i] - m_use);
        const __bf16 hi = static_cast<__bf16>(pv);
        const __bf16 lo = static_cast<__bf16>(pv - static_cast<float>(hi));
        phi[i] = __builtin_bit_cast(short, hi);
        plo[i] = __builtin_bit_cast(short, lo);
        psum += static_cast<float>(hi) + static_cast<float>(lo);
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) st.o[dt] *= alpha;
    if (DMA_V) {
        // V tile has landed (the compiler waits on the DMA before LDS reads)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __builtin_amdgcn_wave_barrier();
    }
    // after the wait: stores count in vmcnt too, so the store of a stage's
    // max waits a stage and leaves with the next one's loads in flight
    if (lmx && lmo >= 0) lmx[lmo] = lmv;
    // O^T += V^T P^T: A = V^T rows d = 16*dt + n, k-slots = tokens 4*g4 .. +3
    const int swz = 2 * g4;  // row_swizzle(4*g4 + jj)
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
        const int d = 16 * dt + n;
        const int off = (((d >> 3) ^ swz) << 4) + ((d & 7) << 1);
        s16x4 a;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            a[jj] = *reinterpret_cast<const short *>(vlds + (4 * g4 + jj) * 512 + off);
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, st.o[dt], 0, 0, 0);
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, st.o[dt], 0, 0, 0);
    }
    return lm;
}

// One stage as a unit: V by LDS DMA into vlds (the wave's 8 KB tile), K into
// registers, then the compute.  Returns stage_compute's block max.
template <bool MULTI, int PMODE>
__device__ __forceinline__ float attn_stage(const EntryList<MULTI, PMODE> &L, int e0, int64_t p,
                                           int64_t pq,
                                           const uint16_t *__restrict__ Kg,
                                           const uint16_t *__restrict__ Vg, int64_t rs,
                                           const bf16x8 (&qT)[8], WaveState &st,
                                           unsigned char *vlds, int lane,
                                           float *lmx = nullptr, int lmo = -1, float lmv = 0.f) {
    lds_fence();  // the previous stage's reads of this tile are done
    stage_v_dma(L, e0, p, Vg, rs, vlds, lane);
    uint4 kf[8];
    stage_k(L, e0, p, Kg, rs, kf, lane);
    bf16x8 kb[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) kb[s] = as_bf16x8(kf[s]);
    return stage_compute<true>(L, e0, pq, kb, qT, st, vlds, lane, lmx, lmo, lmv);
}

// Two bf16 of a 32-bit word each: the pairs (dims j, j+1 of word a) and their
// partners (the same elements of word b).
__device__ __forceinline__ void rope_word(uint32_t &a, uint32_t &b, const double *ang, int j) {
    uint16_t a0, a1, b0, b1;
    rope_pair(static_cast<uint16_t>(a & 0xFFFFu), static_cast<uint16_t>(b & 0xFFFFu), ang[j],
              ang[64 + j], a0, b0);
    rope_pair(static_cast<uint16_t>(a >> 16), static_cast<uint16_t>(b >> 16), ang[j + 1],
              ang[65 + j], a1, b1);
    a = static_cast<uint32_t>(a0) | (static_cast<uint32_t>(a1) << 16);
    b = static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16);
}

// Dims j .. j+7 (fragment a) rotated with their partners (fragment b).
__device__ __forceinline__ void rope_quad(uint4 &a, uint4 &b, const double *ang, int j) {
    rope_word(a.x, b.x, ang, j);
    rope_word(a.y, b.y, ang, j + 2);
    rope_word(a.z, b.z, ang, j + 4);
    rope_word(a.w, b.w, ang, j + 6);
}

// Q^T fragments of column tile ct of KV head g: column n is the pair
// 16*ct + n = (query qi, head h of the group), query rows H * kHeadDim apart;
// columns past ncols pairs are zero.  Lane (n, g4) holds dims 32 s + 8 g4 + k
// (k < 8) in qT[s].  With ang (cosines [0, 64), sines [64, 128) of the
// single query's angles) the first 64 * hs dims are rotated on load: the
// NeoX partner of dim j < 32 hs is j + 32 hs, element k of qT[s + hs], so
// every pair sits in one lane (hs = 1 or 2: rope_dim 64 or 128).
__device__ __forceinline__ bool load_q_raw(const uint16_t *__restrict__ qrow, int g, int group,
                                           int H, int ct, int ncols, int lane, uint4 (&v)[8]) {
    const int n = lane & 15, g4 = lane >> 4;
    const int pair = 16 * ct + n;
    const bool ok = pair < ncols;
    const int qi = ok ? pair / group : 0, h = ok ? pair - qi * group : 0;
    const uint16_t *src =
        qrow + (static_cast<int64_t>(qi) * H + g * group + h) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 8; ++s)
        v[s] = ok ? *reinterpret_cast<const uint4 *>(src + 32 * s + 8 * g4)
                  : make_uint4(0, 0, 0, 0);
    return ok;
}

// Rotates the lane's loaded query dims by the angles ang (cosines [0, 64),
// sines [64, 128) of the lane's query position).
__device__ __forceinline__ void rope_q(uint4 (&v)[8], const double *ang, int hs, int lane) {
    const int g4 = lane >> 4;
    if (hs == 1) {
        rope_quad(v[0], v[1], ang, 8 * g4);
    } else {
        rope_quad(v[0], v[2], ang, 8 * g4);
        rope_quad(v[1], v[3], ang, 32 + 8 * g4);
    }
}

__device__ __forceinline__ void load_qT(const uint16_t *__restrict__ qrow, int g, int group,
                                        int H, int ct, int ncols, int lane, bf16x8 (&qT)[8],
                                        const double *ang = nullptr, int hs = 0) {
    uint4 v[8];
    const bool ok = load_q_raw(qrow, g, group, H, ct, ncols, lane, v);
    if (ang && ok) rope_q(v, ang, hs, lane);
#pragma unroll
    for (int s = 0; s < 8; ++s) qT[s] = as_bf16x8(v[s]);
}

__device__ __forceinline__ void state_store(const WaveState &st, float *buf, int lane) {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) buf[(dt * 4 + i) * 64 + lane] = st.o[dt][i];
    buf[4096 + lane] = st.m;
    buf[4096 + 64 + lane] = st.l;
}

__device__ __forceinline__ void state_merge(WaveState &st, const float *buf, int lane) {
    const float mo = buf[4096 + lane];
    const float lo = buf[4096 + 64 + lane];
    const float m_new = fmaxf(st.m, mo);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float a = exp2f(st.m - m_use), b = exp2f(mo - m_use);
    st.l = st.l * a + lo * b;
    st.m = m_new;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st.o[dt][i] = st.o[dt][i] * a + buf[(dt * 4 + i) * 64 + lane] * b;
}

__device__ __forceinline__ float head_total(float l) {
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    return l;
}

__device__ __forceinline__ void state_write(const WaveState &st, float ltot,
                                            float *__restrict__ orow,
                                            float *__restrict__ lse_row, int g, int group,
                                            int lane) {
    const int n = lane & 15, g4 = lane >> 4;
    if (n >= group) return;
    const int hq = g * group + n;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float *dst = orow + static_cast<int64_t>(hq) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
        float4 v = make_float4(st.o[dt][0] * inv, st.o[dt][1] * inv, st.o[dt][2] * inv,
                               st.o[dt][3] * inv);
        *reinterpret_cast<float4 *>(dst + 16 * dt + 4 * g4) = v;
    }
    if (lse_row && g4 == 0)
        lse_row[hq] = ltot > 0.f ? (st.m + log2f(ltot)) * kLn2 : -INFINITY;
}

// Distillation KL under the sparse pattern, fused into the prefill (ai.info
// "Industry relevance": one kernel yields the sparse outputs and the KL loss
// without storing intermediates; chlience section 6, second stage: indexer and
// backbone train under the sparse pattern).  Teacher: each head's attention
// over the query's token set, max-pooled within each selected block, summed
// over the 24 heads, normalised over the selected blocks; student: softmax of
// the selected blocks' indexer scores; loss KL(teacher || student).
// While the attention runs, a wave keeps the block-max logit of every
// (selected block, head of its group) in LDS (the block max is one lane's
// register-local max, and exp is monotone).  After the pass each head's final
// log-sum-exp turns them into probabilities; the per-block head sums of the
// two waves meet in LDS, and the indexer scores of the selected blocks are
// recomputed from the query's indexer row and the pooled keys.
constexpr int kKlGroup = 12;  // query heads per KV head (24 / 2)

// Dynamic LDS of the prefill kernel, in bytes from the start: Hkv V tiles of
// 8 KB, the block list (Kbudget + 1 entries); for the KL form then the block
// maxima [Hkv][Kbudget][12], the per-wave head sums [Hkv][Kbudget], the
// selected blocks' indexer scores [Kbudget] and 16 floats of reduction space.
struct PrefillLds {
    size_t list, mx, ang, part, score, red, total;
    __host__ __device__ PrefillLds(int Hkv, int Kbudget, bool kl) {
        // the plain forms run one wave per workgroup, the KL form one per KV head
        list = static_cast<size_t>(kl ? Hkv : 1) * kVStageBytes;
        mx = list + ((4 * (static_cast<size_t>(Kbudget) + 1) + 15) & ~size_t(15));
        if (!kl) {
            // the plain forms: the query's RoPE angles (64 cosines, 64 sines)
            ang = mx;
            part = score = red = total = ang + 128 * sizeof(double);
            return;
        }
        ang = mx;
        part = mx + 4 * static_cast<size_t>(Hkv) * kKlGroup * Kbudget;
        score = part + 4 * static_cast<size_t>(Hkv) * Kbudget;
        red = score + 4 * static_cast<size_t>(Kbudget);
        total = red + 4 * 16;
    }
};

// Indexer scores of selected entries, 16 per tile: D[head][entry] =
// q_idx[head] . kbar[block of entry] on 16x16x32 bf16 MFMA, A = the 4 indexer
// heads (rows 4..15 zero), B = the pooled keys of the tile's entries.  Lanes
// of group 0 then hold the 4 heads of entry 16 * tile + n.  Tiles
// t0, t0 + dt, ... below ntile; each lane's 4 key loads of 4 tiles are issued
// before their MFMAs.
__device__ __forceinline__ void tile_scores(const uint16_t *__restrict__ qi_row,
                                            const uint16_t *__restrict__ kbar,
                                            const int32_t *lst, int ns, int t0, int dt, int mode,
                                            float *sc, int lane) {
    const int n = lane & 15, g4 = lane >> 4;
    bf16x8 qa[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
        qa[st] = as_bf16x8(n < kIdxHeads ? *reinterpret_cast<const uint4 *>(
                                               qi_row + n * kIdxDim + 32 * st + 8 * g4)
                                         : make_uint4(0, 0, 0, 0));
    const int ntile = (ns + 15) / 16;
    for (int t = t0; t < ntile; t += 4 * dt) {
        uint4 kb[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = min(16 * (t + u * dt) + n, ns - 1);
            const uint16_t *src = kbar + static_cast<int64_t>(lst[e]) * kIdxDim + 8 * g4;
#pragma unroll
            for (int st = 0; st < 4; ++st) kb[u][st] = *reinterpret_cast<const uint4 *>(src + 32 * st);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                acc = mfma_bf16_16x16x32(qa[st], as_bf16x8(kb[u][st]), acc);
            const int e = 16 * (t + u * dt) + n;
            if (g4 == 0 && e < ns) sc[e] = mode == 0 ? combine_heads<0>(acc) : combine_heads<1>(acc);
        }
    }
}

// KL of one query (row of the launch) from the block-max logits of its
// selected blocks, in a workgroup of two waves, wave g holding KV head g:
// mxg = wave g's maxima [ns][12] (LDS or device memory), lse2 = this lane's
// head's log2-unit log-sum-exp (lanes 0..11 hold heads g*12 .. g*12+11).
// part [2][Kbudget], sc [Kbudget] and red [16] are the workgroup's LDS.
__device__ __forceinline__ void kl_epilogue(const AttnArgs &a, int64_t row, int ns,
                                            const int32_t *lst, const float *mxg, float lse2,
                                            float *part, float *sc, float *red, int g, int lane) {
    // teacher mass of each selected block from this wave's 12 heads: the
    // head's probability of the block's best token, exp2(max - lse2)
    float l2[kKlGroup];
#pragma unroll
    for (int h = 0; h < kKlGroup; ++h) l2[h] = __shfl(lse2, h);
    lds_fence();  // the wave's block maxima are in place
    for (int e = lane; e < ns; e += kWave) {
        const float *mr = mxg + e * kKlGroup;
        float tb = 0.f;
#pragma unroll
        for (int h = 0; h < kKlGroup; ++h) tb += exp2f(mr[h] - l2[h]);
        part[g * a.Kbudget + e] = tb;
    }
    // student logits: wave g scores tiles g, g + 2, ...
    tile_scores(a.q_idx + row * (kIdxHeads * kIdxDim), a.kbar, lst, ns, g, 2, a.score_mode, sc,
                lane);
    block_sync();
    // thread i takes blocks i, i + 128, ...: t = both waves' sums; the row's
    // Z = sum t, A = sum t ln t, C = sum t s and the log-sum-exp of s
    float z = 0.f, aa = 0.f, c = 0.f, m = -INFINITY, zs = 0.f;
    for (int e = threadIdx.x; e < ns; e += 2 * kWave) {
        const float tb = part[e] + part[a.Kbudget + e];
        const float se = sc[e];
        z += tb;
        aa += tb > 0.f ? tb * logf(tb) : 0.f;
        c += tb * se;
        if (se > m) {
            zs = zs * expf(m - se) + 1.f;
            m = se;
        } else {
            zs += expf(se - m);
        }
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        z += __shfl_xor(z, off);
        aa += __shfl_xor(aa, off);
        c += __shfl_xor(c, off);
        const float m2 = __shfl_xor(m, off), zs2 = __shfl_xor(zs, off);
        const float mn = fmaxf(m, m2);
        zs = (m == -INFINITY ? 0.f : zs * expf(m - mn)) +
             (m2 == -INFINITY ? 0.f : zs2 * expf(m2 - mn));
        m = mn;
    }
    if (lane == 0) {
        red[5 * g + 0] = z;
        red[5 * g + 1] = aa;
        red[5 * g + 2] = c;
        red[5 * g + 3] = m;
        red[5 * g + 4] = zs;
    }
    block_sync();
    if (threadIdx.x != 0) return;
    // wave 1 after wave 0
    const float m1 = red[8], mn = fmaxf(red[3], m1);
    const float zsum = (red[3] == -INFINITY ? 0.f : red[4] * expf(red[3] - mn)) +
                       (m1 == -INFINITY ? 0.f : red[9] * expf(m1 - mn));
    const float zt = red[0] + red[5], at = red[1] + red[6], ct = red[2] + red[7];
    a.kl[row] = ns > 0 ? at / zt - logf(zt) - ct / zt + (mn + logf(zsum)) : 0.f;
}

// ------------------------------------------------------------------------
// Prefill: one wave per (query, KV head), walking all stages of its head.
// Plain forms: one wave per workgroup, workgroup w = Hkv * query + head, grid
// (Tq * Hkv, B), block 64.  Workgroups are dealt to the 8 XCDs in turn, so
// with Hkv | 8 each XCD serves one KV head only and its L2 holds that head's
// rows alone: the gathers of one head by the queries running together hit
// in L2 about twice as often as when every XCD fetches both heads (a
// loads-only probe of the 128K workload: 41 against 49 ms per step).
// KL form: one workgroup per query, one wave per KV head (the waves share the
// query's block masses), grid (Tq, B), block 64 * Hkv.
// Dynamic LDS: PrefillLds.
// PAGED: K and V are page pools; the list is translated to pool blocks once
// (the tail block as entry ns).
// KL: also the distillation KL of each query (above); contiguous caches, one
// sequence, 2 KV heads of 12 query heads.
// Registers: at most those of 3 waves per SIMD for the plain forms (168: the
// O accumulators then live in VGPRs instead of AGPRs, and 12 waves per CU
// keep 1.5x the stages in flight: 13% faster than 2 waves per SIMD); the KL
// form is held to 2 workgroups per CU by its LDS anyway.
template <bool PAGED, bool KL, bool BMAX>
__global__ void __launch_bounds__(256, KL ? 1 : 3) attn_prefill_kernel(AttnArgs a, RopeArgs ra) {
    static_assert(!(PAGED && KL) && !(BMAX && (PAGED || KL)),
                  "the KL forms run on contiguous caches");
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    const PrefillLds lay(a.Hkv, a.Kbudget, KL);
    int32_t *lst = reinterpret_cast<int32_t *>(dyn_lds + lay.list);
    const int64_t t = KL ? blockIdx.x : blockIdx.x / a.Hkv, b = blockIdx.y;
    const int64_t row = b * a.Tq + t;
    int64_t p = a.pos0 + t;
    const int64_t nc = num_complete_blocks(p, kBlock);
    const int v = a.n_sel[row];
    const int64_t cap = min(static_cast<int64_t>(a.Kbudget), nc);
    const int ns = v < 0 ? 0 : (v > cap ? static_cast<int>(cap) : v);
    const int32_t *src = a.blk_idx + row * a.Kbudget;
    const int32_t *ptab = PAGED ? a.ptable + b * a.pstride : nullptr;
    for (int i = threadIdx.x; i < ns; i += blockDim.x) {
        int32_t bi = src[i];
        bi = bi < 0 ? 0 : (bi >= nc ? static_cast<int32_t>(nc - 1) : bi);
        lst[i] = PAGED ? static_cast<int32_t>(page_row(ptab, a.pshift, 4 * int64_t(bi)) >> 2) : bi;
    }
    const int tail = static_cast<int>((p + 1) % kBlock);
    if (PAGED && threadIdx.x == 0 && tail > 0)
        lst[ns] = static_cast<int32_t>(page_row(ptab, a.pshift, 4 * nc) >> 2);
    double *ang = KL ? nullptr : reinterpret_cast<double *>(dyn_lds + lay.ang);
    if (!KL && static_cast<int>(threadIdx.x) < ra.half)
        rope_angle(p < 0 ? 0 : p, ra.inv_freq[threadIdx.x], ang[threadIdx.x], ang[64 + threadIdx.x]);
    block_sync();
    EntryList<false, PAGED ? 1 : 0> L{lst, 0, ns, tail, nc};
    if (PAGED) p = page_row(ptab, a.pshift, p);  // the safe row for masked tokens
    const int E = ns + (L.tail > 0 ? 1 : 0);
    const int nstages = (E + kStageEntries - 1) / kStageEntries;

    const int lane = threadIdx.x & 63;
    const int g = KL ? static_cast<int>(threadIdx.x >> 6) : static_cast<int>(blockIdx.x - t * a.Hkv);
    const int group = a.H / a.Hkv;
    bf16x8 qT[8];
    load_qT(a.Q + row * a.H * kHeadDim, g, group, a.H, 0, group, lane, qT,
            ra.half > 0 ? ang : nullptr, ra.half / 32);
    const int64_t rs = static_cast<int64_t>(a.Hkv) * kHeadDim;
    const int64_t seq_off = PAGED ? 0 : b * a.Lmax * rs;
    const uint16_t *Kg = a.K + seq_off + g * kHeadDim;
    const uint16_t *Vg = a.V + seq_off + g * kHeadDim;
    const int64_t pq = a.pos0 + t;  // every entry is visible (single query)
    WaveState st;
    state_init(st);
    const int n = lane & 15, g4 = lane >> 4;
    float *mxw = reinterpret_cast<float *>(dyn_lds + lay.mx) +
                 static_cast<int64_t>(g) * a.Kbudget * kKlGroup;
    unsigned char *vl = dyn_lds + (KL ? g : 0) * kVStageBytes;
    if constexpr (!KL) {
        // staged KL form: each selected block's max logit per head of the wave
        float *bmx =
            BMAX ? a.bmax + (row * a.Hkv + g) * static_cast<int64_t>(a.Kbudget) * kKlGroup
                 : nullptr;
        // each stage stores the previous stage's maxima
        float lmv = 0.f;
        int lmo = -1;
        for (int sidx = 0; sidx < nstages; ++sidx) {
            const int e0 = sidx * kStageEntries;
            const float lm = attn_stage(L, e0, p, pq, Kg, Vg, rs, qT, st, vl, lane, bmx, lmo, lmv);
            // this stage's slot: entry e0 + g4, head n (none past the list)
            lmo = BMAX && n < kKlGroup && e0 + g4 < ns ? (e0 + g4) * kKlGroup + n : -1;
            lmv = lm;
        }
        if (BMAX && lmo >= 0) bmx[lmo] = lmv;
    } else {
        // Two stages per step: the first stage's V by LDS DMA as above, its
        // K and the second stage's K and V into registers, all issued before
        // the first wait.  The LDS of the block maxima leaves one wave per
        // SIMD, so each wave keeps two stages' bytes in flight.  Loads past
        // the last stage read the safe row p.
        for (int sidx = 0; sidx < nstages; sidx += 2) {
            const int e0 = sidx * kStageEntries, e1 = e0 + kStageEntries;
            lds_fence();  // the previous stage's reads of the tile are done
            stage_v_dma(L, e0, p, Vg, rs, vl, lane);
            bf16x8 ka[8], kb[8], vb[8];
            stage_k_regs(L, e0, p, Kg, rs, ka, lane);
            stage_k_regs(L, e1, p, Kg, rs, kb, lane);
            stage_v_regs(L, e1, p, Vg, rs, vb, lane);
            float lm = stage_compute<true>(L, e0, pq, ka, qT, st, vl, lane);
            if (n < kKlGroup && e0 + g4 < ns) mxw[(e0 + g4) * kKlGroup + n] = lm;
            if (sidx + 1 < nstages) {
                lds_fence();
                stage_v_store(vb, vl, lane);
                lds_fence();
                lm = stage_compute<false>(L, e1, pq, kb, qT, st, vl, lane);
                if (n < kKlGroup && e1 + g4 < ns) mxw[(e1 + g4) * kKlGroup + n] = lm;
            }
        }
    }
    const float ltot = head_total(st.l);
    state_write(st, ltot, a.O + row * a.H * kHeadDim, a.lse ? a.lse + row * a.H : nullptr, g,
                group, lane);
    if (!KL) {
        if (BMAX && g4 == 0 && n < group)
            a.lse2[row * a.H + g * group + n] = ltot > 0.f ? st.m + log2f(ltot) : INFINITY;
        return;
    }

    const float lse2 = ltot > 0.f ? st.m + log2f(ltot) : INFINITY;
    kl_epilogue(a, row, ns, lst, mxw, lse2, reinterpret_cast<float *>(dyn_lds + lay.part),
                reinterpret_cast<float *>(dyn_lds + lay.score),
                reinterpret_cast<float *>(dyn_lds + lay.red), g, lane);
}

// Split record in HBM: unnormalised O of head n (column n of O^T) at
// [n * 256 + d], then the max of head n at [4096 + n] and its weight sum at
// [4160 + n].  Lanes (n, g4) write float4 runs, 64 bytes per head.
__device__ __forceinline__ void record_store(const WaveState &st, float *rec, int lane) {
    const int n = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
        *reinterpret_cast<float4 *>(rec + n * kHeadDim + 16 * dt + 4 * g4) =
            make_float4(st.o[dt][0], st.o[dt][1], st.o[dt][2], st.o[dt][3]);
    if (g4 == 0) {
        rec[4096 + n] = st.m;
        rec[4096 + 64 + n] = st.l;
    }
}

// ------------------------------------------------------------------------
// Decode: workgroup (4 waves) per (split, column tile, KV head, sequence);
// waves take the split's stages round-robin, merge through LDS, and wave 0
// writes the split's record (unnormalised O^T, max, weight sum) to the
// workspace.  The Tq newest queries of a sequence share its selection (made
// for the first of them, at seq_len - Tq); the columns of a tile are 16
// (query, head) pairs and each column masks the tail past its own query.
// Grid x enumerates (split, column tile) so that the column tiles of one
// split have workgroup ids 8 apart: workgroups go to the 8 XCDs in turn, so
// those tiles run on one XCD back to back and its L2 serves their repeated
// reads of the split's keys and values (one HBM read per split, not one
// per column tile).
template <bool DENSE, bool MULTI, bool PAGED>
__global__ void __launch_bounds__(256) attn_decode_kernel(AttnArgs a, RopeArgs ra, int nsplit,
                                                          int sps, int nct) {
    constexpr int PMODE = PAGED ? (DENSE ? 2 : 1) : 0;
    __shared__ __attribute__((aligned(16))) unsigned char lds[3 * kRecFloats * 4];
    // the value tiles of the 4 waves, then (rotation on load) the angles of
    // up to 16 query positions, 128 doubles each
    static_assert(4 * kVStageBytes + 16 * 128 * 8 <= 3 * kRecFloats * 4, "decode LDS");
    __shared__ int32_t lst[DENSE ? 1 : kMaxListLds];
    const int bx = blockIdx.x, grp = bx / (8 * nct), rem = bx - grp * 8 * nct;
    const int ct = rem >> 3, split = 8 * grp + (rem & 7);
    if (split >= nsplit) return;  // the grid rounds the splits up to 8
    const int g = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int nq = static_cast<int>(a.Tq);
    // the split's first list entries do not depend on the lengths: they are
    // requested together with the length and the selection count
    const int e_lo = split * sps * kStageEntries;
    int32_t pre = 0;
    if (!DENSE && e_lo + static_cast<int>(threadIdx.x) < a.Kbudget)
        pre = a.blk_idx[b * a.Kbudget + e_lo + threadIdx.x];
    int64_t Lb = a.seq_len[b];
    Lb = Lb < 0 ? 0 : (Lb > a.Lmax ? a.Lmax : Lb);
    const int64_t p_last = Lb - 1;
    const int64_t p0 = Lb - nq;  // the selecting query
    const int64_t nc = num_complete_blocks(p0, kBlock);
    int ns;
    if (DENSE) {
        ns = static_cast<int>(nc);
    } else {
        const int v = a.n_sel[b];
        const int64_t cap = min(static_cast<int64_t>(a.Kbudget), nc);
        ns = v < 0 ? 0 : (v > cap ? static_cast<int>(cap) : v);
    }
    const int tail = p_last >= 4 * nc ? static_cast<int>(p_last - 4 * nc + 1) : 0;
    const int E = ns + (tail + 3) / 4;
    const int nstages = (E + kStageEntries - 1) / kStageEntries;
    const int s0 = split * sps, s1 = min(s0 + sps, nstages);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int group = a.H / a.Hkv;
    // the query rows are read while the block list arrives (and, with
    // ra.half > 0, rotated once the angles of their positions are formed)
    uint4 qv[8];
    const bool qok = load_q_raw(a.Q + b * nq * a.H * kHeadDim, g, group, a.H, ct, nq * group,
                                lane, qv);
    const int32_t *ptab = PAGED ? a.ptable + b * a.pstride : nullptr;
    if (!DENSE) {
        // paged: pool blocks of the split's entries, tail entries included
        const int e_hi = min(s1 * kStageEntries, PAGED ? E : ns);
        const int32_t *src = a.blk_idx + b * a.Kbudget;
        for (int i = e_lo + static_cast<int>(threadIdx.x); i < e_hi; i += 256) {
            int64_t bi = i < ns ? (i < e_lo + 256 ? pre : src[i]) : nc + (i - ns);
            if (i < ns) bi = bi < 0 ? 0 : (bi >= nc ? nc - 1 : bi);
            lst[i - e_lo] =
                static_cast<int32_t>(PAGED ? page_row(ptab, a.pshift, 4 * bi) >> 2 : bi);
        }
    }
    // angles of the tile's query positions q_lo .. q_hi (the positions the
    // RoPE kernel gives decode rows: seq_len - Tq + query, at least 0)
    double *ang = reinterpret_cast<double *>(lds + 4 * kVStageBytes);
    const int q_lo = 16 * ct / group;
    if (ra.half > 0) {
        const int q_hi = min(nq - 1, (16 * ct + 15) / group);
        const int cnt = (q_hi - q_lo + 1) * ra.half;
        for (int i = static_cast<int>(threadIdx.x); i < cnt; i += 256) {
            const int qq = i / ra.half, j = i - qq * ra.half;
            const int64_t pp = a.seq_len[b] - nq + q_lo + qq;
            rope_angle(pp < 0 ? 0 : pp, ra.inv_freq[j], ang[qq * 128 + j],
                       ang[qq * 128 + 64 + j]);
        }
    }
    EntryList<MULTI, PMODE> L{DENSE ? nullptr : lst, e_lo, ns, tail, nc, ptab, a.pshift};
    block_sync();

    // position of this lane's column query (-1: no query, every token masked)
    const int pair = 16 * ct + (lane & 15);
    if (ra.half > 0 && qok) rope_q(qv, ang + (pair / group - q_lo) * 128, ra.half / 32, lane);
    bf16x8 qT[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) qT[s] = as_bf16x8(qv[s]);
    const int64_t pq = pair < nq * group ? p0 + pair / group : -1;
    const int64_t rs = static_cast<int64_t>(a.Hkv) * kHeadDim;
    const int64_t seq_off = PAGED ? 0 : b * a.Lmax * rs;
    const uint16_t *Kg = a.K + seq_off + g * kHeadDim;
    const uint16_t *Vg = a.V + seq_off + g * kHeadDim;
    unsigned char *vlds = lds + wave * kVStageBytes;
    // a row that exists for masked tokens
    int64_t psafe = p_last < 0 ? 0 : p_last;
    if (PAGED && E > 0) psafe = page_row(ptab, a.pshift, psafe);
    WaveState st;
    state_init(st);
    if constexpr (PMODE == 2) {
        // the pool page of the wave's next stage is read a stage ahead
        auto page_of = [&](int sidx) {
            return static_cast<int64_t>(ptab[(16 * static_cast<int64_t>(sidx)) >> a.pshift]);
        };
        int64_t pg_next = s0 + wave < s1 ? page_of(s0 + wave) : 0;
        for (int sidx = s0 + wave; sidx < s1; sidx += 4) {
            L.pg = pg_next;
            if (sidx + 4 < s1) pg_next = page_of(sidx + 4);
            attn_stage(L, sidx * kStageEntries, psafe, pq, Kg, Vg, rs, qT, st, vlds, lane);
        }
    } else {
        for (int sidx = s0 + wave; sidx < s1; sidx += 4)
            attn_stage(L, sidx * kStageEntries, psafe, pq, Kg, Vg, rs, qT, st, vlds, lane);
    }
    block_sync();
    float *mbuf = reinterpret_cast<float *>(lds);
    if (wave != 0) state_store(st, mbuf + (wave - 1) * kRecFloats, lane);
    block_sync();
    if (wave == 0) {
        for (int w = 0; w < 3; ++w) state_merge(st, mbuf + w * kRecFloats, lane);
        st.l = head_total(st.l);
        const int64_t rec_id = ((b * a.Hkv + g) * nct + ct) * nsplit + split;
        record_store(st, a.part + rec_id * static_cast<int64_t>(kRecFloats), lane);
    }
}

// ------------------------------------------------------------------------
// Dense decode of several column tiles (the baseline's speculative queries:
// next_n query rows of 12 heads each make 3 tiles at next_n = 4): one
// workgroup per (split, group of up to 4 column tiles, KV head, sequence)
// whose waves are the tiles of the group.  The waves walk the split's
// stages together: a stage's 16 key rows and 16 value rows are read from
// memory once for all tiles (by LDS DMA, the instructions shared among the
// waves, into one of two buffers, so the next stage arrives while this one
// is computed), and every wave multiplies them with its own tile's queries.
// Each wave writes its tile's split record as the one-tile kernel does, so
// the same merge follows.  LDS: the key tile (row tt, chunk c at slot c ^ tt:
// the 16 rows of one fragment read fall in distinct banks) and the value
// tile (slot c ^ row_swizzle(tt), the layout stage_finish reads); before the
// stage loop the first buffer holds the queries' RoPE angles.  (For the
// sparse decode, whose splits hold a few stages each, the one-tile kernel
// with its stages spread over 4 waves was faster: 89.5-90.0 against 91.0 us
// per 4 x 1M step at next_n = 4.)
constexpr int kTileMaxWaves = 4;

template <bool PAGED, int W>
__global__ void __launch_bounds__(64 * W) attn_decode_tiles_kernel(AttnArgs a, RopeArgs ra,
                                                                   int nsplit, int sps, int nct) {
    constexpr int PMODE = PAGED ? 2 : 0;
    constexpr int nthr = 64 * W;  // the waves of the group
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kVStageBytes];
    __shared__ __attribute__((aligned(16))) unsigned char lds2[2 * kVStageBytes];
    static_assert(16 * 128 * 8 <= 2 * kVStageBytes, "angles of 16 query positions");
    const int bx = blockIdx.x, cg = bx / nsplit, split = bx - cg * nsplit;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ct = kTileMaxWaves * cg + wave;
    const int g = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int nq = static_cast<int>(a.Tq);
    int64_t Lb = a.seq_len[b];
    Lb = Lb < 0 ? 0 : (Lb > a.Lmax ? a.Lmax : Lb);
    const int64_t p_last = Lb - 1;
    const int64_t p0 = Lb - nq;  // the first query
    const int64_t nc = num_complete_blocks(p0, kBlock);
    const int ns = static_cast<int>(nc);
    const int tail = p_last >= 4 * nc ? static_cast<int>(p_last - 4 * nc + 1) : 0;
    const int E = ns + (tail + 3) / 4;
    const int nstages = (E + kStageEntries - 1) / kStageEntries;
    const int s0 = split * sps, s1 = min(s0 + sps, nstages);
    const int group = a.H / a.Hkv;
    uint4 qv[8];
    const bool qok = load_q_raw(a.Q + b * nq * a.H * kHeadDim, g, group, a.H, ct, nq * group,
                                lane, qv);
    const int32_t *ptab = PAGED ? a.ptable + b * a.pstride : nullptr;
    // angles of the group's query positions q_lo .. q_hi (at most 16)
    double *ang = reinterpret_cast<double *>(lds);
    const int q_lo = 16 * kTileMaxWaves * cg / group;
    if (ra.half > 0) {
        const int q_hi = min(nq - 1, (16 * (kTileMaxWaves * cg + W) - 1) / group);
        const int cnt = (q_hi - q_lo + 1) * ra.half;
        for (int i = static_cast<int>(threadIdx.x); i < cnt; i += nthr) {
            const int qq = i / ra.half, j = i - qq * ra.half;
            const int64_t pp = a.seq_len[b] - nq + q_lo + qq;
            rope_angle(pp < 0 ? 0 : pp, ra.inv_freq[j], ang[qq * 128 + j],
                       ang[qq * 128 + 64 + j]);
        }
    }
    EntryList<true, PMODE> L{nullptr, 0, ns, tail, nc, ptab, a.pshift};
    block_sync();
    const int pair = 16 * ct + (lane & 15);
    if (ra.half > 0 && qok) rope_q(qv, ang + (pair / group - q_lo) * 128, ra.half / 32, lane);
    bf16x8 qT[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) qT[s] = as_bf16x8(qv[s]);
    const int64_t pq = pair < nq * group ? p0 + pair / group : -1;
    const int64_t rs = static_cast<int64_t>(a.Hkv) * kHeadDim;
    const int64_t seq_off = PAGED ? 0 : b * a.Lmax * rs;
    const uint16_t *Kg = a.K + seq_off + g * kHeadDim;
    const uint16_t *Vg = a.V + seq_off + g * kHeadDim;
    int64_t psafe = p_last < 0 ? 0 : p_last;
    if (PAGED && E > 0) psafe = page_row(ptab, a.pshift, psafe);
    WaveState st;
    state_init(st);
    // A stage's tiles by LDS DMA: 16 instructions of 1 KB, wave w issuing
    // w, w + W, ...; instruction d fills bytes 1024 d .. (keys for d < 8,
    // values after), lane l row tt = 2 (d % 8) + l / 32 at slot l % 32, which
    // holds chunk (l % 32) ^ tt (keys) or (l % 32) ^ row_swizzle(tt) (values).
    // Two buffers: the next stage's rows arrive while this one is computed.
    // Token 16 sidx + tt is visible up to p_last; paged, a stage's 16 tokens
    // lie in one page (pages hold a power of two of at least 16 tokens), and
    // its pool page is read a stage ahead.
    const int64_t pmask = PAGED ? (int64_t(1) << a.pshift) - 1 : 0;
    auto page_of = [&](int sidx) -> int64_t {
        return PAGED ? static_cast<int64_t>(ptab[(16 * static_cast<int64_t>(sidx)) >> a.pshift])
                     : 0;
    };
    auto issue = [&](int sidx, int64_t pg, unsigned char *buf) {
        for (int d = wave; d < 16; d += W) {
            const int tt = 2 * (d & 7) + (lane >> 5);
            const int64_t t = 16 * static_cast<int64_t>(sidx) + tt;
            const int64_t tok = t > p_last ? psafe : (PAGED ? (pg << a.pshift) | (t & pmask) : t);
            const bool val = d >= 8;
            const int c = (lane & 31) ^ (val ? row_swizzle(tt) : tt);
            const uint16_t *src = (val ? Vg : Kg) + tok * rs + 8 * c;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)src,
                (__attribute__((address_space(3))) void *)(buf + 1024 * d), 16, 0, 0);
        }
    };
    auto compute = [&](int sidx, const unsigned char *buf) {
        if (ct >= nct) return;
        // S^T = K Q^T with the key fragments read from the tile step by step
        const int n = lane & 15, g4 = lane >> 4;
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s)
            sacc = mfma_bf16_16x16x32(
                *reinterpret_cast<const bf16x8 *>(buf + n * 512 + 16 * ((4 * s + g4) ^ n)), qT[s],
                sacc);
        stage_finish<false>(L, sidx * kStageEntries, pq, sacc, st, buf + kVStageBytes, lane);
    };
    const int nst = s1 > s0 ? s1 - s0 : 0;
    block_sync();  // the angles are read
    int64_t pg = nst > 0 ? page_of(s0) : 0;
    int64_t pg_next = nst > 1 ? page_of(s0 + 1) : 0;
    if (nst > 0) issue(s0, pg, lds);
    for (int k = 0; k < nst; k += 2) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's rows of stage k have landed
        block_sync();  // every wave's, and every wave is done with the other buffer
        if (k + 1 < nst) {
            pg = pg_next;
            issue(s0 + k + 1, pg, lds2);
            if (k + 2 < nst) pg_next = page_of(s0 + k + 2);
        }
        compute(s0 + k, lds);
        if (k + 1 >= nst) break;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        block_sync();
        if (k + 2 < nst) {
            pg = pg_next;
            issue(s0 + k + 2, pg, lds);
            if (k + 3 < nst) pg_next = page_of(s0 + k + 3);
        }
        compute(s0 + k + 1, lds2);
    }
    if (ct < nct) {
        st.l = head_total(st.l);
        const int64_t rec_id = ((b * a.Hkv + g) * nct + ct) * nsplit + split;
        record_store(st, a.part + rec_id * static_cast<int64_t>(kRecFloats), lane);
    }
}

// Merge the split records: SUB neighbouring threads per 4 consecutive
// dimensions of an output row (b, query, head), thread k folding splits k,
// k + SUB, ... in order with an online rescale (the loads of 4 splits issued
// before their folds), then the SUB partial states combined by shuffles in a
// fixed order.  SUB = 4 when the splits are many (few output rows, e.g.
// 4 sequences over 33 splits), else 1.  Neighbouring threads read
// neighbouring 16-byte words of a record.
__device__ __forceinline__ void merge_step(float &M, float4 &acc, float &l, float m2,
                                           const float4 &acc2, float l2) {
    const float mn = fmaxf(M, m2);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float a1 = exp2f(M - mu), a2 = exp2f(m2 - mu);
    acc.x = acc.x * a1 + acc2.x * a2;
    acc.y = acc.y * a1 + acc2.y * a2;
    acc.z = acc.z * a1 + acc2.z * a2;
    acc.w = acc.w * a1 + acc2.w * a2;
    l = l * a1 + l2 * a2;
    M = mn;
}

constexpr int kMergeLanes = kHeadDim / 4;  // 4-dimension groups per output row
constexpr int kMergeSubMin = 16;           // splits from which SUB = 4

template <int SUB>
__global__ void __launch_bounds__(256) attn_decode_merge(AttnArgs a, int nsplit, int nct) {
    const int group = a.H / a.Hkv;
    const int64_t total = static_cast<int64_t>(a.B) * a.Tq * a.H * kMergeLanes;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int sub = static_cast<int>(tid % SUB);
    int64_t idx = tid / SUB;
    const bool valid = idx < total;  // the SUB threads of an element agree
    idx = valid ? idx : total - 1;
    const int d4 = static_cast<int>(idx % kMergeLanes);
    const int64_t row = idx / kMergeLanes;  // (b * Tq + qi) * H + hq
    const int hq = static_cast<int>(row % a.H);
    const int64_t bq = row / a.H;
    const int64_t b = bq / a.Tq;
    const int qi = static_cast<int>(bq - b * a.Tq);
    const int g = hq / group, pair = qi * group + (hq - g * group);
    const int ct = pair >> 4, n = pair & 15;
    const float *rec =
        a.part + ((b * a.Hkv + g) * nct + ct) * nsplit * static_cast<int64_t>(kRecFloats);
    float M = -INFINITY, l = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = sub;
    for (; s + 3 * SUB < nsplit; s += 4 * SUB) {
        float m2[4], l2[4];
        float4 a2[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float *r = rec + (s + k * SUB) * static_cast<int64_t>(kRecFloats);
            m2[k] = r[4096 + n];
            l2[k] = r[4096 + 64 + n];
            a2[k] = *reinterpret_cast<const float4 *>(r + n * kHeadDim + 4 * d4);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) merge_step(M, acc, l, m2[k], a2[k], l2[k]);
    }
    for (; s < nsplit; s += SUB) {
        const float *r = rec + s * static_cast<int64_t>(kRecFloats);
        const float4 a2 = *reinterpret_cast<const float4 *>(r + n * kHeadDim + 4 * d4);
        merge_step(M, acc, l, r[4096 + n], a2, r[4096 + 64 + n]);
    }
#pragma unroll
    for (int off = 1; off < SUB; off <<= 1) {
        float4 o2;
        o2.x = __shfl_xor(acc.x, off);
        o2.y = __shfl_xor(acc.y, off);
        o2.z = __shfl_xor(acc.z, off);
        o2.w = __shfl_xor(acc.w, off);
        merge_step(M, acc, l, __shfl_xor(M, off), o2, __shfl_xor(l, off));
    }
    if (sub != 0 || !valid) return;
    float4 o;
    o.x = l > 0.f ? acc.x / l : 0.f;
    o.y = l > 0.f ? acc.y / l : 0.f;
    o.z = l > 0.f ? acc.z / l : 0.f;
    o.w = l > 0.f ? acc.w / l : 0.f;
    *reinterpret_cast<float4 *>(a.O + row * kHeadDim + 4 * d4) = o;
    if (a.lse && d4 == 0) a.lse[row] = l > 0.f ? (M + log2f(l)) * kLn2 : -INFINITY;
}

hipError_t launch_sparse_prefill(const AttnArgs &a, const RopeArgs &ra, hipStream_t s) {
    if (a.Tq == 0 || a.B == 0) return hipSuccess;
    if (ra.half != 0 && ra.half != 32 && ra.half != 64) return hipErrorInvalidValue;
    if (a.Tq * a.Hkv > kMaxPrefillWaves) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<uint32_t>(a.Tq * a.Hkv), static_cast<uint32_t>(a.B));
    const size_t lds = PrefillLds(a.Hkv, a.Kbudget, false).total;
    if (a.ptable)
        hipLaunchKernelGGL((attn_prefill_kernel<true, false, false>), grid, dim3(kWave), lds, s,
                           a, ra);
    else
        hipLaunchKernelGGL((attn_prefill_kernel<false, false, false>), grid, dim3(kWave), lds, s,
                           a, ra);
    return hipGetLastError();
}

size_t sparse_prefill_kl_lds(int Kbudget) { return PrefillLds(2, Kbudget, true).total; }

int sparse_prefill_concurrency(int Hkv, int Kbudget, bool kl, bool paged) {
    const size_t lds = PrefillLds(Hkv, Kbudget, kl).total;
    const void *fn =
        kl      ? reinterpret_cast<const void *>(&attn_prefill_kernel<false, true, false>)
        : paged ? reinterpret_cast<const void *>(&attn_prefill_kernel<true, false, false>)
                : reinterpret_cast<const void *>(&attn_prefill_kernel<false, false, false>);
    if (kl && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  static_cast<int>(lds)) != hipSuccess)
        return 0;
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kl ? 64 * Hkv : kWave, lds) !=
        hipSuccess)
        return 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    // queries: the plain forms run Hkv workgroups per query
    return kl ? per_cu * cus : per_cu * cus / Hkv;
}

hipError_t launch_sparse_prefill_kl(const AttnArgs &a, hipStream_t s) {
    if (a.Tq == 0 || a.B == 0) return hipSuccess;
    const dim3 grid(static_cast<uint32_t>(a.Tq), static_cast<uint32_t>(a.B));
    const size_t lds = PrefillLds(a.Hkv, a.Kbudget, true).total;
    const void *fn = reinterpret_cast<const void *>(&attn_prefill_kernel<false, true, false>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    RopeArgs none{};
    hipLaunchKernelGGL((attn_prefill_kernel<false, true, false>), grid, dim3(64 * a.Hkv), lds, s,
                       a, none);
    return hipGetLastError();
}

// Second kernel of the staged KL form: one workgroup of two waves per query
// (wave g: KV head g), the block list and the KL epilogue over the block
// maxima and log-sum-exps the attention wrote to device memory.  Dynamic
// LDS: the list (Kbudget + 1 entries), part [2][Kbudget], the scores
// [Kbudget] and 16 floats.
__global__ void __launch_bounds__(128) kl_from_bmax_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    const size_t list_bytes = (4 * (static_cast<size_t>(a.Kbudget) + 1) + 15) & ~size_t(15);
    int32_t *lst = reinterpret_cast<int32_t *>(dyn_lds);
    float *part = reinterpret_cast<float *>(dyn_lds + list_bytes);
    float *sc = part + 2 * a.Kbudget;
    float *red = sc + a.Kbudget;
    const int64_t row = blockIdx.x;
    const int64_t p = a.pos0 + row;
    const int64_t nc = num_complete_blocks(p, kBlock);
    const int v = a.n_sel[row];
    const int64_t cap = min(static_cast<int64_t>(a.Kbudget), nc);
    const int ns = v < 0 ? 0 : (v > cap ? static_cast<int>(cap) : v);
    const int32_t *src = a.blk_idx + row * a.Kbudget;
    for (int i = threadIdx.x; i < ns; i += blockDim.x) {
        int32_t bi = src[i];
        lst[i] = bi < 0 ? 0 : (bi >= nc ? static_cast<int32_t>(nc - 1) : bi);
    }
    block_sync();
    const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
    const float lse2 = (lane & 15) < kKlGroup ? a.lse2[row * a.H + g * kKlGroup + (lane & 15)] : 0.f;
    const float *mxg = a.bmax + (row * 2 + g) * static_cast<int64_t>(a.Kbudget) * kKlGroup;
    kl_epilogue(a, row, ns, lst, mxg, lse2, part, sc, red, g, lane);
}

size_t sparse_prefill_kl_staged_floats(int64_t Tq, int Kbudget) {
    // block maxima [Tq][2][Kbudget][12], then lse2 [Tq][24]
    return static_cast<size_t>(Tq) * (2 * static_cast<size_t>(Kbudget) * kKlGroup + 2 * kKlGroup);
}

hipError_t launch_sparse_prefill_kl_staged(const AttnArgs &a, const RopeArgs &ra,
                                           hipStream_t s) {
    if (a.Tq == 0 || a.B == 0) return hipSuccess;
    if (ra.half != 0 && ra.half != 32 && ra.half != 64) return hipErrorInvalidValue;
    if (a.B != 1 || a.Hkv != 2 || a.H != 2 * kKlGroup || a.ptable || !a.bmax || !a.lse2)
        return hipErrorInvalidValue;
    if (a.Tq * a.Hkv > kMaxPrefillWaves) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<uint32_t>(a.Tq * a.Hkv));
    hipLaunchKernelGGL((attn_prefill_kernel<false, false, true>), grid, dim3(kWave),
                       PrefillLds(a.Hkv, a.Kbudget, false).total, s, a, ra);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = ((4 * (static_cast<size_t>(a.Kbudget) + 1) + 15) & ~size_t(15)) +
                       4 * 3 * static_cast<size_t>(a.Kbudget) + 4 * 16;
    hipLaunchKernelGGL(kl_from_bmax_kernel, dim3(static_cast<uint32_t>(a.Tq)), dim3(2 * kWave),
                       lds, s, a);
    return hipGetLastError();
}

int decode_col_tiles(int Tq, int group) { return (Tq * group + 15) / 16; }

// Entries of the longest list: the selection (or every complete block) plus
// the tail (at most 3 + Tq tokens).
int64_t decode_max_entries(int Tq, int64_t sel_entries) { return sel_entries + (Tq + 6) / 4; }

bool decode_uses_tiles(int nct, bool dense) { return dense && nct >= 2; }

int decode_num_splits(int B, int Hkv, int nct, int64_t max_entries, bool dense) {
    const int64_t nstages = (max_entries + kStageEntries - 1) / kStageEntries;
    if (decode_uses_tiles(nct, dense)) {
        // the tiles kernel: workgroups of min(nct, 4) waves, every wave
        // through all stages of its split; as many workgroups as fit at
        // once (2 waves per SIMD: 8 waves per CU, 256 CUs), no empty split
        const int w = nct < kTileMaxWaves ? nct : kTileMaxWaves;
        const int64_t ncg = (nct + kTileMaxWaves - 1) / kTileMaxWaves;
        int64_t want = (256 * (8 / w)) / (static_cast<int64_t>(B) * Hkv * ncg);
        if (want < 1) want = 1;
        if (nstages <= 0) return 1;
        const int64_t per = (nstages + want - 1) / want;
        return static_cast<int>((nstages + per - 1) / per);
    }
    Hkv *= nct;
    // at most 512 workgroups (the two per CU that fit at once: one more and a
    // second round of workgroups doubles the time).  The grid rounds the
    // splits up to a multiple of 8 (the XCD mapping), so from 8 on the count
    // is a multiple of 8 itself: 21 splits of 24 column tiles would launch
    // 576 workgroups, 16 launch 384 (next_n = 4 at 4 x 1M: 38.9 against
    // 28.5 us for attention and merge).  At least two stages per wave, which
    // caps short lists (4 x 1M: 17 splits, 0.081 ms per step; at one stage
    // per wave 33 splits, 0.081-0.083 ms; at four 9 splits, 0.0875 ms).
    int64_t want = 512 / (static_cast<int64_t>(B) * Hkv);
    if (want >= 8) want -= want % 8;
    const int64_t cap = (nstages + 7) / 8;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    return static_cast<int>(want);
}

size_t decode_partial_floats(int B, int Hkv, int nsplit) {
    return static_cast<size_t>(B) * Hkv * nsplit * kRecFloats;
}

template <bool DENSE, bool MULTI>
static void launch_decode_paging(const AttnArgs &a, const RopeArgs &ra, dim3 grid, int nsplit,
                                 int sps, int nct, bool paged, hipStream_t s) {
    if (paged)
        hipLaunchKernelGGL((attn_decode_kernel<DENSE, MULTI, true>), grid, dim3(256), 0, s, a,
                           ra, nsplit, sps, nct);
    else
        hipLaunchKernelGGL((attn_decode_kernel<DENSE, MULTI, false>), grid, dim3(256), 0, s, a,
                           ra, nsplit, sps, nct);
}

static void launch_decode_variant(const AttnArgs &a, const RopeArgs &ra, dim3 grid, int nsplit,
                                  int sps, int nct, bool dense, bool multi, bool paged,
                                  hipStream_t s) {
    if (dense) {
        if (multi)
            launch_decode_paging<true, true>(a, ra, grid, nsplit, sps, nct, paged, s);
        else
            launch_decode_paging<true, false>(a, ra, grid, nsplit, sps, nct, paged, s);
    } else {
        if (multi)
            launch_decode_paging<false, true>(a, ra, grid, nsplit, sps, nct, paged, s);
        else
            launch_decode_paging<false, false>(a, ra, grid, nsplit, sps, nct, paged, s);
    }
}

// Scratch of the no-allocation decode entry point: the split records of one
// call, in a file-scope device array (each GPU the library runs on holds its
// own copy until the process ends).  Host code never passes the array's
// name to a kernel: its device address comes from hipGetSymbolAddress, once
// per device, with that device current.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];
}  // namespace

hipError_t decode_scratch(size_t need, float **ptr) {
    *ptr = nullptr;
    if (need > kDecodeScratchBytes) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = p;
    }
    *ptr = static_cast<float *>(scratch_ptr[dev]);
    return hipSuccess;
}

template <int W>
static void launch_tiles(const AttnArgs &a, const RopeArgs &ra, dim3 grid, int nsplit, int sps,
                         int nct, bool paged, hipStream_t s) {
    const dim3 block(kWave * W);
    if (paged)
        hipLaunchKernelGGL((attn_decode_tiles_kernel<true, W>), grid, block, 0, s, a, ra, nsplit,
                           sps, nct);
    else
        hipLaunchKernelGGL((attn_decode_tiles_kernel<false, W>), grid, block, 0, s, a, ra, nsplit,
                           sps, nct);
}

hipError_t launch_attn_decode(const AttnArgs &a, const RopeArgs &ra, int nsplit, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    const int nq = static_cast<int>(a.Tq);
    const int nct = decode_col_tiles(nq, a.H / a.Hkv);
    const int64_t max_entries =
        decode_max_entries(nq, a.blk_idx ? static_cast<int64_t>(a.Kbudget) : a.Lmax / kBlock);
    const int64_t nstages = (max_entries + kStageEntries - 1) / kStageEntries;
    const int sps = static_cast<int>((nstages + nsplit - 1) / nsplit);
    const bool dense = a.blk_idx == nullptr, paged = a.ptable != nullptr;
    if (decode_uses_tiles(nct, dense)) {
        const int w = nct < kTileMaxWaves ? nct : kTileMaxWaves;
        const int ncg = (nct + kTileMaxWaves - 1) / kTileMaxWaves;
        const dim3 grid(static_cast<uint32_t>(nsplit * ncg), static_cast<uint32_t>(a.Hkv),
                        static_cast<uint32_t>(a.B));
        if (w == 2)
            launch_tiles<2>(a, ra, grid, nsplit, sps, nct, paged, s);
        else if (w == 3)
            launch_tiles<3>(a, ra, grid, nsplit, sps, nct, paged, s);
        else
            launch_tiles<4>(a, ra, grid, nsplit, sps, nct, paged, s);
    } else {
        const dim3 grid(static_cast<uint32_t>((nsplit + 7) / 8 * 8 * nct),
                        static_cast<uint32_t>(a.Hkv), static_cast<uint32_t>(a.B));
        launch_decode_variant(a, ra, grid, nsplit, sps, nct, dense, nq > 1, paged, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows4 = static_cast<int64_t>(a.B) * nq * a.H * kMergeLanes;
    if (nsplit >= kMergeSubMin)
        hipLaunchKernelGGL(attn_decode_merge<4>,
                           dim3(static_cast<uint32_t>((4 * rows4 + 255) / 256)), dim3(256), 0, s,
                           a, nsplit, nct);
    else
        hipLaunchKernelGGL(attn_decode_merge<1>, dim3(static_cast<uint32_t>((rows4 + 255) / 256)),
                           dim3(256), 0, s, a, nsplit, nct);
    return hipGetLastError();
}

}  // namespace qsa
