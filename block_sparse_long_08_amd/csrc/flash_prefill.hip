// A8 baseline: dense causal attention, prefill form (the reference point of
// the QSA speedup; same softmax attention as chlience section 6 but over every
// earlier token).  A flash-attention forward pass on MFMA:
//
// Workgroup: 128 queries of one head, 4 waves x 32 queries; KV tiles of 32
// tokens stream through LDS, double-buffered, one barrier per tile: the next
// tile is loaded into registers while the current one is consumed, then
// written to the other LDS buffer.
//   S^T[32 tok, 32 q] = K . Q^T   v_mfma_f32_32x32x16_bf16, K and Q both from
//                                   LDS (16-byte chunks XOR-swizzled by row);
//   online softmax per query column in fp32 (log2 domain) with lazy
//   rescaling: the running reference max moves only when a tile's max
//   exceeds it by more than 2^8, so P <= 256 and O, l are rarely rescaled;
//   O^T[256, 32 q] += V^T . P^T   v_mfma_f32_32x32x16_f16: the S^T accumulator
//                                   of a lane is exactly the P^T fragment it
//                                   supplies (fp16, P <= 256), V^T read from a
//                                   transposed fp16 LDS tile (bf16 -> fp16 is
//                                   exact for |v| in the fp16 normal range).
// MFMA 32x32x16 layouts (lane l, n = l%32, h = l/32):
//   A[m][k]: row m = n, k-slots 8h .. 8h+7;  B[k][j]: column j = n, same slots;
//   D[m][j]: column j = n, rows 8*(r/4) + 4h + r%4 for r = 0..15.
// The S^T rows a lane holds for one 16-token step are tokens 4h..4h+3 and
// 8+4h..8+4h+3; the V^T tile stores each 16-token group in that order
// (slots 8h..8h+7), so every MFMA operand read is one 16-byte LDS read.
#include "qsa_internal.h"

namespace qsa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kFaQ = 128;                // queries per workgroup
constexpr int kFaN = 32;                 // tokens per KV tile
constexpr int kFaKRow = 512;             // K tile row (256 bf16), 16-byte chunks swizzled
constexpr int kFaKTile = kFaN * kFaKRow; // 16 KB
constexpr int kFaVRow = 80;              // V^T tile row: 32 token slots + 16 B pad
constexpr int kFaVTile = 256 * kFaVRow;  // 20 KB
constexpr int kFaQTile = kFaQ * 512;     // 64 KB: the workgroup's queries, chunks swizzled
constexpr int kFaLds = kFaQTile + 2 * kFaKTile + 2 * kFaVTile;
constexpr float kFaScaleLog2 = 0.09016844005556021f;  // log2(e) / sqrt(256)
constexpr float kFaLn2 = 0.6931471805599453f;
constexpr float kFaSlack = 8.f;          // lazy-rescale threshold (log2 units)

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// fp16 pair (a in the low half) of two bf16 values; exact for magnitudes in
// the fp16 normal range, where truncation and nearest rounding agree.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t lo_bits, uint32_t hi_bits) {
    const auto v = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(lo_bits << 16),
                                              __uint_as_float(hi_bits << 16));
    return __builtin_bit_cast(uint32_t, v);
}

// Slot of token t (0..31) in a V^T row: inside each 16-token group, tokens
// 4h+i go to slot 8h+i and tokens 8+4h+i to slot 8h+4+i.
__device__ __forceinline__ int vslot(int t) {
    const int t16 = t & 15;
    return (t & ~15) | (t16 & 3) | (((t16 >> 3) & 1) << 2) | (((t16 >> 2) & 1) << 3);
}

struct FaArgs {
    const uint16_t *Q;  // [B][Tq][H][256]
    const uint16_t *K;  // [B][Lmax][Hkv][256]
    const uint16_t *V;
    float *O;           // [B][Tq][H][256]
    float *lse;         // [B][Tq][H] or nullptr
    int64_t Tq, Lmax, pos0;
    int H, Hkv;
    const int32_t *ptable;  // paged K/V: page table [B][pstride], or nullptr
    int64_t pstride;
    int pshift;
};

// Row of token tok in K/V: the sequence's own rows, or a page-pool row.
template <bool PAGED>
__device__ __forceinline__ int64_t fa_row(const int32_t *ptab, int psh, int64_t tok) {
    return PAGED ? page_row(ptab, psh, tok) : tok;
}

// K tile into registers: thread t takes row t/8 (token) and the chunks
// (16 B each) c = t%8 + 8u, u = 0..3, of that row.
template <bool PAGED>
__device__ __forceinline__ void fa_load_k(const uint16_t *Kg, int64_t rs, int64_t tok0,
                                          int64_t tok_max, int tid, uint4 (&kr)[4],
                                          const int32_t *ptab, int psh) {
    const int r = tid >> 3;
    int64_t tok = tok0 + r;
    tok = tok < tok_max ? tok : tok_max - 1;
    const uint16_t *src = Kg + fa_row<PAGED>(ptab, psh, tok) * rs + 8 * (tid & 7);
#pragma unroll
    for (int u = 0; u < 4; ++u) kr[u] = *reinterpret_cast<const uint4 *>(src + 64 * u);
}

// ... and into the K tile: row r, chunk c at slot c ^ r.
__device__ __forceinline__ void fa_store_k(const uint4 (&kr)[4], unsigned char *kbuf, int tid) {
    const int r = tid >> 3;
    unsigned char *row = kbuf + r * kFaKRow;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int c = (tid & 7) + 8 * u;
        *reinterpret_cast<uint4 *>(row + 16 * (c ^ r)) = kr[u];
    }
}

// V tile into registers: thread t takes tokens 4a .. 4a+3 (a = t % 8) and
// dims 8c .. 8c+7 (c = t / 8).
template <bool PAGED>
__device__ __forceinline__ void fa_load_v(const uint16_t *Vg, int64_t rs, int64_t tok0,
                                          int64_t tok_max, int tid, uint4 (&v)[4],
                                          const int32_t *ptab, int psh) {
    const int a = tid & 7, c = tid >> 3;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        int64_t tok = tok0 + 4 * a + u;
        tok = tok < tok_max ? tok : tok_max - 1;
        v[u] = *reinterpret_cast<const uint4 *>(Vg + fa_row<PAGED>(ptab, psh, tok) * rs + 8 * c);
    }
}

// ... and transposed into the V^T tile as fp16: for each of the 8 dims, the
// 4 tokens' values as one 8-byte write.
__device__ __forceinline__ void fa_store_vt(const uint4 (&v)[4], unsigned char *vbuf, int tid) {
    const int a = tid & 7, c = tid >> 3;
    const int slot = vslot(4 * a);
    const uint32_t w[4][4] = {{v[0].x, v[0].y, v[0].z, v[0].w},
                              {v[1].x, v[1].y, v[1].z, v[1].w},
                              {v[2].x, v[2].y, v[2].z, v[2].w},
                              {v[3].x, v[3].y, v[3].z, v[3].w}};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // dim 2k: low halves of word k; dim 2k+1: high halves
        const uint32_t lo0 = bf16x2_to_f16x2(w[0][k] & 0xFFFFu, w[1][k] & 0xFFFFu);
        const uint32_t lo1 = bf16x2_to_f16x2(w[2][k] & 0xFFFFu, w[3][k] & 0xFFFFu);
        const uint32_t hi0 = bf16x2_to_f16x2(w[0][k] >> 16, w[1][k] >> 16);
        const uint32_t hi1 = bf16x2_to_f16x2(w[2][k] >> 16, w[3][k] >> 16);
        *reinterpret_cast<uint2 *>(vbuf + (8 * c + 2 * k) * kFaVRow + 2 * slot) =
            make_uint2(lo0, lo1);
        *reinterpret_cast<uint2 *>(vbuf + (8 * c + 2 * k + 1) * kFaVRow + 2 * slot) =
            make_uint2(hi0, hi1);
    }
}

template <bool PAGED>
__global__ void __launch_bounds__(256) fa_prefill_kernel(FaArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char fa_lds[kFaLds];
    unsigned char *const qbase = fa_lds;                            // Q tile
    unsigned char *const kbase = fa_lds + kFaQTile;                 // two K tiles
    unsigned char *const vbase = fa_lds + kFaQTile + 2 * kFaKTile;  // two V^T tiles

    const int qblk = gridDim.x - 1 - blockIdx.x;  // longest rows first
    const int hq = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, h = lane >> 5;
    const int group = a.H / a.Hkv, g = hq / group;
    const int64_t rs = static_cast<int64_t>(a.Hkv) * kHeadDim;
    const int64_t seq_off = PAGED ? 0 : b * a.Lmax * rs;
    const uint16_t *Kg = a.K + seq_off + g * kHeadDim;
    const uint16_t *Vg = a.V + seq_off + g * kHeadDim;
    const int32_t *ptab = PAGED ? a.ptable + b * a.pstride : nullptr;
    const int psh = a.pshift;

    const int64_t q0 = static_cast<int64_t>(qblk) * kFaQ;
    const int64_t q_last = min(q0 + kFaQ, a.Tq) - 1;
    const int64_t tok_end = a.pos0 + q_last + 1;  // tokens the workgroup needs
    const int ntiles = static_cast<int>((tok_end + kFaN - 1) / kFaN);
    // this lane's query (column n of the wave's 32)
    const int64_t tq = q0 + 32 * wave + n;
    const int64_t qpos = a.pos0 + (tq < a.Tq ? tq : a.Tq - 1);
    const int64_t wave_first = a.pos0 + min(q0 + 32 * wave, a.Tq - 1);
    const int64_t wave_last = a.pos0 + min(q0 + 32 * wave + 31, a.Tq - 1);

    // Q tile: row q (query q0 + q), chunk c at slot c ^ (q % 32); thread t
    // copies chunks (t & 1) + 2u of row t / 2
    {
        const int qr = tid >> 1;
        const int64_t tqr = q0 + qr < a.Tq ? q0 + qr : a.Tq - 1;
        const uint16_t *src = a.Q + ((b * a.Tq + tqr) * a.H + hq) * kHeadDim + 8 * (tid & 1);
        uint4 qv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) qv[u] = *reinterpret_cast<const uint4 *>(src + 16 * u);
        unsigned char *row = qbase + qr * 512;
#pragma unroll
        for (int u = 0; u < 16; ++u)
            *reinterpret_cast<uint4 *>(row + 16 * (((tid & 1) + 2 * u) ^ (qr & 31))) = qv[u];
    }
    // Q^T fragment reads of this lane: row 32*wave + n, chunk 2*ks + h
    const unsigned char *qrow = qbase + (32 * wave + n) * 512;

    f32x16 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m_ref = -INFINITY, l = 0.f;

    uint4 kreg[4], vreg[4];
    fa_load_k<PAGED>(Kg, rs, 0, a.Lmax, tid, kreg, ptab, psh);
    fa_load_v<PAGED>(Vg, rs, 0, a.Lmax, tid, vreg, ptab, psh);
    fa_store_k(kreg, kbase, tid);
    fa_store_vt(vreg, vbase, tid);

    for (int it = 0; it < ntiles; ++it) {
        const int cur = it & 1;
        block_sync();  // tile `it` is in LDS; tile it-1's buffers are free
        const int64_t tile0 = static_cast<int64_t>(it) * kFaN;
        // next tile into registers while this one is consumed (after the last
        // tile this fetches clamped rows into a buffer nothing reads)
        fa_load_k<PAGED>(Kg, rs, tile0 + kFaN, a.Lmax, tid, kreg, ptab, psh);
        fa_load_v<PAGED>(Vg, rs, tile0 + kFaN, a.Lmax, tid, vreg, ptab, psh);
        // S^T, softmax, P^T . V accumulation
        if (tile0 <= wave_last) {  // some query of this wave sees the tile
            const int64_t sub0 = tile0;
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
            const unsigned char *krow = kbase + cur * kFaKTile + n * kFaKRow;
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                const int slot = (2 * ks + h) ^ n;  // row % 32 == n
                const uint4 kv = *reinterpret_cast<const uint4 *>(krow + 16 * slot);
                const uint4 qv = *reinterpret_cast<const uint4 *>(qrow + 16 * slot);
                s = mfma32(as_bf16x8(kv), as_bf16x8(qv), s);
            }
            // online softmax of this lane's query column
            const bool diag = sub0 + 31 > wave_first;
            float tmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[r] * kFaScaleLog2;
                if (diag) {
                    const int64_t tok = sub0 + 8 * (r >> 2) + 4 * h + (r & 3);
                    x = tok <= qpos ? x : -INFINITY;
                }
                s[r] = x;
                tmax = fmaxf(tmax, x);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            if (__ballot(tmax > m_ref + kFaSlack)) {
                const float m_new = fmaxf(m_ref, tmax);
                const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_ref - m_new);
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
                m_ref = m_new;
            }
            const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
            // P^T fragments (fp16, nearest) of the two 16-token steps
            f16x8 pf[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const _Float16 ph = static_cast<_Float16>(exp2f(s[8 * kk + j] - m_use));
                    l += static_cast<float>(ph);
                    pf[kk][j] = ph;
                }
            }
            const unsigned char *vt = vbase + cur * kFaVTile + n * kFaVRow + 16 * h;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const uint4 vv =
                        *reinterpret_cast<const uint4 *>(vt + 32 * dt * kFaVRow + 32 * kk);
                    o[dt] = mfma32h(__builtin_bit_cast(f16x8, vv), pf[kk], o[dt]);
                }
            }
        }
        fa_store_k(kreg, kbase + (cur ^ 1) * kFaKTile, tid);
        fa_store_vt(vreg, vbase + (cur ^ 1) * kFaVTile, tid);
    }

    // ---- normalise and store this lane's query column
    l += __shfl_xor(l, 32);
    if (tq < a.Tq) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *dst = a.O + ((b * a.Tq + tq) * a.H + hq) * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                *reinterpret_cast<float4 *>(dst + 32 * dt + 8 * gq + 4 * h) =
                    make_float4(o[dt][4 * gq] * inv, o[dt][4 * gq + 1] * inv,
                                o[dt][4 * gq + 2] * inv, o[dt][4 * gq + 3] * inv);
        if (a.lse && h == 0)
            a.lse[(b * a.Tq + tq) * a.H + hq] =
                l > 0.f ? (m_ref + log2f(l)) * kFaLn2 : -INFINITY;
    }
}

hipError_t launch_dense_prefill(const AttnArgs &aa, hipStream_t s) {
    if (aa.Tq == 0 || aa.B == 0) return hipSuccess;
    FaArgs a{};
    a.Q = aa.Q; a.K = aa.K; a.V = aa.V; a.O = aa.O; a.lse = aa.lse;
    a.Tq = aa.Tq; a.Lmax = aa.Lmax; a.pos0 = aa.pos0; a.H = aa.H; a.Hkv = aa.Hkv;
    a.ptable = aa.ptable; a.pstride = aa.pstride; a.pshift = aa.pshift;
    const dim3 grid(static_cast<uint32_t>((aa.Tq + kFaQ - 1) / kFaQ),
                    static_cast<uint32_t>(aa.H), static_cast<uint32_t>(aa.B));
    if (aa.ptable)
        hipLaunchKernelGGL(fa_prefill_kernel<true>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(fa_prefill_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace qsa
