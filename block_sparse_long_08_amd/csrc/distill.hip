// Stage-1 indexer distillation, forward (chlience section 6: the first stage
// trains the indexer alone against a teacher distribution made from full
// attention, max-pooled within each micro-block, by minimising KL; ai.info
// "Industry relevance": one fused kernel yields the KL loss without storing
// intermediates).  For the query at position p, with the dense attention
// probabilities A_hj of head h (softmax over the tokens j <= p, from the
// dense pass's log-sum-exp):
//   M_hb = max over the 4 tokens of block b of A_hj, for the nc(p) complete
//          blocks b;
//   T_b  = sum over the 24 heads of M_hb, normalised to sum 1;
//   S_b  = softmax over the complete blocks of the indexer scores s_b;
//   KL   = sum_b T_b (ln T_b - ln S_b)
//        = A / Z - ln Z - C / Z + lse(s),  with Z = sum_b t_b,
//          A = sum_b t_b ln t_b, C = sum_b t_b s_b over the unnormalised t_b.
//
// distill_kl_kernel: a workgroup takes 16 queries and all 24 heads (8 waves,
// wave w: KV head w / 4 and its query heads w % 4 + 4k, k = 0..2).  Key tiles
// of 64 tokens of both KV heads arrive by LDS DMA into two alternating
// buffers.  Per head the transposed logits S^T[16 tok, 16 q] = K . Q^T run on
// 16x16x32 bf16 MFMA, so a lane holds one block (4 tokens) of one query and
// the block max is register-local.  The 8 waves' head sums meet in LDS and
// are added in a fixed order by one thread per (query, block), which keeps
// Z, A, C and the running log-sum-exp of s for its row; the 16 threads of a
// row combine them at the end and write KL.  Nothing per block leaves the
// workgroup.  One barrier per tile: it publishes the tile's head sums and
// the next tile's keys.  The two key buffers and the two head-sum buffers
// are distinct LDS arrays picked at compile time (the tile loop runs in
// pairs), so the compiler can tell that the reads of one buffer do not
// alias the DMA into the other and does not wait for that DMA first.
#include "qsa_internal.h"

namespace qsa {

constexpr int kDsQ = 16;                              // queries per workgroup
constexpr int kDsTok = 64;                            // tokens per key tile (16 blocks)
constexpr int kDsKRow = 512;                          // one token of one KV head
constexpr int kDsKv = 2;                              // KV heads per workgroup
constexpr int kDsBuf = kDsKv * kDsTok * kDsKRow;      // one key tile, both KV heads
constexpr float kDsScaleLog2 = 0.09016844005556021f;  // log2(e) / sqrt(256)
constexpr float kDsLog2e = 1.4426950408889634f;

// Grid: ceil(rows / 16) workgroups of 512 threads.  Q: [rows][24][256] of
// the chunk; lse: [rows][24] natural-log dense log-sum-exp; K: [Tk][2][256];
// scores: [rows][ld] indexer scores of the chunk; kl: [rows].
__global__ void __launch_bounds__(512)
distill_kl_kernel(const uint16_t *__restrict__ Q, const float *__restrict__ lse,
                  const uint16_t *__restrict__ K, const float *__restrict__ scores, int64_t rows,
                  int64_t pos0, int64_t Tk, int64_t ld, float *__restrict__ kl) {
    __shared__ __attribute__((aligned(16))) unsigned char kt0[kDsBuf];
    __shared__ __attribute__((aligned(16))) unsigned char kt1[kDsBuf];
    __shared__ float red0[8][kDsQ][17];
    __shared__ float red1[8][kDsQ][17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g4 = lane >> 4;
    const int g = wave >> 2;  // this wave's KV head
    constexpr int H = 12 * kDsKv;
    constexpr int64_t rs = kDsKv * kHeadDim;
    // longest rows first: the causal tail of the grid is the short rows
    const int64_t row0 = static_cast<int64_t>(gridDim.x - 1 - blockIdx.x) * kDsQ;
    const int64_t last = min(row0 + kDsQ, rows) - 1;
    const int64_t nc_hi = num_complete_blocks(pos0 + last, kBlock);
    const int ntiles = static_cast<int>((nc_hi * kBlock + kDsTok - 1) / kDsTok);

    // Q^T fragments of this lane's query (column n) for the wave's 3 heads:
    // step s holds dims 32s + 8*g4 .. +7; and each head's lse in log2 units
    const int64_t qrow = min(row0 + n, rows - 1);
    uint4 qf[3][8];
    float lse2[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int h = 12 * g + (wave & 3) + 4 * k;
        const uint16_t *src = Q + (qrow * H + h) * kHeadDim + 8 * g4;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[k][s] = *reinterpret_cast<const uint4 *>(src + 32 * s);
        lse2[k] = lse[qrow * H + h] * kDsLog2e;
    }

    // Key tile `it` into dst: DMA instruction j of wave w fills the 1 KB at
    // 1024 * (8w + j) = KV head (8w + j) / 32, token rows
    // 2 * ((8w + j) % 32) + lane / 32, slot lane % 32, where chunk c of row r
    // sits at slot c ^ (r % 32); the lane fetches the chunk of its slot.
    auto dma_tile = [&](int it, unsigned char *dst) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int piece = 8 * wave + j;
            const int kv = piece >> 5, rr = 2 * (piece & 31) + (lane >> 5);
            int64_t tok = static_cast<int64_t>(it) * kDsTok + rr;
            tok = tok < Tk ? tok : Tk - 1;  // past the context: blocks never used
            const int c = (lane & 31) ^ (rr & 31);
            const uint16_t *src = K + tok * rs + kv * kHeadDim + 8 * c;
            // (C-style casts: the builtin takes explicit global / LDS address spaces)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)src,
                (__attribute__((address_space(3))) void *)(dst + 1024 * piece), 16, 0, 0);
        }
    };

    // the reducing thread's (query, block) and its row's running sums
    const int q = tid >> 4, blk = tid & 15;
    const int64_t row = row0 + q;
    const bool reducer = tid < 256 && row < rows;
    const int64_t nc = reducer ? num_complete_blocks(pos0 + row, kBlock) : 0;
    float z = 0.f, a = 0.f, c = 0.f, m = -INFINITY, zs = 0.f;

    // tile `it` from cur while tile it + 1 streams into nxt; head sums in rd
    auto step = [&](int it, const unsigned char *cur, unsigned char *nxt,
                    float (*rd)[kDsQ][17]) {
        if (it + 1 < ntiles) dma_tile(it + 1, nxt);
        const int64_t b = static_cast<int64_t>(it) * 16 + blk;
        const bool live = reducer && b < nc;
        const float s = live ? scores[row * ld + b] : 0.f;  // in flight during the MFMAs
        const unsigned char *kb = cur + g * (kDsTok * kDsKRow);
#pragma unroll 2
        for (int ct = 0; ct < 4; ++ct) {
            const int r = 16 * ct + n;  // token row of this lane's A fragment
            bf16x8 kf[8];
#pragma unroll
            for (int st = 0; st < 8; ++st)
                kf[st] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    kb + r * kDsKRow + 16 * ((4 * st + g4) ^ (r & 31))));
            float tsum = 0.f;  // block 4*ct + g4 of query n, this wave's heads
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 8; ++st)
                    acc = mfma_bf16_16x16x32(kf[st], as_bf16x8(qf[k][st]), acc);
                // the exponential is monotone: the block max takes one exp2
                const float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
                tsum += exp2f(mx * kDsScaleLog2 - lse2[k]);
            }
            rd[wave][n][4 * ct + g4] = tsum;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile it + 1 has landed
        block_sync();
        // rd is written again two tiles on, after the next barrier
        if (live) {
            // the 24 heads in a fixed order: KV head 0's waves, then KV head 1's
            const float t = (((rd[0][q][blk] + rd[1][q][blk]) + rd[2][q][blk]) +
                             rd[3][q][blk]) +
                            (((rd[4][q][blk] + rd[5][q][blk]) + rd[6][q][blk]) +
                             rd[7][q][blk]);
            z += t;
            a += t > 0.f ? t * logf(t) : 0.f;
            c += t * s;
            if (s > m) {
                zs = zs * expf(m - s) + 1.f;
                m = s;
            } else {
                zs += expf(s - m);
            }
        }
    };
    if (ntiles > 0) dma_tile(0, kt0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile 0 has landed
    block_sync();
    for (int it = 0; it < ntiles; it += 2) {
        step(it, kt0, kt1, red0);
        if (it + 1 < ntiles) step(it + 1, kt1, kt0, red1);
    }
    if (tid >= 256) return;
    // the 16 threads of a row are 16 consecutive lanes
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        z += __shfl_xor(z, off);
        a += __shfl_xor(a, off);
        c += __shfl_xor(c, off);
        const float m2 = __shfl_xor(m, off), zs2 = __shfl_xor(zs, off);
        const float mn = fmaxf(m, m2);
        zs = (m == -INFINITY ? 0.f : zs * expf(m - mn)) +
             (m2 == -INFINITY ? 0.f : zs2 * expf(m2 - mn));
        m = mn;
    }
    if (blk == 0 && row < rows) kl[row] = nc > 0 ? a / z - logf(z) - c / z + (m + logf(zs)) : 0.f;
}

hipError_t launch_distill(const uint16_t *Q, const float *lse, const uint16_t *K,
                          const float *scores, int64_t rows, int64_t pos0, int64_t Tk,
                          int64_t ld, float *kl, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(distill_kl_kernel, dim3(static_cast<uint32_t>((rows + kDsQ - 1) / kDsQ)),
                       dim3(512), 0, s, Q, lse, K, scores, rows, pos0, Tk, ld, kl);
    return hipGetLastError();
}

}  // namespace qsa
