// A3: indexer block scores (chlience section 6, I_ib; 4 query heads sharing
// one key head of dim 128 on pooled keys).
//
// The contraction is S[(query, head), block] = q . kbar with K = 128, run on
// bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate).  Rows of an MFMA tile
// are 4 queries x 4 heads, so the 16x16 accumulator layout (lane l holds rows
// 4*(l/16) .. +3 of column l%16) puts one query's four heads in one lane and
// the head combination (max or sum of ReLU) is register-local.
#include "qsa_internal.h"

namespace qsa {

constexpr int kQT = 64;          // queries per prefill workgroup (4 waves x 16)
constexpr int kBT = 64;          // blocks per LDS tile
constexpr int kSplitTiles = 64;  // block tiles per workgroup (grid.y splits longer rows)
constexpr int kRowBytes = 272;   // LDS row stride of one pooled key (256 B + 16 B pad)

// Prefill form: queries pos0 + t, t < Tq, one sequence per blockIdx.z.
template <int MODE>
__global__ void __launch_bounds__(256)
index_scores_prefill(const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ kbar,
                     int64_t Tq, int64_t pos0, int64_t nb_max, float *__restrict__ scores,
                     int64_t ld) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kBT * kRowBytes];
    const int qt = gridDim.x - 1 - blockIdx.x;  // longest rows first
    const int64_t seq = blockIdx.z;
    q_idx += seq * Tq * (kIdxHeads * kIdxDim);
    kbar += seq * nb_max * kIdxDim;
    scores += seq * Tq * ld;

    const int64_t t0 = static_cast<int64_t>(qt) * kQT;
    const int64_t t_last = min(t0 + kQT, Tq) - 1;
    const int64_t nc_hi = min(num_complete_blocks(pos0 + t_last, kBlock), nb_max);
    const int64_t n_tiles = (nc_hi + kBT - 1) / kBT;
    const int64_t tile_begin = static_cast<int64_t>(blockIdx.y) * kSplitTiles;
    const int64_t tile_end = min(tile_begin + kSplitTiles, n_tiles);
    if (tile_begin >= tile_end) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g4 = lane >> 4;

    // A fragments: row m = lane%16 of row tile rt is query 16*wave + 4*rt + m/4,
    // head m%4; k-slots of group g4 cover dims 32*s + 8*g4 .. +7.
    bf16x8 qf[4][4];
    int64_t ncq[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int64_t tq = t0 + 16 * wave + 4 * rt + (n >> 2);
        const int head = n & 3;
        const bool ok = tq < Tq;
        const uint16_t *src = q_idx + (ok ? tq : 0) * (kIdxHeads * kIdxDim) + head * kIdxDim;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 v = ok ? *reinterpret_cast<const uint4 *>(src + 32 * s + 8 * g4)
                         : make_uint4(0, 0, 0, 0);
            qf[rt][s] = as_bf16x8(v);
        }
        // the query whose scores this lane will hold: 16*wave + 4*rt + g4
        const int64_t tout = t0 + 16 * wave + 4 * rt + g4;
        ncq[rt] = tout < Tq ? min(num_complete_blocks(pos0 + tout, kBlock), nb_max) : -1;
    }

    for (int64_t tile = tile_begin; tile < tile_end; ++tile) {
        const int64_t b0 = tile * kBT;
        // cooperative load: thread -> block tid/4, bytes 64*(tid%4) .. +63
        {
            const int bl = tid >> 2, part = tid & 3;
            const int64_t bb = b0 + bl;
            uint4 v[4];
            if (bb < nb_max) {
                const uint4 *src =
                    reinterpret_cast<const uint4 *>(kbar + bb * kIdxDim) + part * 4;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = src[i];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = make_uint4(0, 0, 0, 0);
            }
            uint4 *dst = reinterpret_cast<uint4 *>(lds + bl * kRowBytes + part * 64);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = v[i];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8 kf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kf[s] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                    lds + (16 * j + n) * kRowBytes + 64 * s + 16 * g4));
            const int64_t blk = b0 + 16 * j + n;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma_bf16_16x16x32(qf[rt][s], kf[s], acc);
                if (ncq[rt] >= 0 && blk < ld) {
                    const float v = blk < ncq[rt] ? combine_heads<MODE>(acc) : -INFINITY;
                    const int64_t tout = t0 + 16 * wave + 4 * rt + g4;
                    scores[tout * ld + blk] = v;
                }
            }
        }
        __syncthreads();
    }
}

// Decode form: one query per sequence at seq_len[b] - 1; the kernel streams
// the pooled-key cache.  Each wave scores 64 pooled keys: 16 LDS-DMA
// instructions copy them into a 16 KB tile, each instruction 1 KB of
// contiguous HBM (4 keys), with the 16-byte chunks of row r stored at slot
// chunk ^ (r % 16) so that the MFMA B-fragment reads (16 rows, one chunk
// each) hit distinct banks.  MFMA rows 0..3 are the 4 heads, rows 4..15 zero.
template <int MODE>
__global__ void __launch_bounds__(256)
index_scores_decode(const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ kbar,
                    const int64_t *__restrict__ seq_len, int64_t nb_max,
                    float *__restrict__ scores, int64_t ld) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * 64 * kIdxDim * 2];
    const int64_t seq = blockIdx.y;
    const int64_t p = seq_len[seq] - 1;
    const int64_t nc = min(num_complete_blocks(p, kBlock), nb_max);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g4 = lane >> 4;
    const int64_t w0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 64;  // first block
    if (w0 >= nc) return;
    unsigned char *tile = lds + wave * (64 * kIdxDim * 2);
    const uint16_t *kb = kbar + seq * nb_max * kIdxDim;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int r = 4 * j + (lane >> 4);
        int64_t blk = w0 + r;
        blk = blk < nb_max ? blk : nb_max - 1;
        const uint16_t *src = kb + blk * kIdxDim + 8 * ((lane & 15) ^ (r & 15));
        // (C-style casts: the builtin takes explicit global / LDS address spaces)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)(tile + 1024 * j),
                                         16, 0, 0);
    }
    const uint16_t *q = q_idx + seq * (kIdxHeads * kIdxDim);
    bf16x8 qf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint4 v = n < kIdxHeads
                      ? *reinterpret_cast<const uint4 *>(q + n * kIdxDim + 32 * s + 8 * g4)
                      : make_uint4(0, 0, 0, 0);
        qf[s] = as_bf16x8(v);
    }
    float *out = scores + seq * ld;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile has landed
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const int row = 16 * jt + n;  // row % 16 == n
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 kv =
                *reinterpret_cast<const uint4 *>(tile + 256 * row + 16 * ((4 * s + g4) ^ n));
            acc = mfma_bf16_16x16x32(qf[s], as_bf16x8(kv), acc);
        }
        const int64_t blk = w0 + row;
        if (g4 == 0 && blk < nc) out[blk] = combine_heads<MODE>(acc);
    }
}

hipError_t launch_index_scores(const uint16_t *q_idx, const uint16_t *kbar, int B, int64_t Tq,
                               int64_t pos0, const int64_t *seq_len, int64_t nb_max, int mode,
                               float *scores, int64_t ld, hipStream_t s) {
    if (B == 0 || Tq == 0 || nb_max == 0) return hipSuccess;
    if (seq_len) {
        const dim3 grid(static_cast<uint32_t>((nb_max + 255) / 256), static_cast<uint32_t>(B));
        if (mode == 0)
            hipLaunchKernelGGL(index_scores_decode<0>, grid, dim3(256), 0, s, q_idx, kbar,
                               seq_len, nb_max, scores, ld);
        else
            hipLaunchKernelGGL(index_scores_decode<1>, grid, dim3(256), 0, s, q_idx, kbar,
                               seq_len, nb_max, scores, ld);
        return hipGetLastError();
    }
    const int64_t n_qt = (Tq + kQT - 1) / kQT;
    const int64_t nc_hi = min(num_complete_blocks(pos0 + Tq - 1, kBlock), nb_max);
    const int64_t n_tiles = (nc_hi + kBT - 1) / kBT;
    const int64_t n_split = n_tiles > 0 ? (n_tiles + kSplitTiles - 1) / kSplitTiles : 1;
    const dim3 grid(static_cast<uint32_t>(n_qt), static_cast<uint32_t>(n_split),
                    static_cast<uint32_t>(B));
    if (mode == 0)
        hipLaunchKernelGGL(index_scores_prefill<0>, grid, dim3(256), 0, s, q_idx, kbar, Tq,
                           pos0, nb_max, scores, ld);
    else
        hipLaunchKernelGGL(index_scores_prefill<1>, grid, dim3(256), 0, s, q_idx, kbar, Tq,
                           pos0, nb_max, scores, ld);
    return hipGetLastError();
}

}  // namespace qsa
