// A3: indexer block scores (chlience section 6, I_ib; 4 query heads sharing
// one key head of dim 128 on pooled keys).
//
// The contraction is S[(query, head), block] = q . kbar with K = 128, run on
// bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate).  Rows of an MFMA tile
// are 4 queries x 4 heads, so the 16x16 accumulator layout (lane l holds rows
// 4*(l/16) .. +3 of column l%16) puts one query's four heads in one lane and
// the head combination (max or sum of ReLU) is register-local.
#include <type_traits>

#include "qsa_internal.h"

namespace qsa {

constexpr int kRT = 8;           // MFMA row tiles (4 queries each) per prefill wave
constexpr int kQW = 4 * kRT;     // queries per prefill wave
constexpr int kQT = 4 * kQW;     // queries per prefill workgroup (4 waves)
constexpr int kBT = 64;          // blocks per LDS tile
constexpr int kSplitTiles = 64;  // block tiles per workgroup (grid.y splits longer rows)
constexpr int kRowBytes = 272;   // LDS row stride of one pooled key (256 B + 16 B pad)
constexpr int kTileBytes = kBT * kRowBytes;
constexpr int kStageRow = 272;   // LDS row of one query's 64 staged scores (256 B + pad)

template <bool PAGED>
__device__ __forceinline__ void load_tile(const uint16_t *kbar, int64_t nb_max, int64_t tile,
                                          int bl, int part, uint4 &v0, uint4 &v1, uint4 &v2,
                                          uint4 &v3, const int32_t *ptab, int psh) {
    int64_t bb = tile * kBT + bl;
    bb = bb < nb_max ? bb : nb_max - 1;  // rows past the cache: any valid row, masked later
    if (PAGED) bb = page_row(ptab, psh, bb);
    const uint4 *src = reinterpret_cast<const uint4 *>(kbar + bb * kIdxDim) + part * 4;
    v0 = src[0];
    v1 = src[1];
    v2 = src[2];
    v3 = src[3];
}

__device__ __forceinline__ void store_tile(unsigned char *buf, int bl, int part, const uint4 &v0,
                                           const uint4 &v1, const uint4 &v2, const uint4 &v3) {
    uint4 *dst = reinterpret_cast<uint4 *>(buf + bl * kRowBytes + part * 64);
    dst[0] = v0;
    dst[1] = v1;
    dst[2] = v2;
    dst[3] = v3;
}

// Prefill form: queries pos0 + t, t < Tq, one sequence per blockIdx.z.
// Pooled-key tiles are double-buffered: the next tile is loaded into
// registers while the current one feeds the MFMAs, then written to the other
// LDS buffer (one barrier per tile).  Each wave stages its 32 x 64 scores in
// LDS and writes them back as whole 256-byte row segments.  With gmax set it
// also writes the largest score key of every 16 consecutive blocks,
// gmax[t * gld + g] (blocks a query does not see count as -inf), from which
// the top-K takes its floor.
// Each wave holds 32 queries' fragments (128 VGPRs), so every pooled-key
// fragment read from LDS feeds 8 MFMAs; at 2 waves per SIMD (68 KB of LDS,
// 2 workgroups per CU) that measured 1.30 against 1.50 ms per 4,096 rows at
// a 1M-token context for 16 queries per wave at 3 waves per SIMD.
template <int MODE, bool PAGED>
__global__ void __launch_bounds__(256, 2)
index_scores_prefill(const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ kbar,
                     int64_t Tq, int64_t pos0, int64_t nb_max, float *__restrict__ scores,
                     int64_t ld, uint32_t *__restrict__ gmax, int64_t gld, PageTable pg) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kTileBytes + 4 * kQW * kStageRow];
    const int qt = gridDim.x - 1 - blockIdx.x;  // longest rows first
    const int64_t seq = blockIdx.z;
    q_idx += seq * Tq * (kIdxHeads * kIdxDim);
    if (!PAGED) kbar += seq * nb_max * kIdxDim;
    const int32_t *ptab = PAGED ? pg.table + seq * pg.stride : nullptr;
    scores += seq * Tq * ld;
    if (gmax) gmax += seq * Tq * gld;

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
    unsigned char *stage = lds + 2 * kTileBytes + wave * kQW * kStageRow;

    // A fragments: row m = lane%16 of row tile rt is query kQW*wave + 4*rt + m/4,
    // head m%4; k-slots of group g4 cover dims 32*s + 8*g4 .. +7.
    bf16x8 qf[kRT][4];
    int ncq[kRT];  // complete blocks of the query whose scores this lane holds
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        const int64_t tq = t0 + kQW * wave + 4 * rt + (n >> 2);
        const int head = n & 3;
        const bool ok = tq < Tq;
        const uint16_t *src = q_idx + (ok ? tq : 0) * (kIdxHeads * kIdxDim) + head * kIdxDim;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 v = ok ? *reinterpret_cast<const uint4 *>(src + 32 * s + 8 * g4)
                         : make_uint4(0, 0, 0, 0);
            qf[rt][s] = as_bf16x8(v);
        }
        // the query whose scores this lane will hold: kQW*wave + 4*rt + g4
        const int64_t tout = t0 + kQW * wave + 4 * rt + g4;
        ncq[rt] = tout < Tq ? static_cast<int>(min(num_complete_blocks(pos0 + tout, kBlock), nb_max))
                            : -1;
    }
    // the wave's rows are consecutive queries, so the first one's complete
    // blocks bound every row's from below (-1: some row past Tq): a tile
    // below that bound needs no causal mask
    const int64_t tw0 = t0 + kQW * wave;
    const int64_t nc_wave =
        tw0 + kQW - 1 < Tq ? min(num_complete_blocks(pos0 + tw0, kBlock), nb_max) : -1;
    // write-back mapping: lane -> staged query row 4*i + lane/16, 16-byte chunk lane%16
    const int wr_q = lane >> 4, wr_c = lane & 15;

    // cooperative tile load: thread -> block tid/4, bytes 64*(tid%4) .. +63
    const int ld_bl = tid >> 2, ld_part = tid & 3;
    uint4 kv0, kv1, kv2, kv3;
    // rows past the valid blocks are clamped (paged: to the ones this tile
    // of queries sees, whose pages exist)
    const int64_t nb_rows = PAGED ? nc_hi : nb_max;
    load_tile<PAGED>(kbar, nb_rows, tile_begin, ld_bl, ld_part, kv0, kv1, kv2, kv3, ptab,
                     pg.shift);
    store_tile(lds, ld_bl, ld_part, kv0, kv1, kv2, kv3);

    for (int64_t tile = tile_begin; tile < tile_end; ++tile) {
        const int cur = static_cast<int>((tile - tile_begin) & 1);
        unsigned char *buf = lds + cur * kTileBytes;
        block_sync();  // tile ready; the other buffer is free
        // next tile into registers (past the last tile: a clamped re-read of
        // rows nothing will use)
        load_tile<PAGED>(kbar, nb_rows, tile + 1, ld_bl, ld_part, kv0, kv1, kv2, kv3, ptab,
                         pg.shift);
        const int64_t b0 = tile * kBT;
        // the scores of the tile's 64 blocks into the stage (MASKED: blocks
        // a row does not see score -inf)
        auto score_tile = [&](auto masked) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x8 kf[4];
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    kf[s] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                        buf + (16 * j + n) * kRowBytes + 64 * s + 16 * g4));
                const int blk = static_cast<int>(b0) + 16 * j + n;  // blocks < 2^27
                // the row tiles' accumulators interleaved: no MFMA waits on
                // the one before it
                f32x4 acc[kRT];
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int rt = 0; rt < kRT; ++rt)
                        acc[rt] = mfma_bf16_16x16x32(qf[rt][s], kf[s], acc[rt]);
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) {
                    float v;
                    if constexpr (decltype(masked)::value)
                        v = blk < ncq[rt] ? combine_heads<MODE>(acc[rt]) : -INFINITY;
                    else
                        v = combine_heads<MODE>(acc[rt]);
                    *reinterpret_cast<float *>(stage + (4 * rt + g4) * kStageRow +
                                               4 * (16 * j + n)) = v;
                }
            }
        };
        if (b0 + kBT <= nc_wave)
            score_tile(std::false_type{});
        else
            score_tile(std::true_type{});
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // write back: kRT instructions, each 4 query rows x 256 contiguous
        // bytes (unrolled by 2: fully unrolled, the 8 rounds spill registers)
#pragma unroll 2
        for (int i = 0; i < kRT; ++i) {
            const int ql = 4 * i + wr_q;  // staged row = 4*rt + g4 of query kQW*wave + ql
            const int64_t tout = t0 + kQW * wave + ql;
            const int64_t blk = b0 + 4 * wr_c;
            const float4 v = *reinterpret_cast<const float4 *>(stage + ql * kStageRow + 16 * wr_c);
            // non-temporal: the score rows are read back once, by the top-K,
            // and mostly not at all (it loads only the groups that reach its
            // floor); 18% faster than plain stores at a 1M-token context
            if (tout < Tq && blk < ld)
                __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w},
                                            reinterpret_cast<f32x4 *>(scores + tout * ld + blk));
            if (gmax) {
                // the 16-block group of the 4 lanes wr_c & ~3 .. | 3 (a quad):
                // float max across the quad by DPP moves (lane ^ 1, lane ^ 2),
                // then one key (the key order is the float order)
                float m = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
                m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1,
                                                                     0xF, 0xF, false)));
                m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E,
                                                                     0xF, 0xF, false)));
                const int64_t gi = (b0 >> 4) + (wr_c >> 2);
                if ((wr_c & 3) == 0 && tout < Tq && gi < gld) gmax[tout * gld + gi] = score_key(m);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        store_tile(lds + (cur ^ 1) * kTileBytes, ld_bl, ld_part, kv0, kv1, kv2, kv3);
    }
}

// Decode form: the selection of sequence b is made for the first of its nq
// newest queries (position seq_len[b] - nq, indexer query q_idx[b][0]; nq > 1
// when the speculative steps reuse one selection); the kernel streams
// the pooled-key cache.  Each wave scores 64 pooled keys: 16 LDS-DMA
// instructions copy them into a 16 KB tile, each instruction 1 KB of
// contiguous HBM (4 keys), with the 16-byte chunks of row r stored at slot
// chunk ^ (r % 16) so that the MFMA B-fragment reads (16 rows, one chunk
// each) hit distinct banks.  MFMA rows 0..3 are the 4 heads, rows 4..15 zero.
template <int MODE, bool PAGED>
__global__ void __launch_bounds__(256)
index_scores_decode(const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ kbar,
                    const int64_t *__restrict__ seq_len, int64_t nb_max,
                    float *__restrict__ scores, int64_t ld, uint32_t *__restrict__ gmax,
                    int64_t gld, int nq, PageTable pg) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * 64 * kIdxDim * 2];
    const int64_t seq = blockIdx.y;
    const int64_t p = seq_len[seq] - nq;
    const int64_t nc = min(num_complete_blocks(p, kBlock), nb_max);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g4 = lane >> 4;
    const int64_t w0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 64;  // first block
    if (w0 >= nc) return;
    unsigned char *tile = lds + wave * (64 * kIdxDim * 2);
    const uint16_t *kb = PAGED ? kbar : kbar + seq * nb_max * kIdxDim;
    // paged: lane l holds the page of the wave's l-th page of blocks (only
    // pages of the sequence's complete blocks are read)
    int32_t mypage = 0;
    int64_t pg0 = 0;
    if (PAGED) {
        pg0 = w0 >> pg.shift;
        const int64_t pg_last = min(w0 + 63, nc - 1) >> pg.shift;
        mypage = lane <= pg_last - pg0 ? pg.table[seq * pg.stride + pg0 + lane] : 0;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int r = 4 * j + (lane >> 4);
        int64_t blk = w0 + r;
        if (PAGED) {
            blk = blk < nc ? blk : nc - 1;
            const int32_t page = __shfl(mypage, static_cast<int>((blk >> pg.shift) - pg0));
            blk = (static_cast<int64_t>(page) << pg.shift) | (blk & ((int64_t(1) << pg.shift) - 1));
        } else {
            blk = blk < nb_max ? blk : nb_max - 1;
        }
        const uint16_t *src = kb + blk * kIdxDim + 8 * ((lane & 15) ^ (r & 15));
        // (C-style casts: the builtin takes explicit global / LDS address spaces)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)(tile + 1024 * j),
                                         16, 0, 0);
    }
    const uint16_t *q = q_idx + seq * nq * (kIdxHeads * kIdxDim);
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
    uint32_t kmax = 0u;  // largest key of the wave's valid blocks (lanes 0..15)
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
        const float v = combine_heads<MODE>(acc);
        if (g4 == 0 && blk < nc) {
            out[blk] = v;
            kmax = max(kmax, score_key(v));
        }
    }
    // Group maximum of the 64 blocks (a floor source for the top-K): lanes
    // 0..15 fold within their 16-lane group.
    if (gmax) {
#pragma unroll
        for (int off = 8; off > 0; off >>= 1)
            kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), off)));
        if (lane == 0) gmax[seq * gld + (w0 >> 6)] = kmax;
    }
}

template <int MODE>
static void launch_decode_scan(dim3 grid, hipStream_t s, const uint16_t *q_idx,
                               const uint16_t *kbar, const int64_t *seq_len, int64_t nb_max,
                               float *scores, int64_t ld, uint32_t *gmax, int64_t gld, int nq,
                               const PageTable &pg) {
    if (pg.table)
        hipLaunchKernelGGL((index_scores_decode<MODE, true>), grid, dim3(256), 0, s, q_idx, kbar,
                           seq_len, nb_max, scores, ld, gmax, gld, nq, pg);
    else
        hipLaunchKernelGGL((index_scores_decode<MODE, false>), grid, dim3(256), 0, s, q_idx,
                           kbar, seq_len, nb_max, scores, ld, gmax, gld, nq, pg);
}

template <int MODE>
static void launch_prefill_scores(dim3 grid, hipStream_t s, const uint16_t *q_idx,
                                  const uint16_t *kbar, int64_t Tq, int64_t pos0, int64_t nb_max,
                                  float *scores, int64_t ld, uint32_t *gmax, int64_t gld,
                                  const PageTable &pg) {
    if (pg.table)
        hipLaunchKernelGGL((index_scores_prefill<MODE, true>), grid, dim3(256), 0, s, q_idx,
                           kbar, Tq, pos0, nb_max, scores, ld, gmax, gld, pg);
    else
        hipLaunchKernelGGL((index_scores_prefill<MODE, false>), grid, dim3(256), 0, s, q_idx,
                           kbar, Tq, pos0, nb_max, scores, ld, gmax, gld, pg);
}

hipError_t launch_index_scores(const uint16_t *q_idx, const uint16_t *kbar, int B, int64_t Tq,
                               int64_t pos0, const int64_t *seq_len, int64_t nb_max, int mode,
                               float *scores, int64_t ld, hipStream_t s, uint32_t *gmax,
                               int64_t gld, PageTable pg) {
    if (B == 0 || Tq == 0 || nb_max == 0) return hipSuccess;
    if (seq_len) {
        const dim3 grid(static_cast<uint32_t>((nb_max + 255) / 256), static_cast<uint32_t>(B));
        const int nq = static_cast<int>(Tq);
        if (mode == 0)
            launch_decode_scan<0>(grid, s, q_idx, kbar, seq_len, nb_max, scores, ld, gmax, gld,
                                  nq, pg);
        else
            launch_decode_scan<1>(grid, s, q_idx, kbar, seq_len, nb_max, scores, ld, gmax, gld,
                                  nq, pg);
        return hipGetLastError();
    }
    const int64_t n_qt = (Tq + kQT - 1) / kQT;
    const int64_t nc_hi = min(num_complete_blocks(pos0 + Tq - 1, kBlock), nb_max);
    const int64_t n_tiles = (nc_hi + kBT - 1) / kBT;
    const int64_t n_split = n_tiles > 0 ? (n_tiles + kSplitTiles - 1) / kSplitTiles : 1;
    const dim3 grid(static_cast<uint32_t>(n_qt), static_cast<uint32_t>(n_split),
                    static_cast<uint32_t>(B));
    if (mode == 0)
        launch_prefill_scores<0>(grid, s, q_idx, kbar, Tq, pos0, nb_max, scores, ld, gmax, gld,
                                 pg);
    else
        launch_prefill_scores<1>(grid, s, q_idx, kbar, Tq, pos0, nb_max, scores, ld, gmax, gld,
                                 pg);
    return hipGetLastError();
}

}  // namespace qsa
