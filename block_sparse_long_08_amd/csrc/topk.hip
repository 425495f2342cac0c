// A4: per-query top-K block selection (chlience section 6: at most 512
// complete blocks per query).
//
// One workgroup per query row.  The K-th largest score is found exactly by an
// MSB-first radix select over order-preserving uint32 keys (8-bit digits,
// LDS histograms); a final pass emits, in ascending block order, every block
// whose key is above the threshold plus the lowest-indexed blocks equal to
// it, which realises the (score desc, index asc) order.
#include "qsa_internal.h"

namespace qsa {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / kWave;

__global__ void __launch_bounds__(kTopkThreads)
topk_kernel(const float *__restrict__ scores, int64_t Tq, int64_t ld, int64_t pos0,
            const int64_t *__restrict__ seq_len, int64_t nb_max, int r, int K,
            int32_t *__restrict__ blk_idx, int32_t *__restrict__ n_sel) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_digit, sh_above;
    __shared__ uint32_t wave_cnt[2][kTopkWaves];

    const int64_t row = blockIdx.x;
    const int64_t seq = row / Tq, t = row - seq * Tq;
    int64_t p = seq_len ? seq_len[seq] - 1 : pos0 + t;
    const int64_t nc = min(num_complete_blocks(p, r), nb_max);
    const float *s = scores + row * ld;
    int32_t *out = blk_idx + row * K;
    const int tid = threadIdx.x;

    if (nc <= K) {
        for (int i = tid; i < K; i += kTopkThreads) out[i] = i < nc ? i : -1;
        if (tid == 0) n_sel[row] = static_cast<int32_t>(nc);
        return;
    }

    uint32_t prefix = 0, mask = 0, krem = static_cast<uint32_t>(K);
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int64_t i = tid; i < nc; i += kTopkThreads) {
            const uint32_t key = score_key(s[i]);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l owns digits 255-4l .. 252-4l (descending); inclusive scan
            // of counts from the top digit down
            uint32_t c[4];
            uint32_t local = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[i] = hist[255 - 4 * tid - i];
                local += c[i];
            }
            uint32_t incl = local;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                uint32_t v = __shfl_up(incl, off, kWave);
                if (tid >= off) incl += v;
            }
            uint32_t before = incl - local;  // count of digits above this lane's range
            if (before < krem && krem <= incl) {
                uint32_t acc = before;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (acc < krem && krem <= acc + c[i]) {
                        sh_digit = 255u - 4u * tid - i;
                        sh_above = acc;
                    }
                    acc += c[i];
                }
            }
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        mask |= 255u << shift;
        krem -= sh_above;
        __syncthreads();
    }
    // prefix = key of the K-th largest; krem = how many keys equal to it to take.
    const uint32_t thr = prefix;
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t written = 0, eq_seen = 0;
    for (int64_t base = 0; base < nc; base += kTopkThreads) {
        const int64_t i = base + tid;
        const uint32_t key = i < nc ? score_key(s[i]) : 0u;
        const bool gt = i < nc && key > thr;
        const bool eq = i < nc && key == thr;
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const uint64_t eq_mask = __ballot(eq);
        if (lane == 0) wave_cnt[0][wave] = __popcll(eq_mask);
        __syncthreads();
        uint32_t eq_before = eq_seen + __popcll(eq_mask & below);
        uint32_t eq_total = 0;
        for (int w = 0; w < kTopkWaves; ++w) {
            const uint32_t c = wave_cnt[0][w];
            if (w < wave) eq_before += c;
            eq_total += c;
        }
        const bool take = gt || (eq && eq_before < krem);
        const uint64_t take_mask = __ballot(take);
        if (lane == 0) wave_cnt[1][wave] = __popcll(take_mask);
        __syncthreads();
        uint32_t pos = written + __popcll(take_mask & below);
        uint32_t take_total = 0;
        for (int w = 0; w < kTopkWaves; ++w) {
            const uint32_t c = wave_cnt[1][w];
            if (w < wave) pos += c;
            take_total += c;
        }
        if (take && pos < static_cast<uint32_t>(K)) out[pos] = static_cast<int32_t>(i);
        written += take_total;
        eq_seen += eq_total;
        __syncthreads();
    }
    if (tid == 0) n_sel[row] = K;
}

hipError_t launch_topk(const float *scores, int B, int64_t Tq, int64_t ld, int64_t pos0,
                       const int64_t *seq_len, int64_t nb_max, int r, int K, int32_t *blk_idx,
                       int32_t *n_sel, hipStream_t s) {
    const int64_t rows = static_cast<int64_t>(B) * Tq;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3(static_cast<uint32_t>(rows)), dim3(kTopkThreads), 0, s,
                       scores, Tq, ld, pos0, seq_len, nb_max, r, K, blk_idx, n_sel);
    return hipGetLastError();
}

}  // namespace qsa
