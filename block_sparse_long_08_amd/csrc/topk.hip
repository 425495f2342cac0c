// A4: per-query top-K block selection (chlience section 6: at most 512
// complete blocks per query).
//
// One workgroup (1024 threads) per query row finds the K-th largest score
// exactly and emits the selected blocks in ascending order, realising the
// order (score desc, index asc):
//   1. histogram of the top 12 bits of the order-preserving uint32 keys
//      (LDS atomics) -> the bin B holding the K-th key and how many keys lie
//      above it;
//   2. the keys of bin B (few, for any spread-out row) are gathered into LDS
//      and the low 20 bits resolved by two 10-bit radix passes -> the exact
//      threshold key T and how many keys equal to T are taken (lowest
//      indices first); a bin too full for the LDS buffer is resolved by the
//      same passes over the whole row;
//   3. ordered compaction: wave w owns a contiguous run of the row, lane l
//      holds 4 consecutive keys per 256-key slice, so wave scans plus one
//      cross-wave prefix give every selected block its output slot.
// Rows of up to 32,768 candidates stay in registers (one global read); longer
// rows are streamed in tiles of 16,384 keys (three reads).
#include "qsa_internal.h"

namespace qsa {

constexpr int kNT = 1024;                 // threads per row
constexpr int kNW = kNT / kWave;          // waves
constexpr int kBins = 4096;               // first digit: key bits 31..20
constexpr int kCap = 6144;                // LDS candidates of the threshold bin

struct TopkShared {
    uint32_t hist[kBins];
    uint32_t ckey[kCap];
    uint32_t wsum[kNW];
    uint32_t sel_bin, sel_above, cand_n;
};

// Block-wide inclusive scan of one value per thread (uint32).
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, TopkShared &sh, int lane,
                                                    int wave) {
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    if (lane == kWave - 1) sh.wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += sh.wsum[w];
    __syncthreads();
    return x + before;
}

// Digit search: counts[i] (descending digit order across threads) -> the
// digit holding rank `krem` and the count above it.  Thread t owns `per`
// consecutive digits starting at digit (ndig - 1 - per*t) going down.
template <int PER>
__device__ __forceinline__ void find_digit(const uint32_t *cnt, int ndig, uint32_t krem,
                                           TopkShared &sh, int tid, int lane, int wave) {
    uint32_t c[PER];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int d = ndig - 1 - PER * tid - i;
        c[i] = d >= 0 ? cnt[d] : 0u;
        local += c[i];
    }
    const uint32_t incl = block_incl_scan(local, sh, lane, wave);
    const uint32_t before = incl - local;
    if (before < krem && krem <= incl) {
        uint32_t acc = before;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (acc < krem && krem <= acc + c[i]) {
                sh.sel_bin = static_cast<uint32_t>(ndig - 1 - PER * tid - i);
                sh.sel_above = acc;
            }
            acc += c[i];
        }
    }
    __syncthreads();
}

// Keys of one tile: wave w holds elements base + w*64*VPT + 256*j + 4*lane + c.
// Slots past the row get key 0, which lies below the key of every finite
// score (the smallest, -inf, maps to 0x007FFFFF): such slots never land in a
// searched bin and never compare >= a threshold, so no bounds test is needed.
template <int VPT>
__device__ __forceinline__ void load_keys(const float *__restrict__ s, int64_t n, int64_t base,
                                          int lane, int wave, uint32_t (&k)[VPT]) {
#pragma unroll
    for (int j = 0; j < VPT / 4; ++j) {
        const int64_t i = base + static_cast<int64_t>(wave) * 64 * VPT + 256 * j + 4 * lane;
        if (i + 3 < n) {
            const float4 v = *reinterpret_cast<const float4 *>(s + i);
            k[4 * j + 0] = score_key(v.x);
            k[4 * j + 1] = score_key(v.y);
            k[4 * j + 2] = score_key(v.z);
            k[4 * j + 3] = score_key(v.w);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) k[4 * j + c] = i + c < n ? score_key(s[i + c]) : 0u;
        }
    }
}

template <int VPT>
__device__ __forceinline__ int64_t elem_index(int64_t base, int wave, int lane, int q) {
    return base + static_cast<int64_t>(wave) * 64 * VPT + 256 * (q >> 2) + 4 * lane + (q & 3);
}

// RESIDENT: the whole row is one tile held in registers (n <= 1024*VPT).
template <int VPT, bool RESIDENT>
__global__ void __launch_bounds__(kNT)
topk_kernel(const float *__restrict__ scores, int64_t Tq, int64_t ld, int64_t pos0,
            const int64_t *__restrict__ seq_len, int64_t nb_max, int r, int K,
            int32_t *__restrict__ blk_idx, int32_t *__restrict__ n_sel) {
    __shared__ TopkShared sh;
    constexpr int64_t TILE = static_cast<int64_t>(kNT) * VPT;
    const int64_t row = blockIdx.x;
    const int64_t seq = row / Tq, t = row - seq * Tq;
    const int64_t p = seq_len ? seq_len[seq] - 1 : pos0 + t;
    const int64_t n = min(num_complete_blocks(p, r), nb_max);
    const float *s = scores + row * ld;
    int32_t *out = blk_idx + row * K;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    if (n <= K) {
        for (int i = tid; i < K; i += kNT) out[i] = i < n ? i : -1;
        if (tid == 0) n_sel[row] = static_cast<int32_t>(n);
        return;
    }

    uint32_t k[VPT];
    if (RESIDENT) load_keys<VPT>(s, n, 0, lane, wave, k);

    // ---- 1. histogram of key bits 31..20
    for (int i = tid; i < kBins; i += kNT) sh.hist[i] = 0;
    if (tid == 0) sh.cand_n = 0;
    __syncthreads();
    for (int64_t base = 0; base < n; base += TILE) {
        if (!RESIDENT) load_keys<VPT>(s, n, base, lane, wave, k);
#pragma unroll
        for (int q = 0; q < VPT; ++q)
            if (k[q]) atomicAdd(&sh.hist[k[q] >> 20], 1u);
    }
    __syncthreads();
    find_digit<kBins / kNT>(sh.hist, kBins, static_cast<uint32_t>(K), sh, tid, lane, wave);
    const uint32_t bin = sh.sel_bin;
    uint32_t krem = static_cast<uint32_t>(K) - sh.sel_above;
    const uint32_t nbin = sh.hist[bin];
    const bool in_lds = nbin <= kCap;
    __syncthreads();  // every thread has read the histogram before it is reused

    // ---- 2. gather the threshold bin, resolve the low 20 bits
    if (in_lds) {
        for (int64_t base = 0; base < n; base += TILE) {
            if (!RESIDENT) load_keys<VPT>(s, n, base, lane, wave, k);
#pragma unroll
            for (int q = 0; q < VPT; ++q) {
                if ((k[q] >> 20) == bin) {
                    const uint32_t slot = atomicAdd(&sh.cand_n, 1u);
                    sh.ckey[slot] = k[q];
                }
            }
        }
        __syncthreads();
    }
    uint32_t prefix = bin << 20, mask = 0xFFF00000u;
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = 10 - 10 * pass;
        uint32_t *h = sh.hist;  // reuse: 1024 bins
        for (int i = tid; i < 1024; i += kNT) h[i] = 0;
        __syncthreads();
        if (in_lds) {
            for (uint32_t j = tid; j < nbin; j += kNT) {
                const uint32_t key = sh.ckey[j];
                if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 1023u], 1u);
            }
        } else {
            for (int64_t base = 0; base < n; base += TILE) {
                if (!RESIDENT) load_keys<VPT>(s, n, base, lane, wave, k);
#pragma unroll
                for (int q = 0; q < VPT; ++q)
                    if ((k[q] & mask) == prefix) atomicAdd(&h[(k[q] >> shift) & 1023u], 1u);
            }
        }
        __syncthreads();
        find_digit<1>(h, 1024, krem, sh, tid, lane, wave);
        prefix |= sh.sel_bin << shift;
        mask |= 1023u << shift;
        krem -= sh.sel_above;
        __syncthreads();
    }
    const uint32_t thr = prefix;   // key of the K-th largest
    const uint32_t quota = krem;   // keys equal to thr that are taken

    // ---- 3. ordered compaction.  Per 256-key slice j the wave scans packed
    // (eq << 16 | gt) counts (a tile holds at most 32,768 keys, so neither
    // half overflows); a first sweep only totals them per wave, the second
    // recomputes the scans and writes, so no per-slice state is kept.
    uint32_t gt_all = 0, eq_all = 0;  // over earlier tiles
    for (int64_t base = 0; base < n; base += TILE) {
        if (!RESIDENT) load_keys<VPT>(s, n, base, lane, wave, k);
        auto slice_counts = [&](int j) -> uint32_t {
            uint32_t gt = 0, eq = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                gt += k[4 * j + c] > thr;
                eq += k[4 * j + c] == thr;
            }
            return (eq << 16) | gt;
        };
        auto wave_incl = [&](uint32_t x) -> uint32_t {
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t y = __shfl_up(x, off, kWave);
                if (lane >= off) x += y;
            }
            return x;
        };
        uint32_t wave_run = 0;
#pragma unroll
        for (int j = 0; j < VPT / 4; ++j) wave_run += __shfl(wave_incl(slice_counts(j)), kWave - 1, kWave);
        if (lane == 0) sh.wsum[wave] = wave_run;
        __syncthreads();
        uint32_t run = 0, tile_total = 0;
        for (int w = 0; w < kNW; ++w) {
            const uint32_t tw = sh.wsum[w];
            if (w < wave) run += tw;
            tile_total += tw;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < VPT / 4; ++j) {
            const uint32_t v = slice_counts(j);
            const uint32_t x = wave_incl(v);
            const uint32_t b0 = run + x - v;
            run += __shfl(x, kWave - 1, kWave);
            uint32_t gt_before = gt_all + (b0 & 0xFFFFu);
            uint32_t eq_before = eq_all + (b0 >> 16);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int q = 4 * j + c;
                const bool gt = k[q] > thr, eq = k[q] == thr;
                const uint32_t pos = gt_before + (eq_before < quota ? eq_before : quota);
                if ((gt || (eq && eq_before < quota)) && pos < static_cast<uint32_t>(K))
                    out[pos] = static_cast<int32_t>(elem_index<VPT>(base, wave, lane, q));
                gt_before += gt;
                eq_before += eq;
            }
        }
        gt_all += tile_total & 0xFFFFu;
        eq_all += tile_total >> 16;
    }
    if (tid == 0) n_sel[row] = K;
}

hipError_t launch_topk(const float *scores, int B, int64_t Tq, int64_t ld, int64_t pos0,
                       const int64_t *seq_len, int64_t nb_max, int r, int K, int32_t *blk_idx,
                       int32_t *n_sel, hipStream_t s) {
    const int64_t rows = static_cast<int64_t>(B) * Tq;
    if (rows == 0) return hipSuccess;
    // the longest row any query of the call can have
    const int64_t nmax = seq_len ? nb_max
                                 : min(num_complete_blocks(pos0 + Tq - 1, r), nb_max);
    const dim3 grid(static_cast<uint32_t>(rows));
    if (nmax <= 32 * kNT)
        hipLaunchKernelGGL((topk_kernel<32, true>), grid, dim3(kNT), 0, s, scores, Tq, ld, pos0,
                           seq_len, nb_max, r, K, blk_idx, n_sel);
    else
        hipLaunchKernelGGL((topk_kernel<16, false>), grid, dim3(kNT), 0, s, scores, Tq, ld, pos0,
                           seq_len, nb_max, r, K, blk_idx, n_sel);
    return hipGetLastError();
}

}  // namespace qsa
