// A3 + A4 fused for prefill: block scores and exact top-K selection without a
// score matrix in HBM (chlience section 6: every query scores its fully formed
// micro-blocks and keeps at most 512 of them).
//
// A workgroup (4 waves) owns 32 consecutive queries; wave w owns queries
// 8w .. 8w+7 as two MFMA row tiles of 4 queries x 4 heads.  The workgroup
// streams the pooled keys of every block the tile can see through LDS in
// tiles of 64 blocks and scores them with v_mfma_f32_16x16x32_bf16 (the same
// arithmetic, bit for bit, as qsa_index_scores).  It then makes two passes:
//   pass 1: each query keeps a buffer of 960 order-preserving score keys in
//     LDS, split into 16 slices of 60 owned by the 16 lanes that score its
//     blocks.  A key enters its lane's slice only if it beats the query's
//     current threshold (one masked LDS store, no cross-lane bookkeeping);
//     when a slice could overflow during the next tile, the owning wave
//     reduces the query's buffer to its K largest keys (radix select with
//     8-bit digits on an LDS histogram), 32 per slice, and raises the
//     threshold to the K-th of them.  After the last tile the same select
//     gives the exact K-th largest key T of the whole row and the number of
//     keys equal to T that are taken;
//   pass 2: the blocks are scored again and every block with key > T, plus
//     the first (lowest-index) blocks with key == T up to that number, is
//     written out.  Tiles and lanes run in block order, so the output is
//     ascending without a sort.
// A query with nc <= K takes every complete block.
#include "qsa_internal.h"

namespace qsa {

constexpr int kFQ = 32;      // queries per workgroup
constexpr int kFBT = 64;     // blocks per pooled-key tile
constexpr int kFRow = 272;   // LDS row stride of one pooled key (256 B + 16 B pad)
constexpr int kFCap = 960;   // buffered keys per query: 16 lane slices of 60
constexpr int kFSlice = 60;  // keys per lane slice
constexpr int kFMaxK = 512;  // largest budget: 32 kept keys per slice

struct FusedShared {
    unsigned char kt[2][kFBT * kFRow];  // double-buffered pooled-key tile
    uint32_t buf[kFQ][kFCap];
    uint32_t hist[4][256];              // per-wave radix histogram
};

// Orders this wave's LDS accesses (they complete in issue order; the fence
// keeps the compiler from moving them across the point).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// accesses, not for global loads in flight (a __syncthreads() fence would
// also drain the pooled-key prefetch).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// The K-th largest of the n (K <= n <= kFCap) keys in buf, by an MSB-first
// radix select with 8-bit digits over the wave's LDS histogram; also returns
// how many keys exceed it.  Keys are read into registers (lane l holds
// buf[l + 64*i]; missing slots hold 0, below every valid key).
constexpr int kFPer = (kFCap + 63) / 64;

__device__ __forceinline__ void wave_kth(const uint32_t *buf, uint32_t n, uint32_t K, int lane,
                                         uint32_t *hist, uint32_t (&key)[kFPer], uint32_t &T,
                                         uint32_t &gt) {
#pragma unroll
    for (int i = 0; i < kFPer; ++i) {
        const uint32_t j = lane + 64 * i;
        key[i] = j < n ? buf[j] : 0u;
    }
    uint32_t prefix = 0, mask = 0, krem = K;
#pragma unroll 1
    for (int d = 3; d >= 0; --d) {
        const int shift = 8 * d;
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < kFPer; ++i)
            if (key[i] && (key[i] & mask) == prefix)
                atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
        wave_lds_sync();
        // lane l owns digits 255-4l .. 252-4l, scanned from the top
        uint32_t c[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = hist[255 - 4 * lane - i];
            local += c[i];
        }
        uint32_t incl = local;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        const uint32_t before = incl - local;
        uint32_t digit = 0, above = 0;
        const bool mine = before < krem && krem <= incl;
        if (mine) {
            uint32_t acc = before;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (acc < krem && krem <= acc + c[i]) {
                    digit = 255u - 4u * lane - i;
                    above = acc;
                }
                acc += c[i];
            }
        }
        const int src = __ffsll(static_cast<long long>(__ballot(mine))) - 1;
        digit = __shfl(digit, src, kWave);
        above = __shfl(above, src, kWave);
        prefix |= digit << shift;
        mask |= 255u << shift;
        krem -= above;
    }
    T = prefix;
    gt = K - krem;
}

// Shrink a query's buffer to its K largest keys (ties at the K-th key are
// interchangeable: only key values are kept), laid out kk = ceil(K/16) per
// lane slice with the rest of each slice zeroed, and return the new
// threshold.
__device__ __forceinline__ uint32_t wave_compact(uint32_t *buf, uint32_t K, uint32_t kk,
                                                 int lane, uint32_t *hist) {
    uint32_t key[kFPer], T, gt;
    wave_kth(buf, kFCap, K, lane, hist, key, T, gt);
    const uint32_t quota = K - gt;
    // keep key > T, and `quota` keys equal to T (in lane-major order)
    uint32_t eq_local = 0, gt_local = 0;
#pragma unroll
    for (int i = 0; i < kFPer; ++i) {
        eq_local += key[i] == T;
        gt_local += key[i] > T;
    }
    uint32_t eq_incl = eq_local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(eq_incl, off, kWave);
        if (lane >= off) eq_incl += y;
    }
    const uint32_t eq_before = eq_incl - eq_local;
    const uint32_t eq_keep = eq_before >= quota ? 0u
                             : (quota - eq_before < eq_local ? quota - eq_before : eq_local);
    const uint32_t keep_local = gt_local + eq_keep;
    uint32_t keep_incl = keep_local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(keep_incl, off, kWave);
        if (lane >= off) keep_incl += y;
    }
    uint32_t r = keep_incl - keep_local;  // rank of this lane's first kept key
    uint32_t eq_left = eq_keep;
    wave_lds_sync();  // every lane has its keys before any write
#pragma unroll
    for (int i = 0; i < kFPer; ++i) {
        const uint32_t j = lane + 64 * i;
        if (j < kFCap) buf[j] = 0u;
    }
#pragma unroll
    for (int i = 0; i < kFPer; ++i) {
        const bool k = key[i] > T || (key[i] == T && eq_left > 0);
        eq_left -= key[i] == T && eq_left > 0;
        if (k) {
            buf[(r / kk) * kFSlice + (r % kk)] = key[i];
            ++r;
        }
    }
    wave_lds_sync();
    return T;
}

// State of one MFMA row tile (4 queries x 4 heads) of a wave.  Lane group g4
// holds the counters of query 4*rt + g4 of the wave, equal across its 16
// lanes.  Block indices are 32-bit (the cache holds fewer than 2^24 blocks).
struct RowTile {
    bf16x8 qf[4];     // A fragments, 4 k-steps
    uint32_t nc;      // complete blocks of this lane group's query (0: none)
    uint32_t cnt;     // pass 1: keys in this lane's slice (per lane)
    uint32_t thr;     // pass 1: accept keys above; pass 2: the K-th key T
    uint32_t quota;   // pass 2: keys equal to T to take
    uint32_t outpos;  // pass 2: blocks written
    uint32_t eqseen;  // pass 2: keys equal to T met
};

__device__ __forceinline__ void rowtile_init(RowTile &R, const uint16_t *__restrict__ q_idx,
                                             int64_t Tq, int64_t pos0, int64_t nb_max,
                                             int64_t qbase, int n, int g4) {
    const int64_t tq = qbase + (n >> 2);
    const bool ok = tq < Tq;
    const uint16_t *src = q_idx + (ok ? tq : 0) * (kIdxHeads * kIdxDim) + (n & 3) * kIdxDim;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        R.qf[s] = as_bf16x8(ok ? *reinterpret_cast<const uint4 *>(src + 32 * s + 8 * g4)
                               : make_uint4(0, 0, 0, 0));
    const int64_t tout = qbase + g4;
    R.nc = tout < Tq ? static_cast<uint32_t>(min(num_complete_blocks(pos0 + tout, kBlock), nb_max))
                     : 0u;
    R.cnt = R.thr = R.quota = R.outpos = R.eqseen = 0;
}

// The lane group's 16 bits of a wave ballot, and the bits below lane n.
__device__ __forceinline__ uint32_t group_bits(uint64_t m, int g4) {
    return static_cast<uint32_t>(m >> (16 * g4)) & 0xFFFFu;
}

// Feed 16 scored blocks of one row tile to pass 1 (buffer) or pass 2 (emit).
// Pass 2 fast path: a key can matter only if it reaches the query's final
// threshold; the ordered-output bookkeeping runs only when some lane of the
// wave has such a key (about K of them per query over the whole row).
template <int MODE>
__device__ __forceinline__ void rowtile_feed(RowTile &R, f32x4 acc, uint32_t blk, int pass,
                                             uint32_t *bufq, int32_t *out_row, uint32_t Ku,
                                             int n, int g4) {
    const uint32_t key = score_key(combine_heads<MODE>(acc));
    const bool valid = blk < R.nc;
    const uint32_t below = (1u << n) - 1u;
    if (pass == 0) {
        // lane n appends to its own slice: no cross-lane bookkeeping
        if (valid && key > R.thr) bufq[n * kFSlice + R.cnt++] = key;
    } else {
        const bool cand = valid && key >= R.thr;
        const uint64_t mc = __ballot(cand);
        if (mc) {
            const bool eq = cand && key == R.thr;
            const uint32_t ge = group_bits(__ballot(eq), g4);
            const bool take = (cand && key > R.thr) || (eq && R.eqseen + __popc(ge & below) < R.quota);
            const uint32_t gt_ = group_bits(__ballot(take), g4);
            const uint32_t pos = R.outpos + __popc(gt_ & below);
            if (take && pos < Ku) out_row[pos] = static_cast<int32_t>(blk);
            R.outpos += __popc(gt_);
            R.eqseen += __popc(ge);
        }
    }
}

struct CountThr {
    uint32_t a, b;
};

// Exact K-th key of each query of the row tile from its buffer: returns
// (T, quota) for the lane group's query.
__device__ __forceinline__ CountThr rowtile_finalize(uint32_t nc,
                                                     uint32_t (*buf)[kFCap], int qrow0,
                                                     uint32_t Ku, int lane, int g4,
                                                     uint32_t *hist) {
    CountThr out{0u, 0u};
#pragma unroll 1
    for (int g = 0; g < 4; ++g) {
        const uint32_t nc_g = __shfl(nc, 16 * g, kWave);
        uint32_t T = 0, qu = 0;
        if (nc_g > Ku) {
            uint32_t key[kFPer], gt;
            wave_kth(buf[qrow0 + g], kFCap, Ku, lane, hist, key, T, gt);  // empty slots are 0
            qu = Ku - gt;
        }
        if (g4 == g) out = CountThr{T, qu};  // nc <= K: T = 0 takes every valid block
    }
    return out;
}

// A tile adds at most 4 keys to a lane's slice: shrink the buffers of
// queries with a slice that could overflow during the next tile.  Returns the
// lane's (count, threshold).
__device__ __forceinline__ CountThr rowtile_shrink(uint32_t cnt, uint32_t thr,
                                                   uint32_t (*buf)[kFCap], int qrow0,
                                                   uint32_t Ku, int lane, int g4,
                                                   uint32_t *hist) {
    CountThr out{cnt, thr};
    const uint64_t full = __ballot(cnt > kFSlice - 4);
    if (full == 0) return out;  // usual case: one ballot
#pragma unroll 1
    for (int g = 0; g < 4; ++g) {
        if (group_bits(full, g) == 0) continue;
        const uint32_t kk = (Ku + 15) / 16;
        const uint32_t T = wave_compact(buf[qrow0 + g], Ku, kk, lane, hist);
        if (g4 == g) {
            // slice n now holds min(kk, K - n*kk) keys
            const uint32_t n = lane & 15, first = n * kk;
            out = CountThr{first >= Ku ? 0u : (Ku - first < kk ? Ku - first : kk), T};
        }
    }
    return out;
}

// One pooled-key row slice (64 bytes) per thread; rows past the cache are
// clamped to the last one (their scores are masked by blk < nc), so the
// loads are branch-free and the compiler can count them in flight.
__device__ __forceinline__ void fetch_slice(const uint16_t *__restrict__ kbar, uint32_t nb_max,
                                            uint32_t tile, int bl, int part, uint4 &a, uint4 &b,
                                            uint4 &c, uint4 &d) {
    uint32_t bb = tile * kFBT + bl;
    bb = bb < nb_max ? bb : nb_max - 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(kbar) + (bb * (kIdxDim / 8) + part * 4);
    a = src[0];
    b = src[1];
    c = src[2];
    d = src[3];
}

// One 64-block tile: publish the prefetched slice into LDS buffer (tile & 1),
// refill the register slot two tiles ahead, then score 4 sub-tiles x 2 row
// tiles as 8 independent MFMA chains before the epilogues.
template <int MODE>
__device__ __forceinline__ void fused_tile(FusedShared &sh, const uint16_t *__restrict__ kbar,
                                           uint32_t nb_max, uint32_t tile, int pass, uint4 &a,
                                           uint4 &b, uint4 &c, uint4 &d, RowTile &R0,
                                           RowTile &R1, int32_t *out0, int32_t *out1,
                                           int wave, int lane, int bl, int part, uint32_t Ku) {
    const int n = lane & 15, g4 = lane >> 4;
    unsigned char *kt = sh.kt[tile & 1];
    {
        uint4 *dst = reinterpret_cast<uint4 *>(kt + bl * kFRow + part * 64);
        dst[0] = a;
        dst[1] = b;
        dst[2] = c;
        dst[3] = d;
    }
    fetch_slice(kbar, nb_max, tile + 2, bl, part, a, b, c, d);  // refill two tiles ahead
    // one barrier per tile: the buffer written here was last read two tiles
    // ago, before the previous barrier
    lds_barrier();
    bf16x8 kf[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            kf[j][s] = as_bf16x8(*reinterpret_cast<const uint4 *>(
                kt + (16 * j + n) * kFRow + 64 * s + 16 * g4));
    f32x4 acc0[4], acc1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc0[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc0[j] = mfma_bf16_16x16x32(R0.qf[s], kf[j][s], acc0[j]);
            acc1[j] = mfma_bf16_16x16x32(R1.qf[s], kf[j][s], acc1[j]);
        }
    const uint32_t b0 = tile * kFBT;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t blk = b0 + 16 * j + n;
        rowtile_feed<MODE>(R0, acc0[j], blk, pass, sh.buf[8 * wave + g4], out0, Ku, n, g4);
        rowtile_feed<MODE>(R1, acc1[j], blk, pass, sh.buf[8 * wave + 4 + g4], out1, Ku, n, g4);
    }
    if (pass == 0) {
        const CountThr s0 =
            rowtile_shrink(R0.cnt, R0.thr, sh.buf, 8 * wave, Ku, lane, g4, sh.hist[wave]);
        R0.cnt = s0.a;
        R0.thr = s0.b;
        const CountThr s1 =
            rowtile_shrink(R1.cnt, R1.thr, sh.buf, 8 * wave + 4, Ku, lane, g4, sh.hist[wave]);
        R1.cnt = s1.a;
        R1.thr = s1.b;
    }
}

// The 160 KB of LDS allow one workgroup per CU, so the kernel may use the
// whole register file (one wave per SIMD).
template <int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
select_fused_kernel(const uint16_t *__restrict__ q_idx, const uint16_t *__restrict__ kbar,
                    int64_t Tq, int64_t pos0, int64_t nb_max, int K,
                    int32_t *__restrict__ blk_idx, int32_t *__restrict__ n_sel) {
    __shared__ FusedShared sh;
    const int qt = gridDim.x - 1 - blockIdx.x;  // longest rows first
    const int64_t t0 = static_cast<int64_t>(qt) * kFQ;
    const int64_t t_last = min(t0 + kFQ, Tq) - 1;
    const int64_t nc_hi = min(num_complete_blocks(pos0 + t_last, kBlock), nb_max);
    const uint32_t n_tiles = static_cast<uint32_t>((nc_hi + kFBT - 1) / kFBT);
    const uint32_t nbm = static_cast<uint32_t>(nb_max);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g4 = lane >> 4;
    const uint32_t Ku = static_cast<uint32_t>(K);
    const int bl = tid >> 2, part = tid & 3;

    // empty buffer slots hold 0 (below every valid key)
    for (int i = tid; i < kFQ * kFCap; i += 256) (&sh.buf[0][0])[i] = 0u;
    RowTile R0, R1;
    rowtile_init(R0, q_idx, Tq, pos0, nb_max, t0 + 8 * wave, n, g4);
    rowtile_init(R1, q_idx, Tq, pos0, nb_max, t0 + 8 * wave + 4, n, g4);
    // output rows of the lane group's queries (clamped for queries past Tq,
    // which never emit: their nc is 0)
    const int64_t tq0 = t0 + 8 * wave + g4, tq1 = tq0 + 4;
    int32_t *out0 = blk_idx + (tq0 < Tq ? tq0 : 0) * K;
    int32_t *out1 = blk_idx + (tq1 < Tq ? tq1 : 0) * K;

    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) {
            const CountThr f0 =
                rowtile_finalize(R0.nc, sh.buf, 8 * wave, Ku, lane, g4, sh.hist[wave]);
            R0.thr = f0.a;
            R0.quota = f0.b;
            const CountThr f1 =
                rowtile_finalize(R1.nc, sh.buf, 8 * wave + 4, Ku, lane, g4, sh.hist[wave]);
            R1.thr = f1.a;
            R1.quota = f1.b;
        }
        // two register slots, each refilled two tiles ahead
        uint4 a0, b0, c0, d0, a1, b1, c1, d1;
        fetch_slice(kbar, nbm, 0, bl, part, a0, b0, c0, d0);
        fetch_slice(kbar, nbm, 1, bl, part, a1, b1, c1, d1);
        for (uint32_t tile = 0; tile < n_tiles; tile += 2) {
            fused_tile<MODE>(sh, kbar, nbm, tile, pass, a0, b0, c0, d0, R0, R1, out0, out1,
                             wave, lane, bl, part, Ku);
            if (tile + 1 < n_tiles)
                fused_tile<MODE>(sh, kbar, nbm, tile + 1, pass, a1, b1, c1, d1, R0, R1, out0,
                                 out1, wave, lane, bl, part, Ku);
        }
        __syncthreads();
    }
    // counts and -1 padding
    if (tq0 < Tq) {
        const int ns = static_cast<int>(R0.nc < Ku ? R0.nc : Ku);
        for (int i = ns + n; i < K; i += 16) out0[i] = -1;
        if (n == 0) n_sel[tq0] = ns;
    }
    if (tq1 < Tq) {
        const int ns = static_cast<int>(R1.nc < Ku ? R1.nc : Ku);
        for (int i = ns + n; i < K; i += 16) out1[i] = -1;
        if (n == 0) n_sel[tq1] = ns;
    }
}

hipError_t launch_select_fused(const uint16_t *q_idx, const uint16_t *kbar, int64_t Tq,
                               int64_t pos0, int64_t nb_max, int mode, int K, int32_t *blk_idx,
                               int32_t *n_sel, hipStream_t s) {
    if (Tq == 0) return hipSuccess;
    const dim3 grid(static_cast<uint32_t>((Tq + kFQ - 1) / kFQ));
    if (mode == 0)
        hipLaunchKernelGGL(select_fused_kernel<0>, grid, dim3(256), 0, s, q_idx, kbar, Tq, pos0,
                           nb_max, K, blk_idx, n_sel);
    else
        hipLaunchKernelGGL(select_fused_kernel<1>, grid, dim3(256), 0, s, q_idx, kbar, Tq, pos0,
                           nb_max, K, blk_idx, n_sel);
    return hipGetLastError();
}

}  // namespace qsa
