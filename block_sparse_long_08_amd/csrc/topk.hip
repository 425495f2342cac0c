// A4: per-query top-K block selection (chlience section 6: at most 512
// complete blocks per query, chosen by indexer score).
//
// Every pass runs one workgroup per (row, segment).  A segment of up to
// NT*VPT keys is held in registers: wave w owns a contiguous run of 64*VPT
// keys and lane l holds 4 consecutive keys of every 256-key slice, so one
// float4 load per slice is coalesced and "earlier in the row" is (wave,
// slice, lane, element) order.  Finding the K-th largest key T:
//   1. histogram of key bits 31..20 in LDS -> the bin B holding rank K and
//      the count above it;
//   2. each wave appends the keys of bin B it holds to a private LDS list
//      (ballot + mbcnt, no shared counter); one wave then resolves bits
//      19..0 by two 10-bit histograms over those lists.  If a list overflows
//      (a crowded bin), the same two passes run block-wide over the
//      registers instead;
//   3. selection: every key > T, and the first `quota` keys equal to T (the
//      lowest indices win ties).  Output slots come from ballots of the
//      selection predicate, giving ascending index order without sorting.
// A row longer than one segment is reduced first: each segment emits its
// own top-K (key and index, ascending), and the global top-K is the top-K of
// those lists, because an element among the K best of the row is among the
// K best of its segment.  The order (score desc, index asc) is kept exactly.
// Many long rows at once take the streaming kernel below instead.
#include "qsa_internal.h"

namespace qsa {

constexpr int kBins = 4096;                // first digit: key bits 31..20
constexpr int kWaveCap = 256;              // bin-B keys one wave may list
constexpr uint32_t kMinKey = 0x00100000u;  // smaller keys: empty slots (0) and NaNs only
constexpr int kSegBig = 32768;             // 1024 threads x 32 keys
constexpr int kSegSmall = 4096;            // 256 threads x 16 keys
constexpr int kSegMid = 8192;              // 256 threads x 32 keys
constexpr int kStreamMin = 12288;          // shorter rows stay register-resident

struct TopkArgs {
    const float *scores;     // source 0: fp32 score rows
    int64_t ld;              //   row stride (multiple of 4)
    const uint32_t *ckey;    // source 1: candidate keys of the previous pass
    const int32_t *cidx;     //   and their block indices
    int64_t cin_ld;          //   row stride of the candidate lists
    uint32_t *okey;          // destination 1: this pass's candidate lists
    int32_t *oidx;
    int64_t cout_ld;
    int32_t *blk_idx;        // destination 0: [rows][K] ascending, -1 padded
    int32_t *n_sel;          //   [rows]
    int64_t Tq, pos0, nb_max;
    const int64_t *seq_len;  // decode form: row b at position seq_len[b] - nq
    int nq;
    int r, K;
    int nprev;               // passes before this one (source 1)
    int64_t prev_seg[4];     // their segment lengths
    const uint32_t *gmax;    // streaming pass: largest key of each 16-block group, or null
    int64_t gld;             //   its row stride
};

template <int NT>
struct TopkSmem {
    static constexpr int NW = NT / kWave;
    // Copies of the first-digit histogram (lane l counts into copy
    // l % NREP).  More copies spread the atomics of a wave over more
    // addresses but cost LDS and zeroing; one copy measured best overall.
    static constexpr int NREP = 1;
    uint32_t hist[kBins * NREP];
    uint32_t cand[NW][kWaveCap];
    uint32_t wcnt[NW];
    uint32_t wtot[NW];
    uint32_t fd_bin, fd_above, total;
    uint32_t thr, quota, eqcnt;
};

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Set bits of m in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    return x;
}

// Rank search over NBINS counts held in LDS (bin NBINS-1 is the largest
// digit), each stored as NREP consecutive partial counts.  Thread t owns PER
// consecutive digits, descending from NBINS-1-PER*t.  Finds the digit holding
// rank krem (1-based, counted from the top) and the count above it; the
// total count goes to sh.total.  SKIP0: bin 0 holds empty slots and is not
// counted.
template <int NT, int NBINS, int NREP, bool SKIP0>
__device__ __forceinline__ void block_find(const uint32_t *h, uint32_t krem, TopkSmem<NT> &sh,
                                           int tid, int lane, int wave) {
    constexpr int PER = NBINS / NT;
    static_assert(PER >= 1 && NBINS % NT == 0, "bins per thread");
    static_assert((PER * NREP) % 4 == 0 || PER * NREP < 4, "vector reads");
    const int base = NBINS - PER * (tid + 1);
    uint32_t w[PER * NREP];
    if constexpr ((PER * NREP) % 4 == 0) {
#pragma unroll
        for (int v = 0; v < PER * NREP / 4; ++v) {
            const uint4 q = *reinterpret_cast<const uint4 *>(h + base * NREP + 4 * v);
            w[4 * v + 0] = q.x;
            w[4 * v + 1] = q.y;
            w[4 * v + 2] = q.z;
            w[4 * v + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int v = 0; v < PER * NREP; ++v) w[v] = h[base * NREP + v];
    }
    uint32_t c[PER];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int d = base + PER - 1 - i;
        uint32_t x = 0;
#pragma unroll
        for (int r = 0; r < NREP; ++r) x += w[(PER - 1 - i) * NREP + r];
        c[i] = (SKIP0 && d == 0) ? 0u : x;
        local += c[i];
    }
    const uint32_t x = wave_incl_scan(local, lane);
    if (lane == kWave - 1) sh.wtot[wave] = x;
    block_sync();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int wv = 0; wv < TopkSmem<NT>::NW; ++wv) {
        const uint32_t t = sh.wtot[wv];
        before += wv < wave ? t : 0u;
        total += t;
    }
    const uint32_t incl = x + before;
    uint32_t acc = incl - local;
    if (acc < krem && krem <= incl) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (acc < krem && krem <= acc + c[i]) {
                sh.fd_bin = static_cast<uint32_t>(base + PER - 1 - i);
                sh.fd_above = acc;
            }
            acc += c[i];
        }
    }
    if (tid == 0) sh.total = total;
    block_sync();
}

// The same search by one wave over 64 * PER bins (PER a multiple of 4);
// returns the digit, the count above it, its own count and the total count
// (wave-uniform; with total < krem the digit is 0 and the rest undefined).
template <int PER>
__device__ __forceinline__ void wave_find(const uint32_t *h, uint32_t krem, int lane,
                                          uint32_t &digit, uint32_t &above, uint32_t &cnt,
                                          uint32_t &total) {
    static_assert(PER % 4 == 0, "vector reads");
    constexpr int NB = 64 * PER;
    const int base = NB - PER * (lane + 1);
    uint32_t c[PER];
#pragma unroll
    for (int v = 0; v < PER / 4; ++v) {
        const uint4 q = *reinterpret_cast<const uint4 *>(h + base + 4 * v);
        c[PER - 1 - 4 * v] = q.x;
        c[PER - 2 - 4 * v] = q.y;
        c[PER - 3 - 4 * v] = q.z;
        c[PER - 4 - 4 * v] = q.w;
    }
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) local += c[i];
    const uint32_t incl = wave_incl_scan(local, lane);
    uint32_t acc = incl - local;
    const bool mine = acc < krem && krem <= incl;
    uint32_t d = 0, ab = 0, cn = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (acc < krem && krem <= acc + c[i]) {
            d = static_cast<uint32_t>(base + PER - 1 - i);
            ab = acc;
            cn = c[i];
        }
        acc += c[i];
    }
    const uint64_t m = __ballot(mine);
    const int src = m ? static_cast<int>(__builtin_ctzll(m)) : 0;
    digit = __shfl(d, src, kWave);
    above = __shfl(ab, src, kWave);
    cnt = __shfl(cn, src, kWave);
    total = static_cast<uint32_t>(__shfl(static_cast<int>(incl), kWave - 1, kWave));
}

__device__ __forceinline__ void wave_find1024(const uint32_t *h, uint32_t krem, int lane,
                                              uint32_t &digit, uint32_t &above, uint32_t &cnt) {
    uint32_t total;
    wave_find<16>(h, krem, lane, digit, above, cnt, total);
}

// Writes one selected element (block index idx) to output slot pos.
template <int DST>
__device__ __forceinline__ void emit_one(const TopkArgs &a, int64_t obase, uint32_t pos,
                                         int32_t idx, uint32_t key) {
    if (DST == 0) {
        a.blk_idx[obase + pos] = idx;
    } else {
        a.okey[obase + pos] = key;
        a.oidx[obase + pos] = idx;
    }
}

__device__ __forceinline__ int32_t pick(const int4 &v, int c) {
    return c == 0 ? v.x : (c == 1 ? v.y : (c == 2 ? v.z : v.w));
}

// SRC 0: keys from fp32 score rows; SRC 1: candidate lists of a previous
// pass.  DST 0: final ascending block indices; DST 1: this segment's top-K
// as a candidate list (K entries, unused ones key 0 / index -1).
template <int NT, int VPT, int SRC, int DST>
__global__ void __launch_bounds__(NT) topk_pass(TopkArgs a) {
    constexpr int NW = NT / kWave;
    constexpr int SEG = NT * VPT;
    constexpr int NSL = VPT / 4;  // 256-key slices per wave
    __shared__ TopkSmem<NT> sh;

    const int64_t row = blockIdx.x;
    const int seg = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t sq = row / a.Tq;
    const int64_t p = a.seq_len ? a.seq_len[sq] - a.nq : a.pos0 + (row - sq * a.Tq);
    const int64_t n_row = min(num_complete_blocks(p, a.r), a.nb_max);
    const uint32_t K = static_cast<uint32_t>(a.K);

    if (n_row <= a.K) {  // every complete block is selected
        if (DST == 0) {
            int32_t *out = a.blk_idx + row * a.K;
            for (int i = tid; i < a.K; i += NT) out[i] = i < n_row ? i : -1;
            if (tid == 0) a.n_sel[row] = static_cast<int32_t>(n_row);
        }
        return;
    }
    // entries of this row at this pass's input
    int64_t n_in = n_row;
    if (SRC == 1)
        for (int i = 0; i < a.nprev; ++i) n_in = (n_in + a.prev_seg[i] - 1) / a.prev_seg[i] * a.K;
    const int64_t seg_base = static_cast<int64_t>(seg) * SEG;
    const int m = static_cast<int>(max(int64_t(0), min(n_in - seg_base, int64_t(SEG))));
    const int w0 = wave * 64 * VPT;

    // ---- load keys (slots past the segment get key 0)
    uint32_t k[VPT];
    if (w0 < m) {
        if (SRC == 0) {
            const float *s = a.scores + row * a.ld + seg_base;
#pragma unroll
            for (int j = 0; j < NSL; ++j) {
                const int i = w0 + 256 * j + 4 * lane;
                const float4 v = *reinterpret_cast<const float4 *>(s + (i < m ? i : 0));
                k[4 * j + 0] = i + 0 < m ? score_key(v.x) : 0u;
                k[4 * j + 1] = i + 1 < m ? score_key(v.y) : 0u;
                k[4 * j + 2] = i + 2 < m ? score_key(v.z) : 0u;
                k[4 * j + 3] = i + 3 < m ? score_key(v.w) : 0u;
            }
        } else {
            const uint32_t *s = a.ckey + row * a.cin_ld + seg_base;
#pragma unroll
            for (int j = 0; j < NSL; ++j) {
                const int i = w0 + 256 * j + 4 * lane;
                const uint4 v = *reinterpret_cast<const uint4 *>(s + (i < m ? i : 0));
                k[4 * j + 0] = i + 0 < m ? v.x : 0u;
                k[4 * j + 1] = i + 1 < m ? v.y : 0u;
                k[4 * j + 2] = i + 2 < m ? v.z : 0u;
                k[4 * j + 3] = i + 3 < m ? v.w : 0u;
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < VPT; ++q) k[q] = 0u;
    }
    // slices of this wave that hold keys (wave-uniform)
    const int nsl = w0 < m ? min(NSL, (m - w0 + 255) >> 8) : 0;

    bool all = m <= a.K;  // the whole segment is selected
    uint32_t thr = kMinKey, quota = 0, eqcnt = 0;
    if (!all) {
        // ---- 1. first digit
        constexpr int NREP = TopkSmem<NT>::NREP;
        for (int i = tid; i < kBins * NREP / 4; i += NT)
            reinterpret_cast<uint4 *>(sh.hist)[i] = make_uint4(0u, 0u, 0u, 0u);
        block_sync();
        const int rep = lane % NREP;
#pragma unroll
        for (int j = 0; j < NSL; ++j) {
            if (j < nsl) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    atomicAdd(&sh.hist[(k[4 * j + c] >> 20) * NREP + rep], 1u);
            }
        }
        block_sync();
        block_find<NT, kBins, NREP, true>(sh.hist, K, sh, tid, lane, wave);
        if (sh.total <= K) {
            all = true;  // the segment holds at most K keys
        } else {
            const uint32_t bin = sh.fd_bin;
            uint32_t krem = K - sh.fd_above;
            // ---- 2. list the keys of the threshold bin, per wave
            uint32_t wc = 0;  // wave-uniform
#pragma unroll
            for (int j = 0; j < NSL; ++j) {
                if (j < nsl) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t key = k[4 * j + c];
                        const bool hit = (key >> 20) == bin;
                        const uint64_t bm = __ballot(hit);
                        if (bm) {
                            const uint32_t slot = wc + lanes_below(bm);
                            if (hit && slot < kWaveCap) sh.cand[wave][slot] = key;
                            wc += static_cast<uint32_t>(__popcll(bm));
                        }
                    }
                }
            }
            if (lane == 0) sh.wcnt[wave] = wc;
            block_sync();  // lists written; every thread is done with hist
            bool overflow = false;
#pragma unroll
            for (int w = 0; w < NW; ++w) overflow |= sh.wcnt[w] > kWaveCap;
            uint32_t prefix = bin << 20, mask = 0xFFF00000u;
            if (!overflow) {
                if (wave == 0) {
                    uint32_t *h = sh.hist;
                    uint32_t cnt = 0;
                    for (int pass = 0; pass < 2; ++pass) {
                        const int shift = 10 - 10 * pass;
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            *reinterpret_cast<uint4 *>(h + 16 * lane + 4 * v) =
                                make_uint4(0u, 0u, 0u, 0u);
                        wave_lds_sync();
                        // LPL lanes walk each list, all lists at once
                        constexpr int LPL = kWave / NW;
                        const int lw = lane / LPL, li0 = lane % LPL;
                        const int nw = static_cast<int>(sh.wcnt[lw]);
                        for (int i0 = li0; i0 < nw; i0 += 8 * LPL) {
#pragma unroll
                            for (int u = 0; u < 8; ++u) {
                                const int i = i0 + u * LPL;
                                if (i < nw) {
                                    const uint32_t key = sh.cand[lw][i];
                                    if ((key & mask) == prefix)
                                        atomicAdd(&h[(key >> shift) & 1023u], 1u);
                                }
                            }
                        }
                        wave_lds_sync();
                        uint32_t d, ab;
                        wave_find1024(h, krem, lane, d, ab, cnt);
                        prefix |= d << shift;
                        mask |= 1023u << shift;
                        krem -= ab;
                        wave_lds_sync();
                    }
                    if (lane == 0) {
                        sh.thr = prefix;
                        sh.quota = krem;
                        sh.eqcnt = cnt;
                    }
                }
                block_sync();
            } else {
                // crowded bin: resolve block-wide over the registers
                uint32_t cnt = 0;
                for (int pass = 0; pass < 2; ++pass) {
                    const int shift = 10 - 10 * pass;
                    for (int i = tid; i < 1024; i += NT) sh.hist[i] = 0u;
                    block_sync();
#pragma unroll
                    for (int j = 0; j < NSL; ++j) {
                        if (j < nsl) {
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const uint32_t key = k[4 * j + c];
                                if ((key & mask) == prefix)
                                    atomicAdd(&sh.hist[(key >> shift) & 1023u], 1u);
                            }
                        }
                    }
                    block_sync();
                    block_find<NT, 1024, 1, false>(sh.hist, krem, sh, tid, lane, wave);
                    const uint32_t d = sh.fd_bin;
                    prefix |= d << shift;
                    mask |= 1023u << shift;
                    krem -= sh.fd_above;
                    cnt = sh.hist[d];
                    block_sync();
                }
                if (tid == 0) {
                    sh.thr = prefix;
                    sh.quota = krem;
                    sh.eqcnt = cnt;
                }
                block_sync();
            }
            thr = sh.thr;
            quota = sh.quota;
            eqcnt = sh.eqcnt;
        }
    }
    if (all) {
        thr = kMinKey;
        quota = 0;
        eqcnt = 0;
    }
    const bool split = quota != eqcnt;  // only some of the keys equal to T are taken

    // ---- 3. selection in index order.  First sweep: per-wave counts.
    uint32_t gt_w = 0, eq_w = 0;
#pragma unroll
    for (int j = 0; j < NSL; ++j) {
        if (j < nsl) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t key = k[4 * j + c];
                if (!split) {
                    gt_w += static_cast<uint32_t>(__popcll(__ballot(key >= thr)));
                } else {
                    gt_w += static_cast<uint32_t>(__popcll(__ballot(key > thr)));
                    eq_w += static_cast<uint32_t>(__popcll(__ballot(key == thr)));
                }
            }
        }
    }
    if (lane == 0) sh.wtot[wave] = (eq_w << 16) | gt_w;  // each <= 64*VPT <= 2048
    block_sync();
    uint32_t gt_off = 0, eq_off = 0, gt_all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t t = sh.wtot[w];
        if (w < wave) {
            gt_off += t & 0xFFFFu;
            eq_off += t >> 16;
        }
        gt_all += t & 0xFFFFu;
    }
    const uint32_t nsel = split ? K : gt_all;  // selected in this segment

    // second sweep: emit.  The block indices of candidate-list entries are
    // fetched for all slices at once, before any store depends on them.
    const int64_t obase = DST == 0 ? row * a.K : row * a.cout_ld + static_cast<int64_t>(seg) * a.K;
    int4 cidx[SRC == 1 ? NSL : 1];
    if (SRC == 1) {
        const int32_t *src = a.cidx + row * a.cin_ld + seg_base;
#pragma unroll
        for (int j = 0; j < NSL; ++j) {
            const int i = w0 + 256 * j + 4 * lane;
            cidx[j] = j < nsl ? *reinterpret_cast<const int4 *>(src + (i < m ? i : 0))
                              : make_int4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < NSL; ++j) {
        if (j < nsl) {
            const int lbase = static_cast<int>(seg_base) + w0 + 256 * j + 4 * lane;
            if (!split) {
                uint64_t bm[4];
                uint32_t rk = gt_off;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    bm[c] = __ballot(k[4 * j + c] >= thr);
                    rk += lanes_below(bm[c]);
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (k[4 * j + c] >= thr) {
                        const int32_t idx = SRC == 0 ? lbase + c : pick(cidx[SRC == 1 ? j : 0], c);
                        emit_one<DST>(a, obase, rk, idx, k[4 * j + c]);
                        ++rk;
                    }
                    gt_off += static_cast<uint32_t>(__popcll(bm[c]));
                }
            } else {
                uint64_t bg[4], be[4];
                uint32_t gr = gt_off, er = eq_off;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    bg[c] = __ballot(k[4 * j + c] > thr);
                    be[c] = __ballot(k[4 * j + c] == thr);
                    gr += lanes_below(bg[c]);
                    er += lanes_below(be[c]);
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t key = k[4 * j + c];
                    const bool gt = key > thr, eq = key == thr;
                    if (gt || (eq && er < quota)) {
                        const int32_t idx = SRC == 0 ? lbase + c : pick(cidx[SRC == 1 ? j : 0], c);
                        emit_one<DST>(a, obase, gr + min(er, quota), idx, key);
                    }
                    gr += gt;
                    er += eq;
                    gt_off += static_cast<uint32_t>(__popcll(bg[c]));
                    eq_off += static_cast<uint32_t>(__popcll(be[c]));
                }
            }
        }
    }
    // pad the unused slots
    if (DST == 0) {
        for (uint32_t i = nsel + tid; i < K; i += NT) a.blk_idx[obase + i] = -1;
        if (tid == 0) a.n_sel[row] = static_cast<int32_t>(nsel);
    } else {
        for (uint32_t i = nsel + tid; i < K; i += NT) {
            a.okey[obase + i] = 0u;
            a.oidx[obase + i] = -1;
        }
    }
}

// ------------------------------------------------------------ streaming --
// One workgroup (256 or 1024 threads) per row; the row is read twice from HBM/L2
// and never held whole, so rows of any length take one launch and few
// registers (several rows in flight per CU).  Wave w owns the contiguous
// range [w*chunk, (w+1)*chunk) of the row (chunk a multiple of 256), lane l
// the 4 consecutive keys 4l..4l+3 of every 256-key slice.
//   pass 1: per-lane maxima of 4 key groups (slices j mod 4).  If at least K
//           groups hold keys, the K-th largest maximum has K keys at or
//           above it: its bin's lower edge is a floor under T;
//   pass 2: keys at or above the floor (typically 1-3 K) are appended, in
//           index order, to per-wave LDS lists with their positions;
//   then the exact T and tie quota come from the lists (first digit block-
//   wide, low 20 bits by one wave), and the lists are emitted in order.
// If a list overflows (a crowded floor bin, e.g. heavy ties), the threshold
// is found by three streaming radix passes instead and the row is emitted by
// two more streaming passes; the result is the same.
// With the scores' 16-block group maxima at hand (gmax), pass 1 reads those
// instead of the row, and pass 2 loads only the groups whose maximum reaches
// the floor (the others hold no key at or above it): each lane takes 8
// consecutive groups of its wave's range at a time, a wave prefix sum over
// the lanes' survivor counts places the surviving groups in order in an LDS
// list, and their keys are loaded 64 groups at a time (4 steps of 16 groups,
// 4 lanes per group, all loads issued before the ordered appends), so lane
// order stays block order.
template <int NT>
struct StreamSmem {
    static constexpr int CAP = NT >= 1024 ? 256 : 512;  // list entries per wave
    TopkSmem<NT> t;  // histogram, counts, results
    uint32_t ckey[NT / kWave][CAP];
    int32_t cidx[NT / kWave][CAP];
    uint32_t eqtot[NT / kWave];
    int32_t glist[NT / kWave][kWave];  // surviving 16-block groups of one batch
};

__device__ __forceinline__ void stream_keys(const float *s, int i, int lim, uint32_t (&kk)[4]) {
    const float4 v = *reinterpret_cast<const float4 *>(s + (i < lim ? i : 0));
    kk[0] = i + 0 < lim ? score_key(v.x) : 0u;
    kk[1] = i + 1 < lim ? score_key(v.y) : 0u;
    kk[2] = i + 2 < lim ? score_key(v.z) : 0u;
    kk[3] = i + 3 < lim ? score_key(v.w) : 0u;
}

__device__ __forceinline__ uint32_t max4(const uint32_t (&kk)[4]) {
    return max(max(kk[0], kk[1]), max(kk[2], kk[3]));
}

// Ordered append of the keys of one slice that satisfy key >= floor.
__device__ __forceinline__ void stream_append(const uint32_t (&kk)[4], uint32_t floor_key,
                                              int pos0, uint32_t cap, uint32_t &wc, uint32_t *lk,
                                              int32_t *li) {
    uint64_t b[4];
    uint32_t rk = wc;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        b[c] = __ballot(kk[c] >= floor_key);
        rk += lanes_below(b[c]);
    }
    if ((b[0] | b[1] | b[2] | b[3]) == 0) return;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (kk[c] >= floor_key) {
            if (rk < cap) {
                lk[rk] = kk[c];
                li[rk] = pos0 + c;
            }
            ++rk;
        }
        wc += static_cast<uint32_t>(__popcll(b[c]));
    }
}

template <int kStNT>
__device__ __forceinline__ void stream_row(const TopkArgs &a, int64_t row,
                                           StreamSmem<kStNT> &sm) {
    constexpr int kStNW = kStNT / kWave;
    constexpr uint32_t kCap = StreamSmem<kStNT>::CAP;
    TopkSmem<kStNT> &sh = sm.t;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t sq = row / a.Tq;
    const int64_t p = a.seq_len ? a.seq_len[sq] - a.nq : a.pos0 + (row - sq * a.Tq);
    const int64_t n_row = min(num_complete_blocks(p, a.r), a.nb_max);
    const uint32_t K = static_cast<uint32_t>(a.K);
    int32_t *out = a.blk_idx + row * a.K;
    if (n_row <= a.K) {  // every complete block is selected
        for (int i = tid; i < a.K; i += kStNT) out[i] = i < n_row ? i : -1;
        if (tid == 0) a.n_sel[row] = static_cast<int32_t>(n_row);
        return;
    }
    const int n = static_cast<int>(n_row);
    const float *s = a.scores + row * a.ld;
    const int chunk = ((n + kStNW - 1) / kStNW + 255) / 256 * 256;
    const int w0 = min(n, wave * chunk), w1 = min(n, w0 + chunk);
    const int l4 = 4 * lane;

    // ---- pass 1: group maxima -> floor
    // (the precomputed 16-block maxima when they are at least as many groups
    // as the per-lane maxima below, 4 per thread: a looser floor could
    // overflow the lists)
    const uint32_t *gm =
        a.gmax && ((n + 15) >> 4) >= 4 * kStNT ? a.gmax + row * a.gld : nullptr;
    if (gm) {
        // the precomputed maxima of the ceil(n / 16) groups holding blocks
        for (int i = tid; i < kBins; i += kStNT) sh.hist[i] = 0u;
        block_sync();
        const int ng = (n + 15) >> 4;
        for (int i = tid; i < ng; i += kStNT) atomicAdd(&sh.hist[gm[i] >> 20], 1u);
    } else {
        uint32_t lm[4] = {0u, 0u, 0u, 0u};
        for (int base = w0; base < w1; base += 1024) {
            uint32_t kk[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) stream_keys(s, base + 256 * u + l4, w1, kk[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) lm[u] = max(lm[u], max4(kk[u]));
        }
        for (int i = tid; i < kBins; i += kStNT) sh.hist[i] = 0u;
        block_sync();
#pragma unroll
        for (int u = 0; u < 4; ++u) atomicAdd(&sh.hist[lm[u] >> 20], 1u);
    }
    block_sync();
    block_find<kStNT, kBins, 1, true>(sh.hist, K, sh, tid, lane, wave);
    const uint32_t floor_key = sh.total >= K ? sh.fd_bin << 20 : kMinKey;

    // ---- pass 2: candidate lists
    uint32_t wc = 0;  // wave-uniform
    if (gm) {
        constexpr int kQ = 8;  // consecutive groups per lane and round
        const int g_lo = w0 >> 4, g_hi = (w1 + 15) >> 4;
        int32_t *gl = sm.glist[wave];
        for (int r0 = g_lo; r0 < g_hi; r0 += kWave * kQ) {
            const int gb = r0 + kQ * lane;
            uint32_t gk[kQ];
            uint32_t cnt = 0;
#pragma unroll
            for (int q = 0; q < kQ; ++q) {
                gk[q] = gb + q < g_hi ? gm[gb + q] : 0u;
                cnt += gk[q] >= floor_key ? 1u : 0u;
            }
            const uint32_t incl = wave_incl_scan(cnt, lane);
            const uint32_t total = static_cast<uint32_t>(__shfl(static_cast<int>(incl), kWave - 1));
            for (uint32_t p0 = 0; p0 < total; p0 += kWave) {
                // the survivors at list positions p0 .. p0+63
                uint32_t pos = incl - cnt;
#pragma unroll
                for (int q = 0; q < kQ; ++q) {
                    if (gk[q] >= floor_key) {
                        if (pos >= p0 && pos < p0 + kWave) gl[pos - p0] = gb + q;
                        ++pos;
                    }
                }
                wave_lds_sync();
                const int np = static_cast<int>(min(total - p0, static_cast<uint32_t>(kWave)));
                uint32_t kk[4][4];
                int ii[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int sidx = 16 * u + (lane >> 2);
                    ii[u] = 0;
#pragma unroll
                    for (int c = 0; c < 4; ++c) kk[u][c] = 0u;
                    if (sidx < np) {
                        ii[u] = 16 * gl[sidx] + 4 * (lane & 3);
                        stream_keys(s, ii[u], w1, kk[u]);
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (16 * u < np)
                        stream_append(kk[u], floor_key, ii[u], kCap, wc, sm.ckey[wave],
                                      sm.cidx[wave]);
                wave_lds_sync();  // the list is rewritten by the next piece
            }
        }
    } else {
        for (int base = w0; base < w1; base += 1024) {
            uint32_t kk[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) stream_keys(s, base + 256 * u + l4, w1, kk[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                stream_append(kk[u], floor_key, base + 256 * u + l4, kCap, wc, sm.ckey[wave],
                              sm.cidx[wave]);
        }
    }
    if (lane == 0) sh.wcnt[wave] = wc;
    block_sync();
    bool overflow = false;
    uint32_t total_c = 0;
#pragma unroll
    for (int w = 0; w < kStNW; ++w) {
        overflow |= sh.wcnt[w] > kCap;
        total_c += sh.wcnt[w];
    }

    uint32_t thr, quota = 0, eqcnt = 0;
    if (!overflow) {
        if (total_c <= K) {
            thr = floor_key;  // exactly K keys reach the floor: take them all
        } else {
            // first digit over the lists
            block_sync();  // every thread has read wcnt / the floor histogram
            for (int i = tid; i < kBins; i += kStNT) sh.hist[i] = 0u;
            block_sync();
            for (int i = lane; i < static_cast<int>(wc); i += kWave)
                atomicAdd(&sh.hist[sm.ckey[wave][i] >> 20], 1u);
            block_sync();
            block_find<kStNT, kBins, 1, true>(sh.hist, K, sh, tid, lane, wave);
            const uint32_t bin = sh.fd_bin;
            uint32_t krem = K - sh.fd_above;
            block_sync();  // done with the histogram
            if (wave == 0) {
                uint32_t *h = sh.hist;
                uint32_t prefix = bin << 20, mask = 0xFFF00000u, cnt = 0;
                for (int pass = 0; pass < 2; ++pass) {
                    const int shift = 10 - 10 * pass;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        *reinterpret_cast<uint4 *>(h + 16 * lane + 4 * v) = make_uint4(0u, 0u, 0u, 0u);
                    wave_lds_sync();
                    constexpr int LPL = kWave / kStNW;
                    const int lw = lane / LPL, li0 = lane % LPL;
                    const int nw = static_cast<int>(sh.wcnt[lw]);
                    for (int i0 = li0; i0 < nw; i0 += 8 * LPL) {
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int i = i0 + u * LPL;
                            if (i < nw) {
                                const uint32_t key = sm.ckey[lw][i];
                                if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 1023u], 1u);
                            }
                        }
                    }
                    wave_lds_sync();
                    uint32_t d, ab;
                    wave_find1024(h, krem, lane, d, ab, cnt);
                    prefix |= d << shift;
                    mask |= 1023u << shift;
                    krem -= ab;
                    wave_lds_sync();
                }
                if (lane == 0) {
                    sh.thr = prefix;
                    sh.quota = krem;
                    sh.eqcnt = cnt;
                }
            }
            block_sync();
            thr = sh.thr;
            quota = sh.quota;
            eqcnt = sh.eqcnt;
        }
        // ---- emission from the lists, in index order
        const bool split = quota != eqcnt;
        uint32_t gt_w = 0, eq_w = 0;
        for (int i0 = 0; i0 < static_cast<int>(wc); i0 += kWave) {
            const int i = i0 + lane;
            const uint32_t key = i < static_cast<int>(wc) ? sm.ckey[wave][i] : 0u;
            if (!split) {
                gt_w += static_cast<uint32_t>(__popcll(__ballot(key >= thr)));
            } else {
                gt_w += static_cast<uint32_t>(__popcll(__ballot(key > thr)));
                eq_w += static_cast<uint32_t>(__popcll(__ballot(key == thr)));
            }
        }
        if (lane == 0) {
            sh.wtot[wave] = gt_w;
            sm.eqtot[wave] = eq_w;
        }
        block_sync();
        uint32_t gt_off = 0, eq_off = 0, gt_all = 0;
#pragma unroll
        for (int w = 0; w < kStNW; ++w) {
            const uint32_t g = sh.wtot[w], e = sm.eqtot[w];
            if (w < wave) {
                gt_off += g;
                eq_off += e;
            }
            gt_all += g;
        }
        for (int i0 = 0; i0 < static_cast<int>(wc); i0 += kWave) {
            const int i = i0 + lane;
            const bool ok = i < static_cast<int>(wc);
            const uint32_t key = ok ? sm.ckey[wave][i] : 0u;
            const int32_t idx = ok ? sm.cidx[wave][i] : 0;
            if (!split) {
                const bool sel = key >= thr;
                const uint64_t b = __ballot(sel);
                if (sel) out[gt_off + lanes_below(b)] = idx;
                gt_off += static_cast<uint32_t>(__popcll(b));
            } else {
                const bool gt = key > thr, eq = key == thr;
                const uint64_t bg = __ballot(gt), be = __ballot(eq);
                const uint32_t gr = gt_off + lanes_below(bg), er = eq_off + lanes_below(be);
                if (gt || (eq && er < quota)) out[gr + min(er, quota)] = idx;
                gt_off += static_cast<uint32_t>(__popcll(bg));
                eq_off += static_cast<uint32_t>(__popcll(be));
            }
        }
        const uint32_t nsel = split ? K : gt_all;
        for (uint32_t i = nsel + tid; i < K; i += kStNT) out[i] = -1;
        if (tid == 0) a.n_sel[row] = static_cast<int32_t>(nsel);
        return;
    }

    // ---- crowded rows: streaming radix select, then streaming emission
    uint32_t prefix = 0, mask = 0, krem = K;
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
        const uint32_t dmask = pass == 0 ? 4095u : 1023u;
        block_sync();
        for (int i = tid; i < kBins; i += kStNT) sh.hist[i] = 0u;
        block_sync();
        for (int base = w0; base < w1; base += 256) {
            uint32_t kk[4];
            stream_keys(s, base + l4, w1, kk);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (kk[c] != 0u && (kk[c] & mask) == prefix)
                    atomicAdd(&sh.hist[(kk[c] >> shift) & dmask], 1u);
        }
        block_sync();
        if (pass == 0)
            block_find<kStNT, kBins, 1, true>(sh.hist, krem, sh, tid, lane, wave);
        else
            block_find<kStNT, 1024, 1, false>(sh.hist, krem, sh, tid, lane, wave);
        const uint32_t d = sh.fd_bin;
        krem -= sh.fd_above;
        prefix |= d << shift;
        mask |= dmask << shift;
        eqcnt = sh.hist[d];
    }
    thr = prefix;
    quota = krem;
    const bool split = quota != eqcnt;
    uint32_t gt_w = 0, eq_w = 0;
    for (int base = w0; base < w1; base += 256) {
        uint32_t kk[4];
        stream_keys(s, base + l4, w1, kk);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            gt_w += static_cast<uint32_t>(__popcll(__ballot(split ? kk[c] > thr : kk[c] >= thr)));
            eq_w += static_cast<uint32_t>(__popcll(__ballot(split && kk[c] == thr)));
        }
    }
    block_sync();
    if (lane == 0) {
        sh.wtot[wave] = gt_w;
        sm.eqtot[wave] = eq_w;
    }
    block_sync();
    uint32_t gt_off = 0, eq_off = 0, gt_all = 0;
#pragma unroll
    for (int w = 0; w < kStNW; ++w) {
        const uint32_t g = sh.wtot[w], e = sm.eqtot[w];
        if (w < wave) {
            gt_off += g;
            eq_off += e;
        }
        gt_all += g;
    }
    for (int base = w0; base < w1; base += 256) {
        uint32_t kk[4];
        stream_keys(s, base + l4, w1, kk);
        uint64_t bg[4], be[4];
        uint32_t gr = gt_off, er = eq_off;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bg[c] = __ballot(split ? kk[c] > thr : kk[c] >= thr);
            be[c] = __ballot(split && kk[c] == thr);
            gr += lanes_below(bg[c]);
            er += lanes_below(be[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool gt = split ? kk[c] > thr : kk[c] >= thr;
            const bool eq = split && kk[c] == thr;
            if (gt || (eq && er < quota)) out[gr + min(er, quota)] = base + l4 + c;
            gr += gt;
            er += eq;
            gt_off += static_cast<uint32_t>(__popcll(bg[c]));
            eq_off += static_cast<uint32_t>(__popcll(be[c]));
        }
    }
    const uint32_t nsel = split ? K : gt_all;
    for (uint32_t i = nsel + tid; i < K; i += kStNT) out[i] = -1;
    if (tid == 0) a.n_sel[row] = static_cast<int32_t>(nsel);
}

template <int kStNT>
__global__ void __launch_bounds__(kStNT) topk_stream(TopkArgs a) {
    __shared__ StreamSmem<kStNT> sm;
    stream_row<kStNT>(a, blockIdx.x, sm);
}

// ------------------------------------------------- decode form, few rows --
// Few long rows (one query per sequence) with the group maxima the decode
// scan writes (the largest key of every 64 consecutive blocks):
//   filter (workgroup per 4,096-key segment of a row): the K-th largest group
//     maximum has at least K keys at or above it, so the lower edge of its
//     12-bit bin is a floor under the row's K-th largest key; the segment's
//     keys at or above the floor go, in index order, to the segment's slots
//     of a candidate list in the workspace (a row with fewer than K groups
//     keeps every key);
//   final (workgroup per row): the segments' lists are packed in LDS, the
//     exact K-th key and tie quota come from three histogram digits, and
//     the selection is emitted in index order.  A row whose lists exceed
//     the LDS capacity (short rows, heavy ties) runs the streaming
//     selection over its scores instead; the result is the same.
// Many workgroups share each row, so the row's keys are read once and at
// the full memory rate instead of by one workgroup per row.
constexpr int kDecSeg = 4096;       // keys per filter workgroup (256 threads x 16)
constexpr int kDecMaxSeg = 1024;    // segments per row (rows of up to 4M blocks)
constexpr int kDecListCap = 8192;   // candidates per row packed in LDS

struct DecTopkArgs {
    TopkArgs t;              // scores, ld, Tq = 1, seq_len, nb_max, r, K, outputs
    const uint32_t *gmax;    // [rows][gld] group maxima (keys)
    int64_t gld;
    uint32_t *lkey;          // [rows][lld] candidate keys, segment s at s * kDecSeg
    int32_t *lidx;           //   and block indices
    int64_t lld;
    uint32_t *lcnt;          // [rows][cld] candidates per segment
    int64_t cld;
};

__device__ __forceinline__ int64_t dec_row_blocks(const TopkArgs &a, int64_t row) {
    const int64_t p = a.seq_len[row] - a.nq;
    return min(num_complete_blocks(p, a.r), a.nb_max);
}

// Block-wide minimum and maximum (every thread gets both); uses wcnt/wtot.
template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t &lo, uint32_t &hi, TopkSmem<NT> &sh,
                                             int lane, int wave) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off)));
        hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off)));
    }
    if (lane == 0) {
        sh.wtot[wave] = lo;
        sh.wcnt[wave] = hi;
    }
    block_sync();
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        lo = min(lo, sh.wtot[w]);
        hi = max(hi, sh.wcnt[w]);
    }
}

// Bit length of x (0 for 0).
__device__ __forceinline__ int bit_len(uint32_t x) { return 32 - __clz(static_cast<int>(x)); }

__global__ void __launch_bounds__(256) topk_dec_filter(DecTopkArgs d) {
    constexpr int NT = 256;
    __shared__ TopkSmem<NT> sh;
    const TopkArgs &a = d.t;
    const int64_t row = blockIdx.y;
    const int seg = blockIdx.x;
    const int64_t n_row = dec_row_blocks(a, row);
    const uint32_t K = static_cast<uint32_t>(a.K);
    if (n_row <= a.K || static_cast<int64_t>(seg) * kDecSeg >= n_row) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = static_cast<int>(n_row);
    const float *srow = a.scores + row * a.ld;
    const int base = seg * kDecSeg + wave * 1024 + 4 * lane;
    uint32_t kk[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) stream_keys(srow, base + 256 * u, n, kk[u]);

    // Floor from the group maxima (the first 4,096 loaded with the keys):
    // 4,096 bins spanning [min, max] of the maxima; the K-th largest maximum
    // lies in bin b, so at least K keys are >= min + (b << shift).
    const int ngrp = (n + 63) >> 6;
    uint32_t floor_key = kMinKey;
    if (ngrp >= a.K) {
        const uint32_t *g = d.gmax + row * d.gld;
        uint32_t gv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int i = tid + NT * j;
            gv[j] = g[i < ngrp ? i : 0];
        }
        uint32_t lo = gv[0], hi = gv[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) {
            lo = min(lo, gv[j]);
            hi = max(hi, gv[j]);
        }
        for (int i = tid + 16 * NT; i < ngrp; i += NT) {
            lo = min(lo, g[i]);
            hi = max(hi, g[i]);
        }
        for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0u;
        block_minmax<NT>(lo, hi, sh, lane, wave);
        const int L = bit_len(hi - lo);
        const int shift = L > 12 ? L - 12 : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (tid + NT * j < ngrp) atomicAdd(&sh.hist[(gv[j] - lo) >> shift], 1u);
        for (int i = tid + 16 * NT; i < ngrp; i += NT)
            atomicAdd(&sh.hist[(g[i] - lo) >> shift], 1u);
        block_sync();
        block_find<NT, kBins, 1, false>(sh.hist, K, sh, tid, lane, wave);
        floor_key = max(lo + (sh.fd_bin << shift), kMinKey);
    }

    // ordered write of the keys at or above the floor
    uint32_t wc = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            wc += static_cast<uint32_t>(__popcll(__ballot(kk[u][c] >= floor_key)));
    if (lane == 0) sh.wcnt[wave] = wc;
    block_sync();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        off += w < wave ? sh.wcnt[w] : 0u;
        tot += sh.wcnt[w];
    }
    const int64_t obase = row * d.lld + static_cast<int64_t>(seg) * kDecSeg;
    uint32_t run = off;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        stream_append(kk[u], floor_key, base + 256 * u, 0xFFFFFFFFu, run, d.lkey + obase,
                      d.lidx + obase);
    if (tid == 0) d.lcnt[row * d.cld + seg] = tot;
}

struct DecFinalSmem {
    TopkSmem<1024> t;
    uint32_t ck[kDecListCap];
    int32_t ci[kDecListCap];
    uint32_t segoff[kDecMaxSeg + 1];
    uint32_t eqtot[16];
};

union DecFinalLds {
    DecFinalSmem f;
    StreamSmem<1024> st;
};

__global__ void __launch_bounds__(1024) topk_dec_final(DecTopkArgs d) {
    constexpr int NT = 1024, NW = NT / kWave;
    __shared__ DecFinalLds lds;
    DecFinalSmem &f = lds.f;
    TopkSmem<NT> &sh = f.t;
    const TopkArgs &a = d.t;
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n_row = dec_row_blocks(a, row);
    const uint32_t K = static_cast<uint32_t>(a.K);
    int32_t *out = a.blk_idx + row * a.K;
    if (n_row <= a.K) {  // every complete block is selected
        for (int i = tid; i < a.K; i += NT) out[i] = i < n_row ? i : -1;
        if (tid == 0) a.n_sel[row] = static_cast<int32_t>(n_row);
        return;
    }
    const int nseg = static_cast<int>((n_row + kDecSeg - 1) / kDecSeg);
    // The first 128 entries of segments wave + 16 q (q < 4) are loaded
    // before the counts are known (typical lists are shorter), so the lists
    // and their counts arrive in one round trip.
    uint32_t pk[4][2];
    int32_t pi[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int sidx = min(wave + NW * q, nseg - 1);
        const int64_t src = row * d.lld + static_cast<int64_t>(sidx) * kDecSeg;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            pk[q][u] = d.lkey[src + lane + kWave * u];
            pi[q][u] = d.lidx[src + lane + kWave * u];
        }
    }
    // exclusive prefix of the segment counts (wave 0)
    if (wave == 0) {
        uint32_t carry = 0;
        const uint32_t *cnt = d.lcnt + row * d.cld;
        for (int s0 = 0; s0 < nseg; s0 += kWave) {
            const int sidx = s0 + lane;
            const uint32_t c = sidx < nseg ? cnt[sidx] : 0u;
            const uint32_t incl = wave_incl_scan(c, lane);
            if (sidx < nseg) f.segoff[sidx] = carry + incl - c;
            carry += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0) f.segoff[nseg] = carry;
    }
    block_sync();
    const uint32_t total = f.segoff[nseg];
    if (total > static_cast<uint32_t>(kDecListCap)) {
        block_sync();  // segoff read by all before the union is reused
        stream_row<NT>(a, row, lds.st);
        return;
    }
    // pack the lists (index order) into LDS
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int sidx = wave + NW * q;
        if (sidx < nseg) {
            const uint32_t o = f.segoff[sidx], c = f.segoff[sidx + 1] - o;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t j = lane + kWave * u;
                if (j < c) {
                    f.ck[o + j] = pk[q][u];
                    f.ci[o + j] = pi[q][u];
                }
            }
        }
    }
    for (int sidx = wave; sidx < nseg; sidx += NW) {
        const uint32_t o = f.segoff[sidx], c = f.segoff[sidx + 1] - o;
        const int64_t src = row * d.lld + static_cast<int64_t>(sidx) * kDecSeg;
        const uint32_t j0 = sidx < 4 * NW ? 2 * kWave : 0u;  // the rest
        for (uint32_t j = j0 + lane; j < c; j += kWave) {
            f.ck[o + j] = d.lkey[src + j];
            f.ci[o + j] = d.lidx[src + j];
        }
    }
    for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0u;
    block_sync();

    uint32_t thr = 0, quota = 0, eqcnt = 0;
    bool split = false;
    if (total > K) {
        // Radix select on v = key - min over the list: digits of up to 12
        // bits from the top of the list's range down to bit 0 (two levels
        // for a range under 2^24), so the bins follow the data.
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
        for (uint32_t i = tid; i < total; i += NT) {
            lo = min(lo, f.ck[i]);
            hi = max(hi, f.ck[i]);
        }
        block_minmax<NT>(lo, hi, sh, lane, wave);
        const int L = bit_len(hi - lo);
        int s = L > 12 ? L - 12 : 0, s_prev = 32;
        uint32_t hp = 0, krem = K;  // hp: the resolved bits v >> s_prev
        for (;;) {
            const uint32_t dmask = (1u << (s_prev - s > 12 ? 12 : s_prev - s)) - 1u;
            for (uint32_t i = tid; i < total; i += NT) {
                const uint32_t v = f.ck[i] - lo;
                if (s_prev == 32 || (v >> s_prev) == hp)
                    atomicAdd(&sh.hist[(v >> s) & dmask], 1u);
            }
            block_sync();
            block_find<NT, kBins, 1, false>(sh.hist, krem, sh, tid, lane, wave);
            const uint32_t dg = sh.fd_bin;
            krem -= sh.fd_above;
            eqcnt = sh.hist[dg];
            hp = s_prev == 32 ? dg : (hp << (s_prev - s)) | dg;
            if (s == 0) break;
            s_prev = s;
            s = s > 12 ? s - 12 : 0;
            block_sync();  // every thread has read the histogram
            for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0u;
            block_sync();
        }
        thr = lo + hp;
        quota = krem;
        split = quota != eqcnt;
    }
    // emission: wave w takes the contiguous run [c0, c1) of the packed list
    const uint32_t chunk = (total + NW * kWave - 1) / (NW * kWave) * kWave;
    const uint32_t c0 = min(total, wave * chunk), c1 = min(total, c0 + chunk);
    uint32_t gt_w = 0, eq_w = 0;
    for (uint32_t i0 = c0; i0 < c1; i0 += kWave) {
        const uint32_t i = i0 + lane;
        const uint32_t key = i < c1 ? f.ck[i] : 0u;
        const bool gt = split ? key > thr : (i < c1 && key >= thr);
        gt_w += static_cast<uint32_t>(__popcll(__ballot(gt)));
        eq_w += static_cast<uint32_t>(__popcll(__ballot(split && key == thr)));
    }
    block_sync();  // every thread has read the histogram
    if (lane == 0) {
        sh.wtot[wave] = gt_w;
        f.eqtot[wave] = eq_w;
    }
    block_sync();
    uint32_t gt_off = 0, eq_off = 0, gt_all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t g = sh.wtot[w], e = f.eqtot[w];
        if (w < wave) {
            gt_off += g;
            eq_off += e;
        }
        gt_all += g;
    }
    for (uint32_t i0 = c0; i0 < c1; i0 += kWave) {
        const uint32_t i = i0 + lane;
        const bool ok = i < c1;
        const uint32_t key = ok ? f.ck[i] : 0u;
        const int32_t idx = ok ? f.ci[i] : 0;
        const bool gt = split ? key > thr : (ok && key >= thr);
        const bool eq = split && key == thr;
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        const uint32_t gr = gt_off + lanes_below(bg), er = eq_off + lanes_below(be);
        if (gt || (eq && er < quota)) out[gr + min(er, quota)] = idx;
        gt_off += static_cast<uint32_t>(__popcll(bg));
        eq_off += static_cast<uint32_t>(__popcll(be));
    }
    const uint32_t nsel = split ? K : gt_all;
    for (uint32_t i = nsel + tid; i < K; i += NT) out[i] = -1;
    if (tid == 0) a.n_sel[row] = static_cast<int32_t>(nsel);
}

// ----------------------------------------- prefill chunks, one wave per row --
// Rows of a prefill score chunk whose indexer also wrote the 16-block group
// maxima, for budgets K <= 512: one wave per row and no workgroup barriers,
// so four rows share a workgroup and 16 rows are in flight per CU.
//   floor: a key at or below the row's K-th largest key, the lower edge of
//     the digit holding rank K in a histogram of 256 bins spanning
//     [smallest, largest] group maximum, refined by a second histogram
//     inside that bin when it is crowded.  Rows of at least 3K/2 groups
//     take the histogram of the group maxima (K groups whose maximum reaches
//     the floor hold K keys at or above it); shorter rows take that of their
//     keys (keys below the smallest group maximum cannot be among the K
//     best once the row has K groups);
//   candidates: the keys at or above the floor, in index order, in a list
//     of up to 1,024 entries in LDS; the group form reads only the groups
//     whose maximum reaches the floor, 128 of them per round;
//   the exact K-th key and its tie quota by 8-bit digits over the list's
//     range, then emission in index order.
// A row with fewer than K groups, or whose list overflows, gets n_sel = -1
// and is finished by the streaming kernel in a second launch (topk_redo).
constexpr int kWvMaxK = 512;    // budgets this form takes
constexpr int kWvCap = 1024;    // candidates per row in LDS
constexpr int kWvBatch = 128;   // surviving groups loaded per round
constexpr int kWvBins = 256;
constexpr uint32_t kWvRefine = 64;  // a floor bin holding more is refined

struct __attribute__((aligned(16))) WaveRowSmem {
    uint32_t hist[kWvBins];
    int32_t glist[kWvBatch];
    uint32_t ckey[kWvCap];
    int32_t cidx[kWvCap];
};

__device__ __forceinline__ void wave_minmax(uint32_t &lo, uint32_t &hi) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        lo = min(lo, static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), off)));
        hi = max(hi, static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), off)));
    }
}

// Calls f(key) for the first cnt group-maximum keys g[0 .. cnt) (a row of
// the group-maximum array, padded to a multiple of 4).
template <class F>
__device__ __forceinline__ void visit_gmax(const uint32_t *g, int cnt, int lane, F f) {
    for (int base = 0; base < cnt; base += 1024) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + 256 * u + 4 * lane;
            v[u] = i < cnt ? *reinterpret_cast<const uint4 *>(g + i) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + 256 * u + 4 * lane;
            if (i + 0 < cnt) f(v[u].x);
            if (i + 1 < cnt) f(v[u].y);
            if (i + 2 < cnt) f(v[u].z);
            if (i + 3 < cnt) f(v[u].w);
        }
    }
}

// Calls f(key) for the keys of score row s[0 .. n).
template <class F>
__device__ __forceinline__ void visit_keys(const float *s, int n, int lane, F f) {
    for (int base = 0; base < n; base += 1024) {
        uint32_t kk[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) stream_keys(s, base + 256 * u + 4 * lane, n, kk[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (base + 256 * u + 4 * lane + c < n) f(kk[u][c]);
    }
}

// The floor: at least K of the keys the visitor yields are >= the returned
// key, and it is at or below the K-th largest of them.  The histogram spans
// [lo, hi]: keys below lo are not counted, keys above hi count in the top
// bin (hi need not be the largest key).  ok = false when fewer than K keys
// are >= lo (the floor is then undefined).
template <class V>
__device__ __forceinline__ uint32_t wave_floor(V visit, uint32_t lo, uint32_t hi, uint32_t K,
                                               uint32_t *hist, int lane, bool &ok) {
    constexpr uint32_t kTop = kWvBins - 1;
    const int L = bit_len(hi - lo);
    const int s1 = L > 8 ? L - 8 : 0;
    *reinterpret_cast<uint4 *>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_sync();
    visit([&](uint32_t k) {
        if (k >= lo) atomicAdd(&hist[min((k - lo) >> s1, kTop)], 1u);
    });
    wave_lds_sync();
    uint32_t d, above, cnt, total;
    wave_find<4>(hist, K, lane, d, above, cnt, total);
    ok = total >= K;
    uint32_t floor_key = lo + (d << s1);
    if (ok && s1 > 0 && cnt > kWvRefine) {
        // the keys of bin d, by the next 8 bits below its edge
        const int s2 = s1 > 8 ? s1 - 8 : 0;
        wave_lds_sync();  // every lane has read the histogram
        *reinterpret_cast<uint4 *>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
        wave_lds_sync();
        visit([&](uint32_t k) {
            if (k >= floor_key && min((k - lo) >> s1, kTop) == d)
                atomicAdd(&hist[min((k - floor_key) >> s2, kTop)], 1u);
        });
        wave_lds_sync();
        uint32_t d2, a2, c2, t2;
        wave_find<4>(hist, K - above, lane, d2, a2, c2, t2);
        floor_key += d2 << s2;
    }
    wave_lds_sync();
    return floor_key;
}

// The group maxima of one row: REG (rows of at most 2,048 groups) holds them
// in registers, group 256 u + 4 lane + c in g[4 u + c], read once; otherwise
// each pass reads them from memory.
template <bool REG>
struct GmaxRow {
    const uint32_t *gm;
    int ng;
    uint32_t g[REG ? 32 : 1];

    __device__ __forceinline__ void load(int lane) {
        if constexpr (REG) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = 256 * u + 4 * lane;
                const uint4 v =
                    i < ng ? *reinterpret_cast<const uint4 *>(gm + i) : make_uint4(0u, 0u, 0u, 0u);
                g[4 * u + 0] = i + 0 < ng ? v.x : 0u;
                g[4 * u + 1] = i + 1 < ng ? v.y : 0u;
                g[4 * u + 2] = i + 2 < ng ? v.z : 0u;
                g[4 * u + 3] = i + 3 < ng ? v.w : 0u;
            }
        }
    }
    template <class F>
    __device__ __forceinline__ void visit(int lane, F f) const {
        if constexpr (REG) {
#pragma unroll
            for (int q = 0; q < 32; ++q)
                if (256 * (q >> 2) + 4 * lane + (q & 3) < ng) f(g[q]);
        } else {
            visit_gmax(gm, ng, lane, f);
        }
    }
    // piece p: groups 1024 p + 256 u + 4 lane + c into gk[4 u + c] (0 past ng)
    __device__ __forceinline__ void piece(int p, int lane, uint32_t (&gk)[16]) const {
        if constexpr (REG) {
#pragma unroll
            for (int q = 0; q < 16; ++q) gk[q] = p == 0 ? g[q] : g[16 + q];
        } else {
            const int base = 1024 * p;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = base + 256 * u + 4 * lane;
                const uint4 v =
                    i < ng ? *reinterpret_cast<const uint4 *>(gm + i) : make_uint4(0u, 0u, 0u, 0u);
                gk[4 * u + 0] = i + 0 < ng ? v.x : 0u;
                gk[4 * u + 1] = i + 1 < ng ? v.y : 0u;
                gk[4 * u + 2] = i + 2 < ng ? v.z : 0u;
                gk[4 * u + 3] = i + 3 < ng ? v.w : 0u;
            }
        }
    }
};

// Candidates of one row: the keys >= the floor, in index order, appended to
// the wave's list (wc counts past the capacity).  Returns the floor.
template <bool REG>
__device__ __forceinline__ uint32_t wave_candidates(const TopkArgs &a, const float *s, int n,
                                                    GmaxRow<REG> &G, WaveRowSmem &sm, int lane,
                                                    uint32_t &wc) {
    const uint32_t K = static_cast<uint32_t>(a.K);
    const int ng = G.ng;
    G.load(lane);
    auto minmax_of = [&](auto visit, uint32_t &lo, uint32_t &hi) {
        lo = 0xFFFFFFFFu;
        hi = 0u;
        visit([&](uint32_t k) {
            lo = min(lo, k);
            hi = max(hi, k);
        });
        wave_minmax(lo, hi);
    };
    auto gvisit = [&](auto f) { G.visit(lane, f); };
    auto kvisit = [&](auto f) { visit_keys(s, n, lane, f); };
    wc = 0;
    bool ok;
    if (2 * ng < 3 * a.K) {
        // ---- row form: floor from the keys themselves, then the keys that
        // reach it.  The histogram spans the group maxima's range; with
        // fewer than K of the keys at or above the smallest maximum (rows of
        // few groups) it spans all the keys instead.
        uint32_t lo, hi;
        minmax_of(gvisit, lo, hi);
        uint32_t floor_key = wave_floor(kvisit, lo, hi, K, sm.hist, lane, ok);
        if (!ok) {
            minmax_of(kvisit, lo, hi);
            floor_key = wave_floor(kvisit, lo, hi, K, sm.hist, lane, ok);
        }
        for (int base = 0; base < n; base += 1024) {
            uint32_t kk[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) stream_keys(s, base + 256 * u + 4 * lane, n, kk[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                stream_append(kk[u], floor_key, base + 256 * u + 4 * lane, kWvCap, wc, sm.ckey,
                              sm.cidx);
        }
        wave_lds_sync();
        return floor_key;
    }
    // ---- group form: floor from the group maxima, then the groups that
    // reach it
    uint32_t floor_key;
    if constexpr (REG) {
        uint32_t lo, hi;
        minmax_of(gvisit, lo, hi);
        floor_key = wave_floor(gvisit, lo, hi, K, sm.hist, lane, ok);
    } else {
        // Long rows: the histogram's range comes from a sample, 256 groups
        // at each quarter of the row (one read instead of a pass over the
        // maxima), from about the 2K ng'/ng-th largest sampled maximum
        // (ng' = 1,024 sampled; the row's K-th largest maximum lies above it
        // unless the sample misleads) to the largest sampled one.  When
        // fewer than K maxima reach the low end, the exact range is taken.
        uint32_t smp[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = ((ng >> 2) * q & ~3) + 4 * lane;  // < ng: ng > 2,048
            const uint4 v = *reinterpret_cast<const uint4 *>(G.gm + i);
            smp[4 * q + 0] = v.x;
            smp[4 * q + 1] = v.y;
            smp[4 * q + 2] = v.z;
            smp[4 * q + 3] = v.w;
        }
        auto svisit = [&](auto f) {
#pragma unroll
            for (int q = 0; q < 16; ++q) f(smp[q]);
        };
        uint32_t lo, hi;
        minmax_of(svisit, lo, hi);
        const uint32_t ks = static_cast<uint32_t>(
            min(static_cast<int64_t>(1024), max(static_cast<int64_t>(1),
                                                2 * static_cast<int64_t>(K) * 1024 / ng)));
        lo = wave_floor(svisit, lo, hi, ks, sm.hist, lane, ok);
        floor_key = wave_floor(gvisit, lo, hi, K, sm.hist, lane, ok);
        if (!ok) {
            minmax_of(gvisit, lo, hi);
            floor_key = wave_floor(gvisit, lo, hi, K, sm.hist, lane, ok);
        }
    }
    uint32_t carry = 0;  // surviving groups listed, not yet loaded
    const int npieces = (ng + 1023) >> 10;
    for (int p = 0; p < npieces; ++p) {
        uint32_t gk[16];
        G.piece(p, lane, gk);
        const int base = 1024 * p;
        // survivors of this piece in (u, lane, c) order = index order
        const bool last = p + 1 >= npieces;
        uint32_t before[4];
        uint32_t tot = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t cu = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) cu += gk[4 * u + c] >= floor_key ? 1u : 0u;
            const uint32_t incl = wave_incl_scan(cu, lane);
            before[u] = tot + incl - cu;
            tot += static_cast<uint32_t>(__shfl(static_cast<int>(incl), kWave - 1));
        }
        // combined positions: the carried survivors of the last piece first
        // (already listed at 0 .. c0-1), then this piece's
        const uint32_t c0 = carry;
        const uint32_t all = c0 + tot;
        carry = 0;
        for (uint32_t w0 = 0; w0 < all; w0 += kWvBatch) {
            const bool full = w0 + kWvBatch <= all;
            // list the survivors at combined positions [w0, w0 + batch)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t pos = c0 + before[u];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (gk[4 * u + c] >= floor_key) {
                        if (pos >= w0 && pos < w0 + kWvBatch)
                            sm.glist[pos - w0] = base + 256 * u + 4 * lane + c;
                        ++pos;
                    }
                }
            }
            wave_lds_sync();
            if (!full && !last) {  // a partial round waits for the next piece
                carry = all - w0;
                break;
            }
            const int np = static_cast<int>(min(all - w0, static_cast<uint32_t>(kWvBatch)));
            uint32_t kk[8][4];
            int ii[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sidx = 16 * u + (lane >> 2);
                ii[u] = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) kk[u][c] = 0u;
                if (sidx < np) {
                    ii[u] = 16 * sm.glist[sidx] + 4 * (lane & 3);
                    stream_keys(s, ii[u], n, kk[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (16 * u < np)
                    stream_append(kk[u], floor_key, ii[u], kWvCap, wc, sm.ckey, sm.cidx);
            wave_lds_sync();  // the list is rewritten by the next round
        }
    }
    return floor_key;
}

__global__ void __launch_bounds__(256) topk_wave(TopkArgs a, int64_t rows) {
    __shared__ WaveRowSmem smem[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (row >= rows) return;
    WaveRowSmem &sm = smem[wave];
    const int64_t sq = row / a.Tq;
    const int64_t p = a.pos0 + (row - sq * a.Tq);
    const int64_t n_row = min(num_complete_blocks(p, a.r), a.nb_max);
    const uint32_t K = static_cast<uint32_t>(a.K);
    int32_t *out = a.blk_idx + row * a.K;
    if (n_row <= a.K) {  // every complete block is selected
        for (int i = lane; i < a.K; i += kWave) out[i] = i < n_row ? i : -1;
        if (lane == 0) a.n_sel[row] = static_cast<int32_t>(n_row);
        return;
    }
    const int n = static_cast<int>(n_row);
    const int ng = (n + 15) >> 4;
    const float *s = a.scores + row * a.ld;
    const uint32_t *gm = a.gmax + row * a.gld;
    uint32_t wc, lo;
    if (ng <= 2048) {
        GmaxRow<true> G{gm, ng, {}};
        lo = wave_candidates<true>(a, s, n, G, sm, lane, wc);
    } else {
        GmaxRow<false> G{gm, ng, {}};
        lo = wave_candidates<false>(a, s, n, G, sm, lane, wc);
    }
    if (wc > static_cast<uint32_t>(kWvCap)) {  // crowded: the streaming kernel takes it
        if (lane == 0) a.n_sel[row] = -1;
        return;
    }

    // ---- exact K-th key over the list (every entry >= lo), digits of up to
    // 8 bits from the top of the list's range
    uint32_t thr = lo, quota = 0, eqcnt = 0;
    bool split = false;
    if (wc > K) {
        uint32_t cmax = 0u;
        for (uint32_t i = lane; i < wc; i += kWave) cmax = max(cmax, sm.ckey[i]);
        uint32_t dummy = 0u;
        wave_minmax(dummy, cmax);
        const int L = bit_len(cmax - lo);
        int sh = L > 8 ? L - 8 : 0, sh_prev = 32;
        uint32_t hp = 0, krem = K;
        for (;;) {
            const uint32_t dmask = (1u << (sh_prev - sh > 8 ? 8 : sh_prev - sh)) - 1u;
            *reinterpret_cast<uint4 *>(sm.hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
            wave_lds_sync();
            for (uint32_t i = lane; i < wc; i += kWave) {
                const uint32_t v = sm.ckey[i] - lo;
                if (sh_prev == 32 || (v >> sh_prev) == hp) atomicAdd(&sm.hist[(v >> sh) & dmask], 1u);
            }
            wave_lds_sync();
            uint32_t dg, ab, cn, tt;
            wave_find<4>(sm.hist, krem, lane, dg, ab, cn, tt);
            krem -= ab;
            eqcnt = cn;
            hp = sh_prev == 32 ? dg : (hp << (sh_prev - sh)) | dg;
            wave_lds_sync();  // every lane has read the histogram
            if (sh == 0) break;
            sh_prev = sh;
            sh = sh > 8 ? sh - 8 : 0;
        }
        thr = lo + hp;
        quota = krem;
        split = quota != eqcnt;
    }
    // ---- emission in index order (the list is in index order)
    uint32_t gt_off = 0, eq_off = 0;
    for (uint32_t i0 = 0; i0 < wc; i0 += kWave) {
        const uint32_t i = i0 + lane;
        const bool ok = i < wc;
        const uint32_t key = ok ? sm.ckey[i] : 0u;
        const int32_t idx = ok ? sm.cidx[i] : 0;
        const bool gt = ok && (split ? key > thr : key >= thr);
        const bool eq = ok && split && key == thr;
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        const uint32_t gr = gt_off + lanes_below(bg), er = eq_off + lanes_below(be);
        if (gt || (eq && er < quota)) out[gr + min(er, quota)] = idx;
        gt_off += static_cast<uint32_t>(__popcll(bg));
        eq_off += static_cast<uint32_t>(__popcll(be));
    }
    const uint32_t nsel = split ? K : gt_off;
    for (uint32_t i = nsel + lane; i < K; i += kWave) out[i] = -1;
    if (lane == 0) a.n_sel[row] = static_cast<int32_t>(nsel);
}

// The rows topk_wave left (n_sel = -1), by the streaming kernel: each
// workgroup checks 64 consecutive rows and runs those in turn.
__global__ void __launch_bounds__(256) topk_redo(TopkArgs a, int64_t rows) {
    __shared__ StreamSmem<256> sm;
    __shared__ uint64_t flagged;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kWave;
    if (threadIdx.x < kWave) {
        const int64_t r = r0 + threadIdx.x;
        const uint64_t b = __ballot(r < rows && a.n_sel[r] == -1);
        if (threadIdx.x == 0) flagged = b;
    }
    block_sync();
    uint64_t m = flagged;
    while (m) {
        const int i = static_cast<int>(__builtin_ctzll(m));
        m &= m - 1;
        stream_row<256>(a, r0 + i, sm);
        block_sync();  // the next row rewrites the histogram and lists
    }
}

// ------------------------------------------------------------------ plan --
TopkPlan topk_plan(int64_t rows, int64_t nmax, int K) {
    TopkPlan pl{};
    // many long rows: one streaming pass per row, no workspace (1024
    // threads past one segment, 256 threads for rows of 12K..32K blocks).
    // Measured faster there than the register-resident and reduction
    // passes; slower for few rows (one workgroup streams a row at a
    // fraction of a CU's share of HBM) and for short rows.
    if (rows >= 256 && nmax > kStreamMin) {
        pl.stream = true;
        pl.stream_nt = nmax > kSegBig ? 1024 : 256;
        pl.final_entries = nmax;
        return pl;
    }
    int64_t e = nmax;
    while (pl.npass < 4) {
        // stop once one final pass can take the rows: always after a
        // reduction pass (a third launch costs more than a longer final
        // pass), else when the rows are many or short
        const bool fits = e <= kSegBig;
        if (fits && (rows >= 128 || pl.npass > 0 || e <= 8192)) break;
        const int64_t big_wgs = rows * ((e + kSegBig - 1) / kSegBig);
        const int64_t seg = (big_wgs < 512 && 4 * K <= kSegSmall) ? kSegSmall : kSegBig;
        const int64_t e2 = (e + seg - 1) / seg * K;
        if (e2 >= e) break;
        pl.seg[pl.npass] = seg;
        pl.entries[pl.npass] = e2;
        ++pl.npass;
        e = e2;
    }
    pl.final_entries = e;
    // ping-pong candidate buffers (keys, then indices); rows padded to 4 entries
    int64_t ea = 0, eb = 0;
    for (int i = 0; i < pl.npass; ++i) {
        const int64_t ld = (pl.entries[i] + 3) / 4 * 4;
        if (i % 2 == 0)
            ea = ea > ld ? ea : ld;
        else
            eb = eb > ld ? eb : ld;
    }
    pl.ld[0] = ea;
    pl.ld[1] = eb;
    pl.ws_bytes = static_cast<size_t>(rows) * static_cast<size_t>(ea + eb) * 8u;
    return pl;
}

hipError_t launch_topk(const float *scores, int B, int64_t Tq, int64_t ld, int64_t pos0,
                       const int64_t *seq_len, int64_t nb_max, int r, int K, int32_t *blk_idx,
                       int32_t *n_sel, void *ws, hipStream_t s, const uint32_t *gmax,
                       int64_t gld) {
    // decode form: one row per sequence, made for the first of its Tq queries
    const int64_t rows = seq_len ? static_cast<int64_t>(B) : static_cast<int64_t>(B) * Tq;
    if (rows == 0) return hipSuccess;
    // With many rows no plan needs workspace, so the kernel choice may follow
    // the longest row of this call (prefill form: the last query's) rather
    // than the cache size the workspace was sized for.
    int64_t nmax = nb_max;
    if (!seq_len && rows >= 256) nmax = min(num_complete_blocks(pos0 + Tq - 1, r), nb_max);
    const TopkPlan pl = topk_plan(rows, nmax, K);
    // prefill chunks with the group maxima: one wave per row, then the rows
    // it leaves (crowded lists) by the streaming kernel
    const bool wave_rows = gmax && !seq_len && rows >= 256 && K <= kWvMaxK;
    TopkArgs a{};
    a.scores = scores;
    a.ld = ld;
    a.blk_idx = blk_idx;
    a.n_sel = n_sel;
    a.Tq = seq_len ? 1 : Tq;
    a.nq = seq_len ? static_cast<int>(Tq) : 1;
    a.pos0 = pos0;
    a.nb_max = nb_max;
    a.seq_len = seq_len;
    a.r = r;
    a.K = K;
    if (wave_rows) {
        a.gmax = gmax;
        a.gld = gld;
        hipLaunchKernelGGL(topk_wave, dim3(static_cast<uint32_t>((rows + 3) / 4)), dim3(256), 0, s,
                           a, rows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(topk_redo, dim3(static_cast<uint32_t>((rows + kWave - 1) / kWave)),
                           dim3(256), 0, s, a, rows);
        return hipGetLastError();
    }
    if (pl.stream) {
        a.gmax = seq_len ? nullptr : gmax;
        a.gld = gld;
        // with the group maxima a row's passes are short: 256 threads, so
        // that more rows are in flight per CU
        if (pl.stream_nt == 1024 && !a.gmax)
            hipLaunchKernelGGL(topk_stream<1024>, dim3(static_cast<uint32_t>(rows)), dim3(1024), 0,
                               s, a);
        else
            hipLaunchKernelGGL(topk_stream<256>, dim3(static_cast<uint32_t>(rows)), dim3(256), 0, s,
                               a);
        return hipGetLastError();
    }
    uint32_t *buf_key[2];
    int32_t *buf_idx[2];
    char *w = static_cast<char *>(ws);
    for (int b = 0; b < 2; ++b) {
        buf_key[b] = reinterpret_cast<uint32_t *>(w);
        if (w) w += rows * pl.ld[b] * 4;
        buf_idx[b] = reinterpret_cast<int32_t *>(w);
        if (w) w += rows * pl.ld[b] * 4;
    }
    const uint32_t gx = static_cast<uint32_t>(rows);
    for (int i = 0; i < pl.npass; ++i) {
        a.nprev = i;
        a.okey = buf_key[i % 2];
        a.oidx = buf_idx[i % 2];
        a.cout_ld = pl.ld[i % 2];
        if (i > 0) {
            a.ckey = buf_key[(i - 1) % 2];
            a.cidx = buf_idx[(i - 1) % 2];
            a.cin_ld = pl.ld[(i - 1) % 2];
        }
        const int64_t e_in = i == 0 ? nb_max : pl.entries[i - 1];
        const dim3 grid(gx, static_cast<uint32_t>((e_in + pl.seg[i] - 1) / pl.seg[i]));
        if (pl.seg[i] == kSegSmall) {
            if (i == 0)
                hipLaunchKernelGGL((topk_pass<256, 16, 0, 1>), grid, dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL((topk_pass<256, 16, 1, 1>), grid, dim3(256), 0, s, a);
        } else {
            if (i == 0)
                hipLaunchKernelGGL((topk_pass<1024, 32, 0, 1>), grid, dim3(1024), 0, s, a);
            else
                hipLaunchKernelGGL((topk_pass<1024, 32, 1, 1>), grid, dim3(1024), 0, s, a);
        }
        a.prev_seg[i] = pl.seg[i];
    }
    a.nprev = pl.npass;
    // final pass: a 4-wave workgroup when the rows fit in 8,192 keys (a
    // shorter chain of barriers), else 16 waves
    const bool small = pl.final_entries <= kSegMid;
    if (pl.npass > 0) {
        a.ckey = buf_key[(pl.npass - 1) % 2];
        a.cidx = buf_idx[(pl.npass - 1) % 2];
        a.cin_ld = pl.ld[(pl.npass - 1) % 2];
        if (small)
            hipLaunchKernelGGL((topk_pass<256, 32, 1, 0>), dim3(gx), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((topk_pass<1024, 32, 1, 0>), dim3(gx), dim3(1024), 0, s, a);
    } else {
        if (small)
            hipLaunchKernelGGL((topk_pass<256, 32, 0, 0>), dim3(gx), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((topk_pass<1024, 32, 0, 0>), dim3(gx), dim3(1024), 0, s, a);
    }
    return hipGetLastError();
}

DecListLayout dec_list_layout(int64_t rows, int64_t nb_max, int K) {
    DecListLayout l{};
    const int64_t nseg = (nb_max + kDecSeg - 1) / kDecSeg;
    // few rows of more blocks than one register-resident pass takes
    l.use = rows > 0 && rows < 256 && nb_max > kStreamMin && nseg <= kDecMaxSeg &&
            K <= kDecSeg;
    if (!l.use) return l;
    l.gld = ((nb_max + 63) / 64 + 3) / 4 * 4;
    l.lld = nseg * kDecSeg;
    l.cld = (nseg + 3) / 4 * 4;
    l.ws_bytes = static_cast<size_t>(rows) * static_cast<size_t>(l.gld + 2 * l.lld + l.cld) * 4u;
    return l;
}

hipError_t launch_topk_dec_lists(const float *scores, int B, int nq, int64_t ld,
                                 const int64_t *seq_len, int64_t nb_max, int r, int K,
                                 int32_t *blk_idx, int32_t *n_sel, void *ws, hipStream_t s) {
    if (B == 0) return hipSuccess;
    const DecListLayout l = dec_list_layout(B, nb_max, K);
    DecTopkArgs d{};
    d.t.scores = scores;
    d.t.ld = ld;
    d.t.blk_idx = blk_idx;
    d.t.n_sel = n_sel;
    d.t.Tq = 1;
    d.t.nq = nq;
    d.t.pos0 = 0;
    d.t.nb_max = nb_max;
    d.t.seq_len = seq_len;
    d.t.r = r;
    d.t.K = K;
    char *w = static_cast<char *>(ws);
    d.gmax = reinterpret_cast<const uint32_t *>(w);
    d.gld = l.gld;
    w += static_cast<size_t>(B) * l.gld * 4;
    d.lkey = reinterpret_cast<uint32_t *>(w);
    w += static_cast<size_t>(B) * l.lld * 4;
    d.lidx = reinterpret_cast<int32_t *>(w);
    w += static_cast<size_t>(B) * l.lld * 4;
    d.lcnt = reinterpret_cast<uint32_t *>(w);
    d.lld = l.lld;
    d.cld = l.cld;
    const dim3 grid(static_cast<uint32_t>(l.lld / kDecSeg), static_cast<uint32_t>(B));
    hipLaunchKernelGGL(topk_dec_filter, grid, dim3(256), 0, s, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_dec_final, dim3(static_cast<uint32_t>(B)), dim3(1024), 0, s, d);
    return hipGetLastError();
}

}  // namespace qsa
