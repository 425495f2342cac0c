// A5-A8: softmax attention over 4-token micro-blocks (chlience section 6:
// selected blocks expand to token indices; the query's incomplete block is
// always kept, later tokens masked).  The same per-wave routine serves the
// sparse prefill (one workgroup per query), split-K decode and the dense
// gather path (every complete block).
//
// Work unit: a chunk of 8 entries (32 tokens) of one KV head.  An entry is a
// selected block (4 tokens) or the trailing partial block ((p+1) mod 4
// tokens).  Per chunk a wave computes
//   S^T[32 tok, 16 heads] = K[32 tok, 256] . Q^T[256, 16 heads]   (bf16 MFMA)
//   online softmax per head in fp32 (log2 domain),
//   O^T[256, 16] += V^T[256, 32 tok] . P^T[32 tok, 16]            (bf16 MFMA)
// with P split as P_hi + P_lo (two bf16 terms, ~16 significant bits) so that
// V stays exact bf16 and no fp16 range issue arises.  Up to 16 query heads
// share one KV head in the MFMA columns (12 here; 4 columns idle).
//
// MFMA 16x16x32 layouts (lane l, n = l%16, g4 = l/16):
//   A[m][k]: lane holds row m = n, k-slots 8*g4 .. 8*g4+7 of the step
//   B[k][j]: lane holds column j = n, the same k-slots
//   D[m][j]: lane holds rows 4*g4 .. 4*g4+3 of column n
// Tile t (16 tokens) of S^T has row 4*e + i = entry e (0..3), token i, so a
// lane's accumulator holds one whole block for one head: exactly the k-slots
// it must supply as the B operand (P^T) of the PV product.
#include "qsa_internal.h"

namespace qsa {

constexpr float kScaleLog2 = 0.09016844005556021f;  // log2(e) / sqrt(256)
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kChunkEntries = 8;
constexpr int kVldsBytes = 32 * 512;          // 32 tokens x 256 bf16, per wave
constexpr int kMergeFloats = 16 * 256 + 128;  // O^T (lane-major) + m + l, per wave
constexpr int kPartFloats = 4096 + 128;       // decode partial record
constexpr int kMaxListLds = 2048;

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Entry e of a query's list: first token and number of valid tokens.
struct EntryList {
    const int32_t *lst;  // LDS copy of the selected blocks (sparse), or nullptr (dense)
    int lst_off;         // index of lst[0] in the query's list
    int ns;              // number of complete-block entries
    int pr;              // tokens in the partial block (0..3)
    int64_t nc;          // complete blocks visible to the query
    __device__ __forceinline__ int count(int e) const { return e < ns ? 4 : (e == ns ? pr : 0); }
    __device__ __forceinline__ int64_t base(int e) const {
        if (e < ns) return 4 * static_cast<int64_t>(lst ? lst[e - lst_off] : e);
        return 4 * nc;
    }
};

struct WaveState {
    f32x4 o[16];  // O^T accumulators, d-tile dt: rows d = 16*dt + 4*g4 + i, column head n
    float m;      // running max (log2 units) of head n
    float l;      // this lane's share of the weight sum of head n
};

__device__ __forceinline__ void state_init(WaveState &st) {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
}

// Process entries e0 .. e0+7 of one KV head.  Kg/Vg point at token 0 of the
// head (row stride `rs` elements); p is the query position (a safe row for
// masked tokens); vlds is this wave's 16 KB LDS staging area.
__device__ __forceinline__ void attn_chunk(const EntryList &L, int e0, int64_t p,
                                           const uint16_t *__restrict__ Kg,
                                           const uint16_t *__restrict__ Vg, int64_t rs,
                                           const bf16x8 (&qT)[8], WaveState &st,
                                           unsigned char *vlds, int lane) {
    const int n = lane & 15, g4 = lane >> 4, h = lane >> 5;
    // ---- issue the loads: K as MFMA A fragments, V as whole 512-byte rows
    uint4 kf[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int e = e0 + 4 * t + (n >> 2), i = n & 3;
        const bool ok = i < L.count(e);
        const int64_t tok = ok ? L.base(e) + i : p;
        const uint16_t *src = Kg + tok * rs + 8 * g4;
#pragma unroll
        for (int s = 0; s < 8; ++s) kf[t][s] = *reinterpret_cast<const uint4 *>(src + 32 * s);
    }
    uint4 vv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int e = e0 + (j >> 1), i = 2 * (j & 1) + h;
        const bool ok = i < L.count(e);
        const int64_t tok = ok ? L.base(e) + i : p;
        vv[j] = *reinterpret_cast<const uint4 *>(Vg + tok * rs + 8 * (lane & 31));
    }
    // ---- V rows -> LDS; 16-byte chunk c of row tt lands at c ^ 2*((tt>>2)&3)
    wave_sync();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int tt = 2 * j + h;
        const int pos = (lane & 31) ^ (2 * ((tt >> 2) & 3));
        *reinterpret_cast<uint4 *>(vlds + tt * 512 + pos * 16) = vv[j];
    }
    // ---- S^T tiles
    f32x4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 8; ++s) sacc[t] = mfma_bf16_16x16x32(as_bf16x8(kf[t][s]), qT[s], sacc[t]);
    }
    float sv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int cnt = L.count(e0 + 4 * t + g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * t + i] = i < cnt ? sacc[t][i] * kScaleLog2 : -INFINITY;
    }
    float cm = sv[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) cm = fmaxf(cm, sv[k]);
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));
    const float m_new = fmaxf(st.m, cm);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(st.m - m_use);
    bf16x8 phi, plo;
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float pv = exp2f(sv[k] - m_use);
        const __bf16 hi = static_cast<__bf16>(pv);
        const __bf16 lo = static_cast<__bf16>(pv - static_cast<float>(hi));
        phi[k] = hi;
        plo[k] = lo;
        psum += static_cast<float>(hi) + static_cast<float>(lo);
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) st.o[dt] *= alpha;
    wave_sync();
    // ---- O^T += V^T P^T: A = V^T rows d = 16*dt + n, k-slots = this lane
    // group's tokens (entry g4 and entry 4+g4 of the chunk)
    const int swz = 2 * g4;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
        const int d = 16 * dt + n;
        const int off = (((d >> 3) ^ swz) * 16) + (d & 7) * 2;
        u16x8 a;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int tt = jj < 4 ? 4 * g4 + jj : 16 + 4 * g4 + (jj - 4);
            a[jj] = *reinterpret_cast<const uint16_t *>(vlds + tt * 512 + off);
        }
        const bf16x8 av = __builtin_bit_cast(bf16x8, a);
        st.o[dt] = mfma_bf16_16x16x32(av, phi, st.o[dt]);
        st.o[dt] = mfma_bf16_16x16x32(av, plo, st.o[dt]);
    }
}

// Q^T fragments of the heads of KV head g (columns n >= group are zero).
__device__ __forceinline__ void load_qT(const uint16_t *__restrict__ qrow, int g, int group,
                                        int lane, bf16x8 (&qT)[8]) {
    const int n = lane & 15, g4 = lane >> 4;
    const bool ok = n < group;
    const uint16_t *src = qrow + static_cast<int64_t>(g * group + (ok ? n : 0)) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        uint4 v = ok ? *reinterpret_cast<const uint4 *>(src + 32 * s + 8 * g4)
                     : make_uint4(0, 0, 0, 0);
        qT[s] = as_bf16x8(v);
    }
}

// Spill a wave's state to LDS (lane-major) for a cross-wave merge.
__device__ __forceinline__ void state_store(const WaveState &st, float *buf, int lane) {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) buf[(dt * 4 + i) * 64 + lane] = st.o[dt][i];
    buf[4096 + lane] = st.m;
    buf[4096 + 64 + lane] = st.l;
}

// Fold a stored state into st (both unnormalised, each relative to its max).
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
        for (int i = 0; i < 4; ++i) st.o[dt][i] = st.o[dt][i] * a + buf[(dt * 4 + i) * 64 + lane] * b;
}

// Reduce the per-lane weight sums of each head over its 4 lane groups.
__device__ __forceinline__ float head_total(float l) {
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    return l;
}

// Normalise and write O[.., head g*group + n, :] and lse.
__device__ __forceinline__ void state_write(const WaveState &st, float ltot, float *__restrict__ orow,
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
        lse_row[hq] = ltot > 0.f ? (st.m + __log2f(ltot)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------------
// Prefill: one workgroup (4 waves) per query; waves split the KV heads and,
// within a head, the chunks.  Grid: (Tq, B).
template <bool DENSE>
__global__ void __launch_bounds__(256) attn_prefill_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * kVldsBytes + 4 * 512];
    __shared__ int32_t lst[kMaxListLds];
    const int64_t t = blockIdx.x, b = blockIdx.y;
    const int64_t row = b * a.Tq + t;
    const int64_t p = a.pos0 + t;
    const int64_t nc = num_complete_blocks(p, kBlock);
    int ns;
    if (DENSE) {
        ns = static_cast<int>(nc);
    } else {
        int v = a.n_sel[row];
        const int64_t cap = min(static_cast<int64_t>(a.Kbudget), nc);
        ns = v < 0 ? 0 : (v > cap ? static_cast<int>(cap) : v);
        const int32_t *src = a.blk_idx + row * a.Kbudget;
        for (int i = threadIdx.x; i < ns; i += 256) {
            int32_t bi = src[i];
            bi = bi < 0 ? 0 : (bi >= nc ? static_cast<int32_t>(nc - 1) : bi);
            lst[i] = bi;
        }
    }
    EntryList L{DENSE ? nullptr : lst, 0, ns, static_cast<int>((p + 1) % kBlock), nc};
    const int E = ns + (L.pr > 0 ? 1 : 0);
    const int nchunks = (E + kChunkEntries - 1) / kChunkEntries;
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wph = 4 / a.Hkv;  // waves per KV head
    const int g = wave / wph, sub = wave % wph;
    const int group = a.H / a.Hkv;
    const uint16_t *qrow = a.Q + row * a.H * kHeadDim;
    bf16x8 qT[8];
    load_qT(qrow, g, group, lane, qT);
    const int64_t rs = static_cast<int64_t>(a.Hkv) * kHeadDim;
    const uint16_t *Kg = a.K + b * a.Lmax * rs + g * kHeadDim;
    const uint16_t *Vg = a.V + b * a.Lmax * rs + g * kHeadDim;
    unsigned char *vlds = lds + wave * kVldsBytes;

    WaveState st;
    state_init(st);
    for (int c = sub; c < nchunks; c += wph)
        attn_chunk(L, c * kChunkEntries, p, Kg, Vg, rs, qT, st, vlds, lane);

    __syncthreads();
    float *mbuf = reinterpret_cast<float *>(lds);
    if (sub != 0) state_store(st, mbuf + wave * kMergeFloats, lane);
    __syncthreads();
    if (sub == 0) {
        for (int w = 1; w < wph; ++w) state_merge(st, mbuf + (wave + w) * kMergeFloats, lane);
        const float ltot = head_total(st.l);
        state_write(st, ltot, a.O + row * a.H * kHeadDim, a.lse ? a.lse + row * a.H : nullptr, g,
                    group, lane);
    }
}

// ------------------------------------------------------------------------
// Decode: workgroup (4 waves) per (split, KV head, sequence); each writes one
// partial record (unnormalised O^T, max, weight sum) to the workspace.
template <bool DENSE>
__global__ void __launch_bounds__(256) attn_decode_kernel(AttnArgs a, int nsplit, int cps) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * kVldsBytes + 4 * 512];
    __shared__ int32_t lst[kMaxListLds];
    const int split = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z;
    int64_t Lb = a.seq_len[b];
    Lb = Lb < 0 ? 0 : (Lb > a.Lmax ? a.Lmax : Lb);
    const int64_t p = Lb - 1;
    const int64_t nc = num_complete_blocks(p, kBlock);
    int ns;
    if (DENSE) {
        ns = static_cast<int>(nc);
    } else {
        int v = a.n_sel[b];
        const int64_t cap = min(static_cast<int64_t>(a.Kbudget), nc);
        ns = v < 0 ? 0 : (v > cap ? static_cast<int>(cap) : v);
    }
    const int pr = p >= 0 ? static_cast<int>((p + 1) % kBlock) : 0;
    const int E = ns + (pr > 0 ? 1 : 0);
    const int nchunks = (E + kChunkEntries - 1) / kChunkEntries;
    const int c0 = split * cps, c1 = min(c0 + cps, nchunks);
    const int e_lo = c0 * kChunkEntries;
    if (!DENSE) {
        const int e_hi = min(c1 * kChunkEntries, ns);
        const int32_t *src = a.blk_idx + b * a.Kbudget;
        for (int i = e_lo + static_cast<int>(threadIdx.x); i < e_hi; i += 256) {
            int32_t bi = src[i];
            bi = bi < 0 ? 0 : (bi >= nc ? static_cast<int32_t>(nc - 1) : bi);
            lst[i - e_lo] = bi;
        }
    }
    EntryList L{DENSE ? nullptr : lst, e_lo, ns, pr, nc};
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int group = a.H / a.Hkv;
    bf16x8 qT[8];
    load_qT(a.Q + b * a.H * kHeadDim, g, group, lane, qT);
    const int64_t rs = static_cast<int64_t>(a.Hkv) * kHeadDim;
    const uint16_t *Kg = a.K + b * a.Lmax * rs + g * kHeadDim;
    const uint16_t *Vg = a.V + b * a.Lmax * rs + g * kHeadDim;
    unsigned char *vlds = lds + wave * kVldsBytes;
    WaveState st;
    state_init(st);
    for (int c = c0 + wave; c < c1; c += 4)
        attn_chunk(L, c * kChunkEntries, p < 0 ? 0 : p, Kg, Vg, rs, qT, st, vlds, lane);
    __syncthreads();
    float *mbuf = reinterpret_cast<float *>(lds);
    if (wave != 0) state_store(st, mbuf + wave * kMergeFloats, lane);
    __syncthreads();
    if (wave == 0) {
        for (int w = 1; w < 4; ++w) state_merge(st, mbuf + w * kMergeFloats, lane);
        st.l = head_total(st.l);
        float *rec = a.part + ((b * a.Hkv + g) * nsplit + split) * static_cast<int64_t>(kPartFloats);
        state_store(st, rec, lane);
    }
}

// Merge the split records of one (sequence, KV head) and write O, lse.
__global__ void __launch_bounds__(64) attn_decode_merge(AttnArgs a, int nsplit) {
    const int g = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int lane = threadIdx.x;
    const float *rec0 = a.part + (b * a.Hkv + g) * nsplit * static_cast<int64_t>(kPartFloats);
    WaveState st;
    state_init(st);
    for (int s = 0; s < nsplit; ++s) state_merge(st, rec0 + s * static_cast<int64_t>(kPartFloats), lane);
    const int group = a.H / a.Hkv;
    state_write(st, st.l, a.O + b * a.H * kHeadDim, a.lse ? a.lse + b * a.H : nullptr, g, group,
                lane);
}

hipError_t launch_sparse_prefill(const AttnArgs &a, hipStream_t s) {
    if (a.Tq == 0 || a.B == 0) return hipSuccess;
    const dim3 grid(static_cast<uint32_t>(a.Tq), static_cast<uint32_t>(a.B));
    hipLaunchKernelGGL(attn_prefill_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_dense_prefill(const AttnArgs &a, hipStream_t s) {
    if (a.Tq == 0 || a.B == 0) return hipSuccess;
    const dim3 grid(static_cast<uint32_t>(a.Tq), static_cast<uint32_t>(a.B));
    hipLaunchKernelGGL(attn_prefill_kernel<true>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

int decode_num_splits(int B, int Hkv, int64_t max_entries) {
    const int64_t nchunks = (max_entries + kChunkEntries - 1) / kChunkEntries;
    int64_t want = (1024 + static_cast<int64_t>(B) * Hkv - 1) / (static_cast<int64_t>(B) * Hkv);
    const int64_t cap = (nchunks + 3) / 4;  // at least 4 chunks (one per wave) per split
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    return static_cast<int>(want);
}

size_t decode_partial_floats(int B, int Hkv, int nsplit) {
    return static_cast<size_t>(B) * Hkv * nsplit * kPartFloats;
}

hipError_t launch_attn_decode(const AttnArgs &a, int nsplit, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    const int64_t max_entries = a.blk_idx ? a.Kbudget + 1 : a.Lmax / kBlock + 1;
    const int64_t nchunks = (max_entries + kChunkEntries - 1) / kChunkEntries;
    const int cps = static_cast<int>((nchunks + nsplit - 1) / nsplit);
    const dim3 grid(static_cast<uint32_t>(nsplit), static_cast<uint32_t>(a.Hkv),
                    static_cast<uint32_t>(a.B));
    if (a.blk_idx)
        hipLaunchKernelGGL(attn_decode_kernel<false>, grid, dim3(256), 0, s, a, nsplit, cps);
    else
        hipLaunchKernelGGL(attn_decode_kernel<true>, grid, dim3(256), 0, s, a, nsplit, cps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_decode_merge, dim3(static_cast<uint32_t>(a.Hkv), static_cast<uint32_t>(a.B)),
                       dim3(64), 0, s, a, nsplit);
    return hipGetLastError();
}

}  // namespace qsa
