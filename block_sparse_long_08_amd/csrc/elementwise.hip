// A1 (partial RoPE) and A2 (micro-block key pooling).  Both are HBM-bound
// streaming kernels; their arithmetic runs in fp64 so that the single bf16
// rounding at the end sees the exact (MEAN) or correctly rounded value.
#include "qsa_internal.h"

namespace qsa {

struct InvFreq {
    double v[64];
};

// One workgroup per row t: angles for the row's position are formed once in
// LDS, then every head's pairs are rotated.  The row's values do not depend
// on its position, so they are requested first (and the untouched dims
// copied) while the position and the angles are formed.
constexpr int kRopePairsPerThread = 4;  // pairs a thread keeps in registers

__global__ void __launch_bounds__(256) rope_kernel(const uint16_t *__restrict__ x,
                                                   uint16_t *__restrict__ y, int64_t T,
                                                   int nheads, int head_dim, int rope_dim,
                                                   InvFreq inv_freq, int64_t pos0,
                                                   const int64_t *__restrict__ seq_len, int nq) {
#pragma clang fp contract(off)
    __shared__ double cs[64], sn[64];
    const int64_t t = blockIdx.x;
    const int half = rope_dim / 2;
    const uint16_t *xr = x + t * nheads * static_cast<int64_t>(head_dim);
    uint16_t *yr = y + t * nheads * static_cast<int64_t>(head_dim);
    const int npairs = nheads * half;
    // the first pairs of this thread, loaded before the position is known
    uint16_t pa[kRopePairsPerThread], pb[kRopePairsPerThread];
#pragma unroll
    for (int u = 0; u < kRopePairsPerThread; ++u) {
        const int idx = threadIdx.x + u * blockDim.x;
        const int ii = idx < npairs ? idx : 0;  // an existing pair for idle threads
        const int h = ii / half, j = ii - h * half;
        const uint16_t *xh = xr + h * head_dim;
        pa[u] = xh[j];
        pb[u] = xh[j + half];
    }
    if (y != x) {
        // copy the untouched dims, 16 bytes at a time (rope_dim % 8 == 0 and
        // head_dim % 8 == 0 are checked by the caller)
        const int per_head = (head_dim - rope_dim) / 8;
        for (int idx = threadIdx.x; idx < nheads * per_head; idx += blockDim.x) {
            int h = idx / per_head, c = idx - h * per_head;
            const uint4 *src =
                reinterpret_cast<const uint4 *>(xr + h * head_dim + rope_dim) + c;
            uint4 *dst = reinterpret_cast<uint4 *>(yr + h * head_dim + rope_dim) + c;
            *dst = *src;
        }
    }
    // decode form: row t is query t % nq of sequence t / nq, the nq newest
    // positions of that sequence
    int64_t p = seq_len ? seq_len[t / nq] - nq + t % nq : pos0 + t;
    if (p < 0) p = 0;
    for (int j = threadIdx.x; j < half; j += blockDim.x) rope_angle(p, inv_freq.v[j], cs[j], sn[j]);
    block_sync();
    for (int idx = threadIdx.x, u = 0; idx < npairs; idx += blockDim.x, ++u) {
        int h = idx / half, j = idx - h * half;
        const uint16_t *xh = xr + h * head_dim;
        const uint16_t ra = u < kRopePairsPerThread ? pa[u & (kRopePairsPerThread - 1)] : xh[j];
        const uint16_t rb =
            u < kRopePairsPerThread ? pb[u & (kRopePairsPerThread - 1)] : xh[j + half];
        uint16_t o0, o1;
        rope_pair(ra, rb, cs[j], sn[j], o0, o1);
        yr[h * head_dim + j] = o0;
        yr[h * head_dim + j + half] = o1;
    }
}

// Rows with few pairs (the keys' 2 heads, the indexer's 4): rpw rows per
// workgroup, so that one round of fp64 angles (one per thread) and one
// barrier serve several rows; the same arithmetic as rope_kernel.  Threads
// take the rows' angles, then their untouched dims, then their pairs.
constexpr int kRopeMaxRows = 8;

__global__ void __launch_bounds__(256) rope_rows_kernel(const uint16_t *__restrict__ x,
                                                        uint16_t *__restrict__ y, int64_t T,
                                                        int nheads, int head_dim, int rope_dim,
                                                        InvFreq inv_freq, int64_t pos0,
                                                        const int64_t *__restrict__ seq_len,
                                                        int nq, int rpw) {
#pragma clang fp contract(off)
    __shared__ double cs[kRopeMaxRows][64], sn[kRopeMaxRows][64];
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * rpw;
    const int rows = static_cast<int>(min(static_cast<int64_t>(rpw), T - t0));
    const int half = rope_dim / 2;
    const int64_t row_elems = static_cast<int64_t>(nheads) * head_dim;
    for (int idx = threadIdx.x; idx < rows * half; idx += blockDim.x) {
        const int r = idx / half, j = idx - r * half;
        const int64_t t = t0 + r;
        // decode form: row t is query t % nq of sequence t / nq
        int64_t p = seq_len ? seq_len[t / nq] - nq + t % nq : pos0 + t;
        if (p < 0) p = 0;
        rope_angle(p, inv_freq.v[j], cs[r][j], sn[r][j]);
    }
    if (y != x) {
        // the untouched dims, 16 bytes at a time
        const int per_head = (head_dim - rope_dim) / 8;
        const int per_row = nheads * per_head;
        for (int idx = threadIdx.x; idx < rows * per_row; idx += blockDim.x) {
            const int r = idx / per_row, rest = idx - r * per_row;
            const int h = rest / per_head, c = rest - h * per_head;
            const int64_t off = (t0 + r) * row_elems + h * head_dim + rope_dim;
            reinterpret_cast<uint4 *>(y + off)[c] = reinterpret_cast<const uint4 *>(x + off)[c];
        }
    }
    block_sync();
    const int npairs = nheads * half;
    for (int idx = threadIdx.x; idx < rows * npairs; idx += blockDim.x) {
        const int r = idx / npairs, rest = idx - r * npairs;
        const int h = rest / half, j = rest - h * half;
        const int64_t off = (t0 + r) * row_elems + h * head_dim;
        uint16_t o0, o1;
        rope_pair(x[off + j], x[off + j + half], cs[r][j], sn[r][j], o0, o1);
        y[off + j] = o0;
        y[off + j + half] = o1;
    }
}

hipError_t launch_rope(const uint16_t *x, uint16_t *y, int64_t T, int nheads, int head_dim,
                       int rope_dim, const double *inv_freq, int64_t pos0,
                       const int64_t *seq_len, int nq, hipStream_t s) {
    if (T == 0) return hipSuccess;
    InvFreq f;
    for (int j = 0; j < 64; ++j) f.v[j] = j < rope_dim / 2 ? inv_freq[j] : 0.0;
    const int npairs = nheads * (rope_dim / 2);
    const int rpw = npairs > 0 ? min(kRopeMaxRows, 256 / npairs) : 1;
    if (rpw >= 2) {
        const int64_t nwg = (T + rpw - 1) / rpw;
        hipLaunchKernelGGL(rope_rows_kernel, dim3(static_cast<uint32_t>(nwg)), dim3(256), 0, s,
                           x, y, T, nheads, head_dim, rope_dim, f, pos0, seq_len, nq, rpw);
    } else {
        hipLaunchKernelGGL(rope_kernel, dim3(static_cast<uint32_t>(T)), dim3(256), 0, s, x, y,
                           T, nheads, head_dim, rope_dim, f, pos0, seq_len, nq);
    }
    return hipGetLastError();
}

// One thread per (sequence, block, 8-dim chunk); the Di/8 threads of a block
// are consecutive lanes, so the RMSNorm reduction stays inside a wave.
// Optional: RMSNorm gain (mode 1) and partial RoPE of the pooled key over its
// first rope_dim dims at the block's first token, r * (block0 + block): the
// pair partner of dim j < rope_dim/2 lives in chunk c ^ (rope_dim/16) of the
// same block (rope_dim a power of two), one lane xor away.
template <int DI>
__global__ void __launch_bounds__(256) compress_kernel(const uint16_t *__restrict__ k, int B,
                                                       int64_t nb, int64_t k_seq_stride, int r,
                                                       int mode, const uint16_t *__restrict__ gain,
                                                       int rope_dim, InvFreq inv_freq,
                                                       int64_t block0, uint16_t *__restrict__ kbar,
                                                       int64_t kbar_seq_stride, PageTable pg) {
#pragma clang fp contract(off)
    constexpr int CH = DI / 8;  // chunks per block row (8, 16 or 32 lanes)
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(B) * nb * CH;
    const bool live = gid < total;
    const int64_t g = live ? gid : total - 1;
    const int c = static_cast<int>(g % CH);
    const int64_t jb = (g / CH) % nb;
    const int64_t b = g / (CH * nb);
    const uint16_t *src = k + b * k_seq_stride + (jb * r) * DI + c * 8;
    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    for (int t = 0; t < r; ++t) {
        uint4 v = *reinterpret_cast<const uint4 *>(src + t * DI);
        const uint16_t *h = reinterpret_cast<const uint16_t *>(&v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += static_cast<double>(bf16_bits_to_f32(h[i]));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] / static_cast<double>(r);
    if (mode == 1) {
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += acc[i] * acc[i];
#pragma unroll
        for (int off = CH / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, CH);
        double inv = 1.0 / sqrt(ss / static_cast<double>(DI) + 1e-6);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] *= inv * (gain ? static_cast<double>(bf16_bits_to_f32(gain[c * 8 + i])) : 1.0);
    }
    if (rope_dim > 0) {
        const int hc = rope_dim / 16;  // chunks in half the rotated dims
        double other[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) other[i] = __shfl_xor(acc[i], hc, CH);
        if (c < 2 * hc) {
            const bool lo = c < hc;  // holds a of the pairs (a, b)
            const double p = static_cast<double>(r) * static_cast<double>(block0 + jb);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = (lo ? c : c - hc) * 8 + i;
                double sn, cs;
                sincos(p * inv_freq.v[j], &sn, &cs);
                const double a = lo ? acc[i] : other[i], bb = lo ? other[i] : acc[i];
                const double ac = a * cs, bs = bb * sn, bc = bb * cs, as = a * sn;
                acc[i] = lo ? ac - bs : bc + as;
            }
        }
    }
    if (!live) return;
    uint16_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = f64_to_bf16_rne(acc[i]);
    uint16_t *dst = pg.table ? kbar + page_row(pg.table + b * pg.stride, pg.shift, block0 + jb) * DI
                             : kbar + b * kbar_seq_stride + jb * DI;
    *reinterpret_cast<uint4 *>(dst + c * 8) = *reinterpret_cast<const uint4 *>(out);
}

hipError_t launch_compress(const uint16_t *k, int B, int64_t Tk, int64_t k_seq_stride, int Di,
                           int r, int mode, const uint16_t *gain, int rope_dim,
                           const double *inv_freq, int64_t block0, uint16_t *kbar,
                           int64_t kbar_seq_stride, hipStream_t s, PageTable pg) {
    const int64_t nb = Tk / r;
    if (nb == 0 || B == 0) return hipSuccess;
    InvFreq f;
    for (int j = 0; j < 64; ++j) f.v[j] = inv_freq && j < rope_dim / 2 ? inv_freq[j] : 0.0;
    const int64_t threads = static_cast<int64_t>(B) * nb * (Di / 8);
    const dim3 grid(static_cast<uint32_t>((threads + 255) / 256));
    switch (Di) {
    case 64:
        hipLaunchKernelGGL(compress_kernel<64>, grid, dim3(256), 0, s, k, B, nb, k_seq_stride,
                           r, mode, gain, rope_dim, f, block0, kbar, kbar_seq_stride, pg);
        break;
    case 128:
        hipLaunchKernelGGL(compress_kernel<128>, grid, dim3(256), 0, s, k, B, nb, k_seq_stride,
                           r, mode, gain, rope_dim, f, block0, kbar, kbar_seq_stride, pg);
        break;
    default:
        hipLaunchKernelGGL(compress_kernel<256>, grid, dim3(256), 0, s, k, B, nb, k_seq_stride,
                           r, mode, gain, rope_dim, f, block0, kbar, kbar_seq_stride, pg);
        break;
    }
    return hipGetLastError();
}

}  // namespace qsa
