// Gather ceiling probe: a measurement kernel, not part of the layer (it is
// built into its own library, libqsa_probe.so, which only the benchmark
// loads).  It reads exactly the key and value bytes the sparse prefill
// attention reads for a selection -- per query and KV head the 512-byte head
// rows of the tokens of each selected 4-token block and of the query's
// incomplete block, in the attention's order of 16-token stages -- with the
// same grid (one workgroup per query, one wave per KV head), and does nothing
// with them but fold them into one word per (query, head).  Each wave keeps
// two stages (32 KB) in flight, so the time of a launch is what the memory
// system needs to deliver the attention's gathers: the ceiling the attention
// kernel is measured against.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kHeadDim = 256;
constexpr int kBlock = 4;

struct Entries {
    const int32_t *blk;  // the query's selected blocks
    int ns;              // selected blocks
    int tail;            // tokens of the incomplete block
    int64_t nc;          // complete blocks of the query
    __device__ __forceinline__ int64_t token(int e, int i, int64_t p) const {
        if (e < ns) {
            int64_t b = blk[e];
            b = b < 0 ? 0 : (b >= nc ? nc - 1 : b);
            return kBlock * b + i;
        }
        return (e == ns && i < tail) ? kBlock * nc + i : p;
    }
};

// Lane l reads 128 contiguous bytes (8 x 16) of token l/4 of a 16-token stage:
// four lanes cover one 512-byte head row.
__device__ __forceinline__ void stage_load(const Entries &L, int e0, int64_t p,
                                           const uint16_t *__restrict__ Kg,
                                           const uint16_t *__restrict__ Vg, int64_t rs, int lane,
                                           uint4 (&k)[8], uint4 (&v)[8]) {
    const int tt = lane >> 2, c0 = (lane & 3) * 8;
    const int64_t tok = L.token(e0 + (tt >> 2), tt & 3, p);
    const uint4 *ks = reinterpret_cast<const uint4 *>(Kg + tok * rs) + c0;
    const uint4 *vs = reinterpret_cast<const uint4 *>(Vg + tok * rs) + c0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        k[j] = ks[j];
        v[j] = vs[j];
    }
}

__device__ __forceinline__ uint32_t fold(const uint4 (&k)[8], const uint4 (&v)[8]) {
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) x ^= k[j].x ^ k[j].y ^ k[j].z ^ k[j].w ^ v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    return x;
}

__global__ void __launch_bounds__(128) gather_probe_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ blk_idx, const int32_t *__restrict__ n_sel, int64_t pos0,
    int Kbudget, int Hkv, uint32_t *__restrict__ out) {
    const int64_t t = blockIdx.x;
    const int64_t p = pos0 + t;
    const int64_t nc = (p + 1) / kBlock;
    const int v = n_sel[t];
    const int64_t cap = nc < Kbudget ? nc : Kbudget;
    const int ns = v < 0 ? 0 : (v > cap ? static_cast<int>(cap) : v);
    const Entries L{blk_idx + t * Kbudget, ns, static_cast<int>((p + 1) % kBlock), nc};
    const int E = ns + (L.tail > 0 ? 1 : 0);
    const int nstages = (E + 3) / 4;
    const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int64_t rs = static_cast<int64_t>(Hkv) * kHeadDim;
    const uint16_t *Kg = K + g * kHeadDim;
    const uint16_t *Vg = V + g * kHeadDim;
    uint32_t acc = 0;
    for (int s = 0; s < nstages; s += 2) {
        uint4 k0[8], v0[8], k1[8], v1[8];
        stage_load(L, 4 * s, p, Kg, Vg, rs, lane, k0, v0);
        if (s + 1 < nstages) {
            stage_load(L, 4 * (s + 1), p, Kg, Vg, rs, lane, k1, v1);
            acc ^= fold(k1, v1);
        }
        acc ^= fold(k0, v0);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off));
    if (lane == 0) out[t * Hkv + g] = acc;
}

}  // namespace

extern "C" {

// Gathers of the sparse prefill attention of Tq queries at pos0 .. pos0+Tq-1
// over contiguous K, V [Tk][Hkv][256] (bf16 bits) for the selection blk_idx
// [Tq][Kbudget] / n_sel [Tq]; out: [Tq][Hkv] words.  Device pointers; the
// call enqueues one launch on stream and returns 0, or 1 when the launch
// was rejected or an argument is out of range.
int qsa_probe_gather(const uint16_t *K, const uint16_t *V, const int32_t *blk_idx,
                     const int32_t *n_sel, int64_t Tq, int64_t pos0, int Kbudget, int Hkv,
                     uint32_t *out, void *stream) {
    if (!K || !V || !blk_idx || !n_sel || !out || Tq < 0 || pos0 < 0 || Kbudget <= 0 ||
        Hkv < 1 || Hkv > 2 || Tq > 2147483647)
        return 1;
    if (Tq == 0) return 0;
    hipLaunchKernelGGL(gather_probe_kernel, dim3(static_cast<uint32_t>(Tq)), dim3(64 * Hkv), 0,
                       reinterpret_cast<hipStream_t>(stream), K, V, blk_idx, n_sel, pos0, Kbudget,
                       Hkv, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
