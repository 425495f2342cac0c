// Gather ceiling probe: a measurement kernel, not part of the layer (it is
// built into its own library, libqsa_probe.so, which only the benchmark
// loads).  It issues exactly the loads of the sparse prefill attention for a
// selection -- per query and KV head, 16-token stages of the selected
// 4-token blocks and the query's incomplete block; per stage the value rows
// by LDS DMA into an 8 KB tile (16-byte chunks at the same XOR-swizzled
// slots) and the key rows into registers with the same lane map -- with the
// same grid (one one-wave workgroup per query and KV head, workgroup
// Hkv * query + head) and one stage in flight per wave, and does no
// arithmetic but folding the key words into one word per (query, head).  It
// needs few registers, so up to five waves per SIMD run; a caller can hold it
// to fewer (the attention's three) with padding LDS.  Its time per launch is
// what the memory system needs for the attention's loads without their
// arithmetic.
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

__device__ __forceinline__ int row_swizzle(int tt) { return 2 * ((tt >> 2) & 3); }

// One stage: V rows by LDS DMA (instruction j fills bytes 1024*j .. of the
// tile: row tt = 2j + lane/32, chunk (lane%32) ^ row_swizzle(tt)), K rows
// into registers (lane l: token l%16 of the stage, dims 8*(l/16) + 32*s).
__device__ __forceinline__ uint32_t stage(const Entries &L, int e0, int64_t p,
                                          const uint16_t *__restrict__ Kg,
                                          const uint16_t *__restrict__ Vg, int64_t rs,
                                          unsigned char *tile, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int tt = 2 * j + h;
        const int64_t tok = L.token(e0 + (tt >> 2), tt & 3, p);
        const int c = (lane & 31) ^ row_swizzle(tt);
        const uint16_t *src = Vg + tok * rs + 8 * c;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)(tile + 1024 * j),
                                         16, 0, 0);
    }
    const int n = lane & 15, g4 = lane >> 4;
    const uint16_t *ks = Kg + L.token(e0 + (n >> 2), n & 3, p) * rs + 8 * g4;
    uint4 k[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) k[s] = *reinterpret_cast<const uint4 *>(ks + 32 * s);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): keys and the value tile have landed
    __builtin_amdgcn_wave_barrier();
    uint32_t x = 0;
#pragma unroll
    for (int s = 0; s < 8; ++s) x ^= k[s].x ^ k[s].y ^ k[s].z ^ k[s].w;
    return x;
}

__global__ void __launch_bounds__(64) gather_probe_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ blk_idx, const int32_t *__restrict__ n_sel, int64_t pos0,
    int Kbudget, int Hkv, uint32_t *__restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) unsigned char tile[];  // 8 KB (+ padding)
    const int64_t t = blockIdx.x / Hkv;
    const int g = static_cast<int>(blockIdx.x - t * Hkv);
    const int64_t p = pos0 + t;
    const int64_t nc = (p + 1) / kBlock;
    const int v = n_sel[t];
    const int64_t cap = nc < Kbudget ? nc : Kbudget;
    const int ns = v < 0 ? 0 : (v > cap ? static_cast<int>(cap) : v);
    const Entries L{blk_idx + t * Kbudget, ns, static_cast<int>((p + 1) % kBlock), nc};
    const int E = ns + (L.tail > 0 ? 1 : 0);
    const int nstages = (E + 3) / 4;
    const int lane = threadIdx.x & 63;
    const int64_t rs = static_cast<int64_t>(Hkv) * kHeadDim;
    const uint16_t *Kg = K + g * kHeadDim;
    const uint16_t *Vg = V + g * kHeadDim;
    uint32_t acc = 0;
    for (int s = 0; s < nstages; ++s) acc ^= stage(L, 4 * s, p, Kg, Vg, rs, tile, lane);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off));
    if (lane == 0) out[t * Hkv + g] = acc;
}

}  // namespace

extern "C" {

// Gathers of the sparse prefill attention of Tq queries at pos0 .. pos0+Tq-1
// over contiguous K, V [Tk][Hkv][256] (bf16 bits) for the selection blk_idx
// [Tq][Kbudget] / n_sel [Tq]; out: [Tq][Hkv] words.  waves_per_simd 1..5
// holds the kernel to that many waves per SIMD (by the LDS of its one-wave
// workgroups: 160 KB per CU); 0 leaves it free.  Device pointers; the call
// enqueues one launch on stream and returns 0, or 1 when the launch was
// rejected or an argument is out of range.
int qsa_probe_gather(const uint16_t *K, const uint16_t *V, const int32_t *blk_idx,
                     const int32_t *n_sel, int64_t Tq, int64_t pos0, int Kbudget, int Hkv,
                     int waves_per_simd, uint32_t *out, void *stream) {
    if (!K || !V || !blk_idx || !n_sel || !out || Tq < 0 || pos0 < 0 || Kbudget <= 0 ||
        Hkv < 1 || Hkv > 2 || Tq >= (int64_t(1) << 25) || waves_per_simd < 0 ||
        waves_per_simd > 5)
        return 1;
    if (Tq == 0) return 0;
    size_t lds = 8192;
    if (waves_per_simd > 0) {
        // workgroups per CU = 4 SIMDs x waves per SIMD
        const size_t wgs = static_cast<size_t>(4 * waves_per_simd);
        // wgs fit in 160 KB, wgs + 1 do not
        const size_t need = (160 * 1024) / (wgs + 1) + 16;
        lds = need > lds ? need : lds;
    }
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gather_probe_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return 1;
    hipLaunchKernelGGL(gather_probe_kernel, dim3(static_cast<uint32_t>(Tq * Hkv)), dim3(64), lds,
                       reinterpret_cast<hipStream_t>(stream), K, V, blk_idx, n_sel, pos0, Kbudget,
                       Hkv, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
