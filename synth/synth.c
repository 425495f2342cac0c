/*
 * Seeded synthetic inputs for the QSA layer: counter-based N(0,1) values
 * rounded to bf16, and the planted "needle" block sets.
 *
 * This module defines inputs only.  It contains none of the layer's
 * arithmetic (no RoPE, pooling, scoring, selection or attention), so that the
 * fp64 oracle and the GPU path can both be fed from it without sharing any
 * method code.
 *
 * Generator (all integer steps are exact, so every platform gives the same
 * bits):
 *   mix(z)      = SplitMix64 output function (Steele, Lea & Flood, "Fast
 *                 splittable pseudorandom number generators", OOPSLA 2014):
 *                 z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27;
 *                 z *= 0x94D049BB133111EB; z ^= z>>31.
 *   key(s, σ)   = mix(s * 0x9E3779B97F4A7C15 + σ * 0xD1B54A32D192ED03 + 1)
 *   word(s,σ,c) = mix(key(s,σ) + (c+1) * 0x9E3779B97F4A7C15)
 *   U(s,σ,c)    = ((word >> 11) + 0.5) * 2^-53            in (0, 1)
 *   element e of stream σ: pair i = e/2, u1 = U(2i), u2 = U(2i+1),
 *   R = sqrt(-2 ln u1), φ = 2π u2, z = R cos φ (e even) or R sin φ (e odd)
 *   (Box & Muller 1958), then rounded to fp32 and to bf16, both to nearest
 *   even.
 * Streams: 1 = Q, 2 = K, 3 = V, 4 = indexer q, 5 = indexer k, 6 = needles.
 * A tensor's elements are numbered in its row-major order; a batched tensor
 * (decode caches) numbers element e of sequence b as b * per_seq + e.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(seed * GOLDEN + stream * 0xD1B54A32D192ED03ULL + 1ULL);
}

static inline double unit_open(uint64_t key, uint64_t counter) {
    uint64_t w = mix64(key + (counter + 1ULL) * GOLDEN);
    return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs only). */
static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

uint64_t synth_word(uint64_t seed, uint64_t stream, uint64_t counter) {
    return mix64(stream_key(seed, stream) + (counter + 1ULL) * GOLDEN);
}

double synth_uniform(uint64_t seed, uint64_t stream, uint64_t counter) {
    return unit_open(stream_key(seed, stream), counter);
}

/* Standard normal value of element e, in fp64 (before any rounding). */
double synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t e) {
    uint64_t key = stream_key(seed, stream);
    uint64_t i = e >> 1;
    double u1 = unit_open(key, 2 * i);
    double u2 = unit_open(key, 2 * i + 1);
    double r = sqrt(-2.0 * log(u1));
    double phi = 6.283185307179586476925286766559 * u2;
    return (e & 1) ? r * sin(phi) : r * cos(phi);
}

/* Fill out[0..count) with bf16 bits of elements first..first+count of the
 * stream.  OpenMP-parallel when built with -fopenmp. */
void synth_fill_normal_bf16(uint64_t seed, uint64_t stream, uint64_t first,
                            int64_t count, uint16_t *out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < count; ++k) {
        uint64_t e = first + (uint64_t)k;
        uint64_t i = e >> 1;
        double u1 = unit_open(key, 2 * i);
        double u2 = unit_open(key, 2 * i + 1);
        double r = sqrt(-2.0 * log(u1));
        double phi = 6.283185307179586476925286766559 * u2;
        double z = (e & 1) ? r * sin(phi) : r * cos(phi);
        out[k] = f32_to_bf16_rne((float)z);
    }
}

/* Strided variant: fills rows of `row_len` elements taken from the stream at
 * element offsets first + j*src_stride, writing them at out + j*dst_stride.
 * Used to fill one sequence's slice of a batched cache. */
void synth_fill_normal_bf16_rows(uint64_t seed, uint64_t stream, uint64_t first,
                                 int64_t nrows, int64_t row_len,
                                 int64_t src_stride, int64_t dst_stride,
                                 uint16_t *out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nrows; ++j) {
        for (int64_t k = 0; k < row_len; ++k) {
            uint64_t e = first + (uint64_t)(j * src_stride + k);
            uint64_t i = e >> 1;
            double u1 = unit_open(key, 2 * i);
            double u2 = unit_open(key, 2 * i + 1);
            double r = sqrt(-2.0 * log(u1));
            double phi = 6.283185307179586476925286766559 * u2;
            double z = (e & 1) ? r * sin(phi) : r * cos(phi);
            out[j * dst_stride + k] = f32_to_bf16_rne((float)z);
        }
    }
}

/* Needle sets: for each of `n_sets` sets, `per_set` distinct block indices in
 * [0, n_blocks), drawn from stream 6 by rejection of repeats (within a set).
 * out is [n_sets][per_set], each set sorted ascending.  Returns 0, or -1 if
 * per_set > n_blocks. */
int synth_needle_blocks(uint64_t seed, int64_t n_blocks, int n_sets, int per_set,
                        int64_t *out) {
    if (per_set > n_blocks || n_blocks <= 0) return -1;
    uint64_t key = stream_key(seed, 6);
    uint64_t c = 0;
    for (int s = 0; s < n_sets; ++s) {
        int64_t *set = out + (int64_t)s * per_set;
        int have = 0;
        while (have < per_set) {
            double u = unit_open(key, c++);
            int64_t b = (int64_t)(u * (double)n_blocks);
            if (b >= n_blocks) b = n_blocks - 1;
            int dup = 0;
            for (int j = 0; j < have; ++j)
                if (set[j] == b) { dup = 1; break; }
            if (!dup) set[have++] = b;
        }
        /* insertion sort, ascending */
        for (int i = 1; i < per_set; ++i) {
            int64_t v = set[i];
            int j = i - 1;
            while (j >= 0 && set[j] > v) { set[j + 1] = set[j]; --j; }
            set[j + 1] = v;
        }
    }
    return 0;
}

/* Multiply bf16 rows by 4 in place (exact: exponent + 2, for finite values
 * far below the bf16 overflow threshold).  rows[i] is a row start index in
 * units of row_len elements. */
void synth_scale_rows_x4(uint16_t *data, const int64_t *rows, int64_t nrows,
                         int64_t row_len, int64_t row_stride) {
    for (int64_t i = 0; i < nrows; ++i) {
        uint16_t *p = data + rows[i] * row_stride;
        for (int64_t k = 0; k < row_len; ++k) {
            uint16_t h = p[k];
            uint16_t exp = (h >> 7) & 0xFF;
            if (exp == 0 || exp >= 0xFD) continue; /* zero/subnormal/near-overflow left as is */
            p[k] = (uint16_t)(h + (2u << 7));
        }
    }
}
