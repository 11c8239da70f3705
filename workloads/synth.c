/*
 * Seeded synthetic input generator: standard-normal values stored as bf16 bit
 * patterns.  Test and benchmark infrastructure only; it holds none of the
 * attention arithmetic and is shared, unchanged, by the fp64 oracle's tests and
 * by the GPU path's tests and benchmark.
 *
 * Element i of stream `stream` under seed `seed` is a pure function of
 * (seed, stream, i), so the output does not depend on chunking or thread count:
 *
 *   key   = mix(mix(seed) ^ (stream * GAMMA))
 *   h     = mix(key + (i + 1) * GAMMA)                 (64 random bits)
 *   u1    = ((h >> 32) + 1) / 2^32  in (0, 1]
 *   u2    = (h & 0xffffffff) / 2^32 in [0, 1)
 *   z     = sqrt(-2 ln u1) * cos(2 pi u2)               (Box and Muller, 1958)
 *   bits  = bf16_rne(float(z))
 *
 * mix() is the SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) and GAMMA its golden-ratio
 * increment.  bf16_rne keeps the upper 16 bits of the IEEE binary32 pattern,
 * rounding to nearest with ties to even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0; /* NaN */
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
    return mix(mix(seed) ^ (stream * GAMMA));
}

/* out[j] = value of element (offset + j), j in [0, n). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                       uint16_t *out, int nthreads) {
    const uint64_t key = synth_key(seed, stream);
    const double two_pi = 6.283185307179586476925286766559;
    const double inv32 = 1.0 / 4294967296.0;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static, 65536)
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        uint64_t h = mix(key + ((offset + (uint64_t)j) + 1) * GAMMA);
        double u1 = ((double)(h >> 32) + 1.0) * inv32;
        double u2 = (double)(h & 0xFFFFFFFFULL) * inv32;
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[j] = f32_to_bf16_rne((float)z);
    }
}

/* Writes `value` into `count` rows of `row_len` uint16 elements starting at the
 * element offsets in `row_starts` (used to poison bytes no kernel may read). */
void synth_fill_rows(uint16_t *base, const int64_t *row_starts, int64_t count,
                     int64_t row_len, uint16_t value) {
    for (int64_t r = 0; r < count; ++r) {
        uint16_t *p = base + row_starts[r];
        for (int64_t e = 0; e < row_len; ++e) p[e] = value;
    }
}
