/*
 * Seeded synthetic inputs for the routed mixture-of-experts layer.
 *
 * This module only draws numbers: it holds none of the layer's arithmetic
 * (no routing, no dequantisation, no FFN).  Both the CPU oracle's tests and
 * the HIP path's tests and benchmark take their inputs from here.
 *
 * Generator: counter-based SplitMix64.  The mixing function is the published
 * SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014; constants as in Vigna's public-domain
 * splitmix64.c).  Element i of tensor `tid` under seed `seed` is
 *     key   = mix(seed * 0x9E3779B97F4A7C15 + tid * 0xD1B54A32D192ED03 + 1)
 *     h(i)  = mix(key + (i + 1) * 0x9E3779B97F4A7C15)
 * so any element can be produced independently (on any thread, in any order).
 *
 * Derived draws (all integer or IEEE basic operations except the normals):
 *   uniform24(h) = (h >> 40) * 2^-24                        in [0, 1), exact in fp32
 *   randint(h, lo, hi) = lo + (((h >> 32) * (hi - lo + 1)) >> 32)   inclusive range
 *   normal: Box-Muller in double from h(2i) and h(2i+1), then rounded to fp32
 *   scale(h, c) = (0.5f + uniform24(h)) * c                  fp32 add then fp32 mul
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tid) {
    return mix64(seed * GOLDEN + tid * 0xD1B54A32D192ED03ULL + 1ULL);
}

static inline uint64_t hash_at(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1ULL) * GOLDEN);
}

static inline float uniform24(uint64_t h) {
    return (float)(h >> 40) * (1.0f / 16777216.0f);
}

/* The plain SplitMix64 sequence from a raw state: out[i] = mix(state + (i+1)*golden).
 * hash_at() is this sequence with state = key; the published test vector
 * (state 1234567) checks it. */
void synth_splitmix64(uint64_t state, int64_t n, uint64_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = hash_at(state, (uint64_t)i);
}

/* Raw 64-bit hashes, for the generator's own self-tests. */
void synth_hash(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, uint64_t* out) {
    uint64_t key = synth_key(seed, tid);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = hash_at(key, start + (uint64_t)i);
}

/* Uniform fp32 on [lo, hi): lo + (hi - lo) * u, evaluated in fp32. */
void synth_uniform(uint64_t seed, uint64_t tid, int64_t n, float lo, float hi, float* out) {
    uint64_t key = synth_key(seed, tid);
    float span = hi - lo;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float u = uniform24(hash_at(key, (uint64_t)i));
        out[i] = lo + span * u;
    }
}

/* Normal(0, std^2), Box-Muller in double, rounded once to fp32. */
void synth_normal(uint64_t seed, uint64_t tid, int64_t n, double std, float* out) {
    uint64_t key = synth_key(seed, tid);
    const double two_pi = 6.283185307179586476925286766559;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t h1 = hash_at(key, 2ULL * (uint64_t)i);
        uint64_t h2 = hash_at(key, 2ULL * (uint64_t)i + 1ULL);
        double u1 = ((double)(h1 >> 11) + 1.0) * (1.0 / 9007199254740992.0); /* (0, 1] */
        double u2 = (double)(h2 >> 11) * (1.0 / 9007199254740992.0);         /* [0, 1) */
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[i] = (float)(z * std);
    }
}

/* Uniform integers on [lo, hi] (inclusive), stored as int8: elements
 * start .. start+n-1 of the tensor (out[i] is element start + i). */
void synth_randint8_at(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, int lo, int hi,
                       int8_t* out) {
    uint64_t key = synth_key(seed, tid);
    uint64_t span = (uint64_t)(hi - lo + 1);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t h = hash_at(key, start + (uint64_t)i);
        out[i] = (int8_t)(lo + (int)(((h >> 32) * span) >> 32));
    }
}

void synth_randint8(uint64_t seed, uint64_t tid, int64_t n, int lo, int hi, int8_t* out) {
    synth_randint8_at(seed, tid, 0, n, lo, hi, out);
}

/*
 * Scales (0.5f + u) * c with c an fp32 constant.  When `special_tid` is
 * non-zero, a hash-chosen subset is overwritten: about 1 in 1024 entries
 * takes one of `n_special` listed values (chosen by the hash) and about 1 in
 * 1024 others takes `exact_value`.  This is how inputs exercise a clamp.
 */
void synth_scale_at(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, float c,
                    uint64_t special_tid, const float* special, int n_special,
                    float exact_value, float* out) {
    uint64_t key = synth_key(seed, tid);
    uint64_t skey = synth_key(seed, special_tid);
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint64_t i = start + (uint64_t)j;
        float u = uniform24(hash_at(key, i));
        float v = (0.5f + u) * c;
        if (special_tid != 0) {
            uint64_t hs = hash_at(skey, i);
            uint64_t sel = hs >> 54;                 /* 10 bits */
            if (sel == 0 && n_special > 0) v = special[(hs >> 20) % (uint64_t)n_special];
            else if (sel == 1) v = exact_value;
        }
        out[j] = v;
    }
}

void synth_scale(uint64_t seed, uint64_t tid, int64_t n, float c,
                 uint64_t special_tid, const float* special, int n_special,
                 float exact_value, float* out) {
    synth_scale_at(seed, tid, 0, n, c, special_tid, special, n_special, exact_value, out);
}

/*
 * Pack int4 codes (values in [-8, 7], one per int8) two per byte along the
 * last axis: element 2i goes to the low nibble of byte i, element 2i+1 to the
 * high nibble, both as 4-bit two's complement.  n_pairs = number of bytes.
 */
void synth_pack_int4(const int8_t* codes, int64_t n_pairs, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_pairs; ++i) {
        uint8_t lo = (uint8_t)codes[2 * i] & 0x0F;
        uint8_t hi = (uint8_t)codes[2 * i + 1] & 0x0F;
        out[i] = (uint8_t)(lo | (hi << 4));
    }
}
