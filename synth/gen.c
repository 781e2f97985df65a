/*
 * Seeded, position-addressable synthetic tensors for Prefix Sliding attention
 * test and benchmark inputs.
 *
 * This module holds no attention, masking or cache arithmetic: it only draws
 * N(0,1) values and, for queries and keys, applies rotary position encoding at
 * the token's Continue-PE position (position IDs keep climbing, so a key is
 * rotated once at its own position and never again; agihunt.info summary of
 * "Prefix Sliding for efficient test-time scaling", paragraph on position
 * encodings).  Every element is a pure function of
 *   (seed, tensor id, layer, sequence, head, position, dimension)
 * so any slice of an arbitrarily long trace can be produced without
 * generating the rest of it.
 *
 * Steps for one row (fixed tensor/layer/seq/head/pos), head size d:
 *   1. key = splitmix64 chain over (seed, tensor, layer, seq, head, pos).
 *      splitmix64 is the counter-based mixer of Steele, Lea & Flood,
 *      "Fast splittable pseudorandom number generators" (OOPSLA 2014), with
 *      the finaliser constants published by S. Vigna.
 *   2. element e: two 53-bit uniforms u1 in (0,1], u2 in [0,1) from
 *      splitmix64(key ^ (2e+1)) and splitmix64(key ^ (2e+2));
 *      z_e = sqrt(-2 ln u1) * cos(2 pi u2)   (Box-Muller, cosine branch).
 *   3. x_e = scale * z_e.
 *   4. tensors 0 (query) and 1 (key) only, when rope_base > 0: rotate the
 *      half-split pairs (x_e, x_{e+d/2}), e < d/2, by the angle
 *      pos * rope_base^(-2e/d), all in double precision.
 *   5. round once to the output type (round-to-nearest-even to bfloat16, or
 *      the nearest float32).
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared gen.c -o libpsgen.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t row_key(uint64_t seed, int64_t tensor, int64_t layer,
                               int64_t seq, int64_t head, int64_t pos) {
    uint64_t h = splitmix64(seed);
    h = splitmix64(h ^ (uint64_t)tensor);
    h = splitmix64(h ^ (uint64_t)layer);
    h = splitmix64(h ^ (uint64_t)seq);
    h = splitmix64(h ^ (uint64_t)head);
    h = splitmix64(h ^ (uint64_t)pos);
    return h;
}

/* round-to-nearest-even from float64 to bfloat16 bits (via the exact float32
 * value nearest to x would double-round, so round directly from the double) */
static inline uint16_t f64_to_bf16_rne(double x) {
    if (isnan(x)) return 0x7FC0;
    /* bf16 has 8 significand bits; find the nearest representable value */
    float f = (float)x;                     /* only used for inf/overflow detection */
    if (isinf(f) && !isinf(x)) {
        /* |x| beyond float range: bf16 shares float's exponent range */
        return (uint16_t)(x > 0 ? 0x7F80 : 0xFF80);
    }
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    double m = frexp(fabs(x), &e);          /* |x| = m * 2^e, m in [0.5, 1) */
    /* normal bf16 numbers: exponent e-1 >= -126 */
    int q = e - 8;                          /* quantum exponent: 8 significant bits */
    if (e - 1 < -126) q = -126 - 7;         /* subnormal range: fixed quantum 2^-133 */
    double scaled = ldexp(fabs(x), -q);     /* exact */
    double r = nearbyint(scaled);           /* current rounding mode: to nearest even */
    double y = ldexp(r, q);
    float fy = (float)y;                    /* exact: y has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &fy, 4);
    uint16_t b = (uint16_t)(u >> 16);
    if (signbit(x)) b |= 0x8000;
    return b;
}

/*
 * Fill out[n_pos][n_heads][d] with rows for positions pos[0..n_pos) and heads
 * head0..head0+n_heads-1.  out_dtype 0 -> uint16 bfloat16 bits, 1 -> float32.
 * Returns 0 on success, -1 on bad arguments.
 */
int psgen_rows(uint64_t seed, int tensor, int layer, int seq, int head0, int n_heads,
               const int64_t* pos, int64_t n_pos, int d, double rope_base,
               double scale, int out_dtype, void* out, int n_threads) {
    if (d <= 0 || (d & 1) || n_heads <= 0 || n_pos < 0 || !out || (n_pos && !pos)) return -1;
    if (out_dtype != 0 && out_dtype != 1) return -1;
    const int half = d / 2;
    const int rotate = (tensor == 0 || tensor == 1) && rope_base > 0.0;
    const int64_t n_rows = n_pos * (int64_t)n_heads;
#pragma omp parallel for schedule(static) num_threads(n_threads > 0 ? n_threads : 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t t = r / n_heads;
        const int hh = head0 + (int)(r % n_heads);
        double x[1024];
        const uint64_t key = row_key(seed, tensor, layer, seq, hh, pos[t]);
        for (int e = 0; e < d; ++e) {
            uint64_t a = splitmix64(key ^ (uint64_t)(2 * e + 1));
            uint64_t b = splitmix64(key ^ (uint64_t)(2 * e + 2));
            double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53;
            double u2 = (double)(b >> 11) * 0x1.0p-53;
            x[e] = scale * sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
        }
        if (rotate) {
            for (int e = 0; e < half; ++e) {
                double theta = (double)pos[t] * pow(rope_base, -2.0 * e / (double)d);
                double c = cos(theta), s = sin(theta);
                double x0 = x[e], x1 = x[e + half];
                x[e] = x0 * c - x1 * s;
                x[e + half] = x0 * s + x1 * c;
            }
        }
        if (out_dtype == 0) {
            uint16_t* o = (uint16_t*)out + r * d;
            for (int e = 0; e < d; ++e) o[e] = f64_to_bf16_rne(x[e]);
        } else {
            float* o = (float*)out + r * d;
            for (int e = 0; e < d; ++e) o[e] = (float)x[e];
        }
    }
    return 0;
}

/* splitmix64 exposed for the generator's own known-answer test */
uint64_t psgen_splitmix64(uint64_t z) { return splitmix64(z); }
