/*
 * datagen.c -- seeded synthetic gradient generators.
 *
 * Shared by the tests, the smoke check and the benchmark to feed the SAME
 * host buffers to the HIP library and to the CPU oracle.  It holds none of
 * the compression method's arithmetic: only random numbers and value
 * encodings of the synthetic workloads.
 *
 * Random numbers come from a counter-based generator: element i of a stream
 * with key k is the SplitMix64 output for state k + (i+1)*0x9E3779B97F4A7C15
 * (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014), so any element range can be generated on its own and the
 * result does not depend on the thread count.  Normal deviates use the
 * Box-Muller transform in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* i-th output of a SplitMix64 generator whose state starts at key */
static inline uint64_t sm_at(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GOLDEN);
}

/* uniform double in [0, 1) with 53 random bits */
static inline double u53(uint64_t z)
{
    return (double)(z >> 11) * 0x1.0p-53;
}

/* standard normal: Box-Muller on the counters 2i and 2i+1 of the stream */
static inline double normal_at(uint64_t key, uint64_t i)
{
    double u1 = 1.0 - u53(sm_at(key, 2 * i));   /* (0, 1] */
    double u2 = u53(sm_at(key, 2 * i + 1));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* A stream key from (seed, a, b, c, d): a chain of SplitMix64 steps. */
uint64_t dg_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d)
{
    uint64_t k = mix64(seed + GOLDEN);
    k = mix64(k ^ (a + 1) * GOLDEN);
    k = mix64(k ^ (b + 1) * GOLDEN);
    k = mix64(k ^ (c + 1) * GOLDEN);
    k = mix64(k ^ (d + 1) * GOLDEN);
    return k;
}

uint64_t dg_u64(uint64_t key, uint64_t i) { return sm_at(key, i); }
double dg_uniform(uint64_t key, uint64_t i) { return u53(sm_at(key, i)); }
double dg_normal(uint64_t key, uint64_t i) { return normal_at(key, i); }

/* out[j] = fp32(sigma * Z(first + j)); with probability p_zero (drawn from
 * the second stream zkey) the element is exactly +0. */
void dg_fill_normal_f32(uint64_t key, uint64_t zkey, double p_zero,
                        uint64_t first, int64_t n, double sigma, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint64_t i = first + (uint64_t)j;
        float v = (float)(sigma * normal_at(key, i));
        if (p_zero > 0.0 && u53(sm_at(zkey, i)) < p_zero)
            v = 0.0f;
        out[j] = v;
    }
}

/* out[j] = fp32(scale * Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3)): a Student-t
 * deviate with 3 degrees of freedom.  The four normals are both outputs of
 * two Box-Muller pairs, on the counters 4i .. 4i+3. */
void dg_fill_student_t3_f32(uint64_t key, uint64_t first, int64_t n,
                            double scale, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint64_t i = 4 * (first + (uint64_t)j);
        double ra = sqrt(-2.0 * log(1.0 - u53(sm_at(key, i))));
        double ta = 6.283185307179586 * u53(sm_at(key, i + 1));
        double rb = sqrt(-2.0 * log(1.0 - u53(sm_at(key, i + 2))));
        double tb = 6.283185307179586 * u53(sm_at(key, i + 3));
        double z0 = ra * cos(ta), z1 = ra * sin(ta);
        double z2 = rb * cos(tb), z3 = rb * sin(tb);
        double chi = (z1 * z1 + z2 * z2 + z3 * z3) / 3.0;
        out[j] = (float)(scale * z0 / sqrt(chi));
    }
}

/* binary32 -> binary16 bit pattern, round to nearest even (value encoding of
 * the fp16 workload; overflow goes to inf). */
static uint16_t f32_to_f16_bits(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u)  /* inf or NaN */
        return (uint16_t)(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
    if (ax >= 0x477ff000u)  /* rounds to >= 65520: overflow */
        return (uint16_t)(sign | 0x7c00u);
    if (ax < 0x38800000u) { /* below 2^-14: binary16 subnormal or zero */
        /* value = ax_float; subnormal quantum 2^-24 */
        float a;
        memcpy(&a, &ax, 4);
        float q = a * 16777216.0f;           /* exact: times 2^24 */
        float r = rintf(q);                   /* half to even */
        return (uint16_t)(sign | (uint32_t)r);
    }
    /* normal: drop 13 fraction bits with round to nearest even */
    uint32_t e = (ax >> 23) - 127 + 15;
    uint32_t m = ax & 0x7fffffu;
    uint32_t h = (e << 10) | (m >> 13);
    uint32_t rest = m & 0x1fffu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u)))
        h += 1;  /* carry into the exponent is the correct result */
    return (uint16_t)(sign | h);
}

/* out[j] = fp16(fp32(sigma * Z(first + j)) * mul): a loss-scaled fp16
 * gradient (mul = the loss scale). */
void dg_fill_normal_f16(uint64_t key, uint64_t first, int64_t n, double sigma,
                        double mul, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint64_t i = first + (uint64_t)j;
        float v = (float)(sigma * mul * normal_at(key, i));
        out[j] = f32_to_f16_bits(v);
    }
}

/* Denormal-rich values: element i is, with probability 1/2 (counter 2i of
 * dkey), a subnormal binary32 with a random sign and a uniform non-zero
 * 23-bit fraction (counter 2i+1 of dkey); otherwise fp32(sigma * Z(i)). */
void dg_fill_denormal_f32(uint64_t key, uint64_t dkey, uint64_t first,
                          int64_t n, double sigma, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint64_t i = first + (uint64_t)j;
        if (sm_at(dkey, 2 * i) & 1ull) {
            uint64_t z = sm_at(dkey, 2 * i + 1);
            uint32_t frac = (uint32_t)(z % 0x7fffffull) + 1u; /* 1 .. 2^23-1 */
            uint32_t bits = frac | ((z >> 63) ? 0x80000000u : 0u);
            float v;
            memcpy(&v, &bits, 4);
            out[j] = v;
        } else {
            out[j] = (float)(sigma * normal_at(key, i));
        }
    }
}

/* 64-bit FNV-1a over a byte buffer (input checksums for the records). */
uint64_t dg_checksum(const void *p, int64_t nbytes)
{
    const unsigned char *b = (const unsigned char *)p;
    uint64_t h = 0xcbf29ce484222325ull;
    for (int64_t i = 0; i < nbytes; ++i) {
        h ^= b[i];
        h *= 0x100000001b3ull;
    }
    return h;
}
