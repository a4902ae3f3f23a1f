/* Drives every oracle entry point over edge inputs, for a build with the
 * host address and undefined-behaviour sanitizers: unit tables starting past
 * element 0, one-element units and buffers, all-zero, subnormal, huge, inf
 * and NaN values, fp16 inputs, up to 64 ranks, planner capacity queries and
 * the chunker's history window.  Prints "ok" and exits 0 when the sanitizers
 * found nothing (they abort the process otherwise). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64(void) {
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static float next_f32(void) {
    const uint32_t r = (uint32_t)(next_u64() >> 40);
    return ((float)r / 16777216.0f - 0.5f) * 1e-2f;
}

static void step(int32_t kind, int32_t W, int64_t n, const int64_t *off, int64_t U, int fill) {
    const size_t esz = kind == ORACLE_F32 ? 4 : 2;
    void **x = calloc((size_t)W, sizeof(void *));
    int8_t **q = calloc((size_t)W, sizeof(int8_t *));
    float **s = calloc((size_t)W, sizeof(float *));
    for (int32_t w = 0; w < W; ++w) {
        x[w] = malloc((size_t)n * esz);
        q[w] = malloc((size_t)n);
        s[w] = malloc((size_t)U * sizeof(float));
        for (int64_t i = 0; i < n; ++i) {
            if (kind == ORACLE_F32) {
                float v = next_f32();
                if (fill == 1) v = 0.0f;
                if (fill == 2) v = ldexpf((float)(i % 200), -149);
                if (fill == 3) v = (i % 2) ? 3.0e38f : -3.0e38f;
                if (fill == 4 && i % 97 == 5) v = (i % 3) ? INFINITY : NAN;
                ((float *)x[w])[i] = v;
            } else {
                ((uint16_t *)x[w])[i] = (uint16_t)next_u64();
            }
        }
    }
    const float in_mul = kind == ORACLE_F32 ? 1.0f : 0x1p-16f;
    uint32_t *amax = malloc((size_t)U * sizeof(uint32_t));
    float *r = malloc((size_t)n * sizeof(float));
    float *ref = malloc((size_t)n * sizeof(float));
    float *s_out = malloc((size_t)U * sizeof(float));
    int8_t *q_out = malloc((size_t)n);
    double *stats = malloc((size_t)U * ORACLE_STATS * sizeof(double));
    for (int32_t w = 0; w < W; ++w) {
        oracle_quantize_units(x[w], kind, in_mul, n, off, U, amax, s[w], q[w]);
        oracle_quantize_with_amax(x[w], kind, in_mul, n, off, U, amax, s[w], q[w]);
    }
    oracle_reduce_dequant((const int8_t *const *)q, (const float *const *)s, W, n, off, U, r);
    oracle_requantize(r, n, off, U, s_out, q_out);
    oracle_sum_f32((const void *const *)x, kind, in_mul, W, n, 0, ref);
    oracle_sum_f32((const void *const *)x, kind, in_mul, W, n, 1, ref);
    oracle_error_report(q_out, s_out, ref, n, off, U, stats);
    for (int32_t w = 0; w < W; ++w) {
        free(x[w]);
        free(q[w]);
        free(s[w]);
    }
    free(x); free(q); free(s); free(amax); free(r); free(ref); free(s_out); free(q_out); free(stats);
}

int main(void) {
    /* unit tables: one element, ragged units, a table starting past 0 */
    const int64_t one[2] = {0, 1};
    const int64_t ragged[6] = {0, 1, 17, 18, 300, 1001};
    const int64_t late[4] = {7, 8, 100, 333};
    for (int fill = 0; fill <= 4; ++fill) {
        step(ORACLE_F32, 1, 1, one, 1, fill);
        step(ORACLE_F32, 3, 1001, ragged, 5, fill);
        step(ORACLE_F32, 2, 333, late, 3, fill);
    }
    step(ORACLE_F16, 4, 1001, ragged, 5, 0);
    step(ORACLE_F16, 64, 333, late, 3, 0);
    step(ORACLE_F32, 64, 1001, ragged, 5, 0);

    /* planner: capacity query, exact capacity, one element, fp16 sizes */
    int64_t count = 0, offs[64];
    const int64_t sizes[6] = {1, 32767, 32768, 65536, 1000000, 1 << 20};
    for (int i = 0; i < 6; ++i) {
        for (int32_t e = 2; e <= 4; e += 2) {
            (void)oracle_plan_chunks(sizes[i], e, 131072, 64, NULL, 0, &count);
            if (count + 1 <= 64) (void)oracle_plan_chunks(sizes[i], e, 131072, 64, offs, count + 1, &count);
        }
    }

    /* chunker: empty history, a window shorter than the history */
    int64_t hs[300];
    double lat[300];
    for (int i = 0; i < 300; ++i) {
        hs[i] = (int64_t)(32768 << (next_u64() % 6));
        lat[i] = 1e-6 * (double)(1 + next_u64() % 1000);
    }
    (void)oracle_chunker_predict(hs, lat, 0, 100, 0.25, 131072);
    (void)oracle_chunker_predict(hs, lat, 300, 100, 0.25, 131072);
    (void)oracle_chunker_predict(hs, lat, 50, 100, 1.0, 131072);

    /* scalar helpers over every fp16 pattern and special floats */
    for (uint32_t h = 0; h < 65536; ++h) (void)oracle_half_to_float((uint16_t)h);
    const float vals[6] = {0.0f, -0.0f, 1e-45f, 3.0e38f, INFINITY, NAN};
    for (int i = 0; i < 6; ++i)
        for (int j = 0; j < 6; ++j) (void)oracle_code(vals[i], vals[j]);
    puts("ok");
    return 0;
}
