/*
 * oracle.c -- plain, single-threaded CPU oracle (TEST INFRASTRUCTURE ONLY;
 * see oracle.h).  Each function follows one step of the method as the
 * pipelined HCCL AllReduce article (bjdmk.com.cn/news/6235379) states it,
 * in the article's order, with no blocking, fusion or reordering.
 *
 * Readings taken where the article is silent (each is also listed in the
 * design notes):
 *   R1  the INT8 AllReduce primitive of §2.2.1 is not defined there; its
 *       reduction step is read as: dequantize each rank's codes with that
 *       rank's scale, add the contributions in fp32 in rank order 0..W-1
 *       (a multiply, then an add, two roundings, no fused multiply-add),
 *       then quantize the sum again with a fresh absmax scale.
 *   R2  an all-zero unit makes the article's formula divide 0 by 0; the
 *       scale is then 0 and every code is 0 (also for a subnormal max whose
 *       scale rounds to 0).
 *   R3  a quotient g/s that is NaN (only possible when the unit holds a NaN
 *       or an infinity) gives code 0; IEEE arithmetic is kept everywhere
 *       else, so an overflowed sum keeps its inf/NaN.
 *   R4  the chunk plan is exactly torch.chunk(t, k): pieces of ceil(n/k)
 *       elements, the last one shorter, ceil(n / ceil(n/k)) pieces.
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>

/* §2.1 dynamic_chunk: the chunk count is the tensor's byte size divided by
 * the base chunk size rounded down to the alignment, at least 1; the pieces
 * are those of torch.chunk (R4). */
int oracle_plan_chunks(int64_t numel, int32_t elem_bytes, int64_t chunk_bytes,
                       int32_t align_bytes, int64_t *off_out, int64_t cap,
                       int64_t *count_out)
{
    if (numel < 1 || elem_bytes < 1 || chunk_bytes < 1 || align_bytes < 1 ||
        count_out == NULL)
        return -1;
    int64_t denom = chunk_bytes - chunk_bytes % align_bytes;
    if (denom < 1)
        return -1;
    int64_t nbytes = numel * (int64_t)elem_bytes;
    int64_t k = nbytes / denom;
    if (k < 1)
        k = 1;
    /* torch.chunk: split size ceil(n/k); as many pieces as that size needs */
    int64_t c = (numel + k - 1) / k;
    int64_t count = (numel + c - 1) / c;
    *count_out = count;
    if (off_out == NULL || cap < count + 1)
        return 1;
    for (int64_t j = 0; j < count; ++j)
        off_out[j] = j * c;
    off_out[count] = numel;
    return 0;
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0: value = fraction * 2^-24; exponent 31: inf (fraction 0) or
 * NaN; otherwise (1024 + fraction) * 2^(exponent - 25).  Every binary16
 * value is exactly representable in binary32, so ldexpf is exact here. */
float oracle_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexpf((float)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* §6.1: the loss-scaled fp16 gradient is unscaled before quantizing; the
 * unscale is one binary32 multiply by in_mul (1/S).  fp32 input uses
 * in_mul = 1. */
void oracle_load(const void *x, int32_t kind, float in_mul, int64_t n, float *g)
{
    for (int64_t i = 0; i < n; ++i) {
        float v;
        if (kind == ORACLE_F16)
            v = oracle_half_to_float(((const uint16_t *)x)[i]);
        else
            v = ((const float *)x)[i];
        g[i] = v * in_mul;
    }
}

static uint32_t f2u(float f)
{
    union { float f; uint32_t u; } c;
    c.f = f;
    return c.u;
}

static float u2f(uint32_t u)
{
    union { float f; uint32_t u; } c;
    c.u = u;
    return c.f;
}

/* §2.2.1: torch.max(torch.abs(grad)).  |g| is g with its sign bit cleared;
 * for non-negative binary32 values the bit patterns order like the values,
 * and NaN patterns sit above +inf, so a NaN anywhere wins (as torch.max
 * propagates NaN). */
uint32_t oracle_absmax_bits(const float *g, int64_t len)
{
    uint32_t m = 0;
    for (int64_t i = 0; i < len; ++i) {
        uint32_t a = f2u(g[i]) & 0x7fffffffu;
        if (a > m)
            m = a;
    }
    return m;
}

/* §2.2.1: scale = max|g| / 127.0, a binary32 division (the tensor is fp32
 * and 127.0 is a Python scalar, so torch keeps fp32). */
float oracle_scale(uint32_t amax_bits)
{
    return u2f(amax_bits) / 127.0f;
}

/* §2.2.1: clamp(round(g / scale), -128, 127) cast to int8.  torch.round
 * rounds halves to even, which is rintf under the default rounding mode.
 * R2: s == 0 gives 0.  R3: NaN quotient gives 0. */
int8_t oracle_code(float g, float s)
{
    if (s == 0.0f)
        return 0;
    float t = g / s;
    if (isnan(t))
        return 0;
    float r = rintf(t);
    if (r < -128.0f)
        r = -128.0f;
    if (r > 127.0f)
        r = 127.0f;
    return (int8_t)(int)r;
}

static void quantize_one_unit(const float *g, int64_t len, float s, int8_t *q)
{
    for (int64_t i = 0; i < len; ++i)
        q[i] = oracle_code(g[i], s);
}

/* quantize_gradient applied to every unit: load, absmax, scale, codes. */
void oracle_quantize_units(const void *x, int32_t kind, float in_mul, int64_t n,
                           const int64_t *off, int64_t n_units,
                           uint32_t *amax_out, float *scale_out, int8_t *q_out)
{
    (void)n;
    int64_t esz = (kind == ORACLE_F16) ? 2 : 4;
    for (int64_t u = 0; u < n_units; ++u) {
        int64_t a = off[u], len = off[u + 1] - off[u];
        float *g = (float *)malloc((size_t)len * sizeof(float));
        if (g == NULL)
            abort();
        oracle_load((const char *)x + a * esz, kind, in_mul, len, g);
        uint32_t m = oracle_absmax_bits(g, len);
        float s = oracle_scale(m);
        if (amax_out)
            amax_out[u] = m;
        scale_out[u] = s;
        quantize_one_unit(g, len, s, q_out + a);
        free(g);
    }
}

/* Same codes from a max already taken (the absmax and quantize steps run as
 * two separate calls). */
void oracle_quantize_with_amax(const void *x, int32_t kind, float in_mul,
                               int64_t n, const int64_t *off, int64_t n_units,
                               const uint32_t *amax, float *scale_out,
                               int8_t *q_out)
{
    (void)n;
    int64_t esz = (kind == ORACLE_F16) ? 2 : 4;
    for (int64_t u = 0; u < n_units; ++u) {
        int64_t a = off[u], len = off[u + 1] - off[u];
        float *g = (float *)malloc((size_t)len * sizeof(float));
        if (g == NULL)
            abort();
        oracle_load((const char *)x + a * esz, kind, in_mul, len, g);
        float s = oracle_scale(amax[u]);
        scale_out[u] = s;
        quantize_one_unit(g, len, s, q_out + a);
        free(g);
    }
}

/* R1: the reduction of the INT8 AllReduce (§2.2.1) on one device.  Each
 * rank's contribution is its code times its unit's scale (one rounding);
 * contributions are added to a +0 accumulator in rank order (one rounding
 * each). */
void oracle_reduce_dequant(const int8_t *const *q, const float *const *s,
                           int32_t W, int64_t n, const int64_t *off,
                           int64_t n_units, float *r_out)
{
    (void)n;
    for (int64_t u = 0; u < n_units; ++u) {
        for (int64_t i = off[u]; i < off[u + 1]; ++i) {
            float acc = 0.0f;
            for (int32_t w = 0; w < W; ++w) {
                float d = (float)q[w][i] * s[w][u];
                acc = acc + d;
            }
            r_out[i] = acc;
        }
    }
}

/* R1: the summed gradient is quantized again, one fresh scale per unit. */
void oracle_requantize(const float *r, int64_t n, const int64_t *off,
                       int64_t n_units, float *scale_out, int8_t *q_out)
{
    oracle_quantize_units(r, ORACLE_F32, 1.0f, n, off, n_units, NULL,
                          scale_out, q_out);
}

/* fp32 reference for the A/B check: the same rank-order reduction as the
 * INT8 path, on the unquantized gradients. */
void oracle_sum_f32(const void *const *x, int32_t kind, float in_mul, int32_t W,
                    int64_t n, int32_t mean, float *r_out)
{
    float *g = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (g == NULL)
        abort();
    for (int64_t i = 0; i < n; ++i)
        r_out[i] = 0.0f;
    for (int32_t rank = 0; rank < W; ++rank) {
        oracle_load(x[rank], kind, in_mul, n, g);
        for (int64_t i = 0; i < n; ++i)
            r_out[i] = r_out[i] + g[i];
    }
    if (mean)
        for (int64_t i = 0; i < n; ++i)
            r_out[i] = r_out[i] / (float)W;
    free(g);
}

static uint64_t d2u(double d)
{
    union { double d; uint64_t u; } c;
    c.d = d;
    return c.u;
}

static double u2d(uint64_t u)
{
    union { double d; uint64_t u; } c;
    c.u = u;
    return c.d;
}

/* |a| as a bit pattern, ordered like the value, NaN above +inf. */
static uint64_t abs_bits(double a)
{
    return d2u(a) & 0x7fffffffffffffffull;
}

static double ratio_or_zero(double a, double b)
{
    if (a == 0.0 && b == 0.0)
        return 0.0;
    return a / b;
}

void oracle_error_report(const int8_t *q, const float *scale, const float *ref,
                         int64_t n, const int64_t *off, int64_t n_units,
                         double *stats_out)
{
    (void)n;
    for (int64_t u = 0; u < n_units; ++u) {
        uint64_t max_err = 0, max_ref = 0;
        double sum_err = 0.0, sum_ref = 0.0, dd = 0.0, rr = 0.0, dr = 0.0;
        for (int64_t i = off[u]; i < off[u + 1]; ++i) {
            double d = (double)((float)q[i] * scale[u]);
            double r = (double)ref[i];
            double e = fabs(d - r);
            if (abs_bits(e) > max_err)
                max_err = abs_bits(e);
            if (abs_bits(r) > max_ref)
                max_ref = abs_bits(r);
            sum_err = sum_err + e;
            sum_ref = sum_ref + fabs(r);
            dd = dd + d * d;
            rr = rr + r * r;
            dr = dr + d * r;
        }
        double *o = stats_out + ORACLE_STATS * u;
        o[0] = u2d(max_err);
        o[1] = u2d(max_ref);
        o[2] = ratio_or_zero(o[0], o[1]);
        o[3] = sum_err;
        o[4] = sum_ref;
        o[5] = ratio_or_zero(sum_err, sum_ref);
        o[6] = dd;
        o[7] = rr;
        o[8] = dr;
        if (dd == 0.0 && rr == 0.0)
            o[9] = 1.0;
        else if (dd == 0.0 || rr == 0.0)
            o[9] = 0.0;
        else
            o[9] = dr / sqrt(dd * rr);
    }
}

/* §6.2 DynamicChunker: history of the last `capacity` observations, a
 * per-size exponentially weighted moving average of latency per byte, the
 * size with the lowest average (see oracle.h for the reading). */
int64_t oracle_chunker_predict(const int64_t *sizes, const double *lat, int64_t count,
                               int32_t capacity, double alpha, int64_t default_bytes)
{
    int64_t first = count > capacity ? count - capacity : 0;
    int64_t best_size = default_bytes;
    double best_cost = 0.0;
    int have_best = 0;
    for (int64_t i = first; i < count; ++i) {
        int64_t c = sizes[i];
        int seen_before = 0;
        for (int64_t j = first; j < i; ++j)
            if (sizes[j] == c)
                seen_before = 1;
        if (seen_before)
            continue;
        /* the average of size c over the history, oldest first */
        double e = 0.0;
        int started = 0;
        for (int64_t j = i; j < count; ++j) {
            if (sizes[j] != c)
                continue;
            double x = lat[j] / (double)c;
            if (!started) {
                e = x;
                started = 1;
            } else {
                e = alpha * x + (1.0 - alpha) * e;
            }
        }
        if (!have_best || e < best_cost || (e == best_cost && c > best_size)) {
            best_cost = e;
            best_size = c;
            have_best = 1;
        }
    }
    return best_size;
}
