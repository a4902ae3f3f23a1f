/*
 * oracle.h -- plain, single-threaded CPU oracle for the INT8-compressed
 * gradient AllReduce compute.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this code: it exists so that tests, the smoke check and the
 * benchmark's CPU-baseline leg can compare the HIP library against an
 * independent, obviously correct implementation.  It shares no source with
 * the HIP library.
 *
 * Source of the method: the pipelined HCCL AllReduce article
 * (bjdmk.com.cn/news/6235379):
 *   - §2.1  (three-stage pipeline, data chunking): the dynamic_chunk rule,
 *   - §2.2.1 (gradient quantization compression): quantize_gradient, the
 *            int8 codes + fp32 scale pair, and the INT8 AllReduce primitive,
 *   - §6.1  (mixed-precision pipeline): unscale before quantizing.
 *
 * All buffers are host memory owned by the caller.  Every function is pure
 * (no global state) and single-threaded.  Built with -O2 -ffp-contract=off,
 * no fast-math and no flush-to-zero, so every float operation below is one
 * IEEE-754 binary32 operation rounded to nearest-even.
 */
#ifndef GQ_ORACLE_H
#define GQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input element kinds. */
#define ORACLE_F32 0
#define ORACLE_F16 1

/* Chunk plan (§2.1, dynamic_chunk): the offsets of torch.chunk(t, k) with
 * k = max(1, numel*elem_bytes // (chunk_bytes - chunk_bytes % align_bytes)).
 * Writes count+1 offsets to off_out when cap >= count+1 and sets *count_out.
 * Returns 0 on success, 1 if cap is too small (count still set), -1 on bad
 * arguments. */
int oracle_plan_chunks(int64_t numel, int32_t elem_bytes, int64_t chunk_bytes,
                       int32_t align_bytes, int64_t *off_out, int64_t cap,
                       int64_t *count_out);

/* IEEE-754 binary16 bit pattern -> binary32 value (exact). */
float oracle_half_to_float(uint16_t h);

/* Load + unscale (§6.1): g[i] = float(x[i]) * in_mul, one rounding. */
void oracle_load(const void *x, int32_t kind, float in_mul, int64_t n, float *g);

/* max |g| over g[0..len) as the bit pattern of |g| (sign bit cleared),
 * compared as unsigned integers: NaN beats +inf beats every finite value. */
uint32_t oracle_absmax_bits(const float *g, int64_t len);

/* s = max|g| / 127 in binary32 (§2.2.1). */
float oracle_scale(uint32_t amax_bits);

/* One int8 code (§2.2.1): round(g/s) half-to-even, clamped to [-128, 127].
 * s == 0 gives 0; a NaN quotient gives 0. */
int8_t oracle_code(float g, float s);

/* Quantize one gradient with one scale per unit.  Units are the ranges
 * [off[u], off[u+1]) of g; off[0] == 0, off[n_units] == n.
 * scale_out[n_units], q_out[n]; amax_out[n_units] may be NULL. */
void oracle_quantize_units(const void *x, int32_t kind, float in_mul, int64_t n,
                           const int64_t *off, int64_t n_units,
                           uint32_t *amax_out, float *scale_out, int8_t *q_out);

/* Quantize with given per-unit absmax bits (no max pass). */
void oracle_quantize_with_amax(const void *x, int32_t kind, float in_mul,
                               int64_t n, const int64_t *off, int64_t n_units,
                               const uint32_t *amax, float *scale_out,
                               int8_t *q_out);

/* Reduction step of the INT8 AllReduce on one device: for every element,
 *   r = (((+0 + q_0*s_0) + q_1*s_1) + ...) + q_{W-1}*s_{W-1}
 * with each product and each sum rounded to binary32, ranks in order.
 * q[w] points to rank w's n codes, s[w] to its n_units scales. */
void oracle_reduce_dequant(const int8_t *const *q, const float *const *s,
                           int32_t W, int64_t n, const int64_t *off,
                           int64_t n_units, float *r_out);

/* Requantize the reduced sum with the same units: quantize of fp32 r. */
void oracle_requantize(const float *r, int64_t n, const int64_t *off,
                       int64_t n_units, float *scale_out, int8_t *q_out);

/* ---- Unquantized A/B path and error report ------------------------------
 * The article's troubleshooting section (gradient anomalies) checks whether
 * a problem comes from precision by switching gradient quantization off;
 * the torchtitan-npu article's mixed-precision listing all-reduces fp32
 * gradients and divides them by the data-parallel group size.  These two
 * functions give that fp32 reference next to the INT8 path and measure the
 * INT8 result against it. */

/* fp32 AllReduce reduction on one device, no quantization:
 *   r = (((+0 + g_0) + g_1) + ...) + g_{W-1},  g_w = load(x_w) as above,
 * each sum rounded to binary32, ranks in order; with mean != 0 the sum is
 * then divided by W (one binary32 division). */
void oracle_sum_f32(const void *const *x, int32_t kind, float in_mul, int32_t W,
                    int64_t n, int32_t mean, float *r_out);

/* Per-unit error statistics of an INT8 result against a reference, all in
 * binary64.  d_i = float(q_i) * s_u (binary32, one rounding) is the value
 * the codes stand for; ref_i is the reference.  Field order of the 10
 * doubles written per unit to stats_out[10*u ...]:
 *   0 max_abs_err   max_i |d_i - ref_i|     (difference in binary64)
 *   1 max_abs_ref   max_i |ref_i|
 *   2 max_rel_err   max_abs_err / max_abs_ref
 *   3 sum_abs_err   sum_i |d_i - ref_i|     (element order)
 *   4 sum_abs_ref   sum_i |ref_i|
 *   5 mean_rel_err  sum_abs_err / sum_abs_ref
 *   6 sum_dd        sum_i d_i^2
 *   7 sum_rr        sum_i ref_i^2
 *   8 sum_dr        sum_i d_i ref_i
 *   9 cos           sum_dr / sqrt(sum_dd * sum_rr)
 * Maxima compare |x| as binary64 bit patterns (a NaN anywhere gives NaN).
 * A ratio 0/0 is 0 (an all-zero unit has no error); cos is 1 when both
 * vectors are zero and 0 when exactly one is. */
#define ORACLE_STATS 10
void oracle_error_report(const int8_t *q, const float *scale, const float *ref,
                         int64_t n, const int64_t *off, int64_t n_units,
                         double *stats_out);

/* ---- Adaptive chunk size (§6.2 adaptive chunking) -------------------------
 * The article keeps the last 100 (chunk size, latency) observations and
 * predicts the best chunk size from them with an exponentially weighted
 * moving average; the prediction step itself is not printed.  Reading
 * taken here: each observation's cost is its latency per byte of chunk;
 * for every chunk size present in the history, the costs of that size are
 * averaged in history order (oldest first) as e = alpha * x + (1 - alpha) * e,
 * starting from the first such cost; the size with the smallest average
 * wins, ties going to the larger size; an empty history gives the default.
 *
 * sizes[i], lat[i] for i < count are all observations in arrival order;
 * only the last `capacity` of them form the history.  All arithmetic is
 * binary64, one rounding per operation. */
int64_t oracle_chunker_predict(const int64_t *sizes, const double *lat, int64_t count,
                               int32_t capacity, double alpha, int64_t default_bytes);

#ifdef __cplusplus
}
#endif
#endif /* GQ_ORACLE_H */
