// gq_check.hip -- gfx950 kernels of the precision check with quantization
// switched off (pipelined HCCL AllReduce article, bjdmk.com.cn/news/6235379,
// §5.2 gradient anomalies: switch gradient quantization off to see whether
// a problem is one of precision).
//
//   k_sum_f32          the fp32 AllReduce reduction of the unquantized
//                      gradients: r = (((+0 + g_0) + g_1) + ...) + g_{W-1},
//                      g_w = float(x_w) * in_mul, binary32 adds in rank
//                      order, optionally divided by W (the averaged gradient
//                      of data-parallel training, as in the torchtitan-npu
//                      article's mixed-precision listing).  Elementwise and
//                      HBM-bound: W*n*e bytes in, 4n out.
//   k_report_tiles     per-tile binary64 statistics of an INT8 result
//                      d = fl32(float(q) * s) against an fp32 reference.
//   k_report_finalize  per-unit combination of the tiles (one wave per
//                      unit, fixed order) and the derived ratios and cosine.
//
// The report's maxima are exact (a binary64 difference of two binary32
// values is rounded once, and rounding is monotone); its sums are taken in
// a fixed order (per lane, then a butterfly over the wave, then waves in
// order; per unit, tiles strided over a wave's lanes, then a butterfly),
// so they repeat bit for bit from run to run.
#include <hip/hip_fp16.h>

#include "gq_internal.h"

namespace gq {
namespace {

constexpr int SUM_BLOCK = 256;
constexpr int SUM_SLOTS = 2;      // 16-byte input slots per lane and rank group
constexpr int SUM_RG = 8;         // ranks loaded together
constexpr int REPORT_BLOCK = R_BLOCK;  // one work group per reduce-table tile
constexpr int REPORT_V = 16;
constexpr uint64_t kAbs64 = 0x7fffffffffffffffull;

// Streaming accesses: the sum reads its inputs once and writes its result
// once, so its whole-slot loads and stores carry the non-temporal hint (the
// nt bit).  The report keeps plain loads: it reads a reference and codes
// that were usually written just before, and the hint made it slower.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(float *p, float a, float b, float c, float d) {
    const f32x4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}

__device__ __forceinline__ float half_bits_to_float(uint32_t b) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(b)));
}

// Element k of a raw 16-byte slot of binary32 or binary16 values.
template <typename TIn>
__device__ __forceinline__ float slot_elem(const uint4 &v, int k);

template <>
__device__ __forceinline__ float slot_elem<float>(const uint4 &v, int k) {
    return __uint_as_float(k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w);
}

template <>
__device__ __forceinline__ float slot_elem<__half>(const uint4 &v, int k) {
    const uint32_t w = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
    return half_bits_to_float((k & 1) ? (w >> 16) : (w & 0xffffu));
}

// ---- fp32 reference sum -------------------------------------------------------
// Lane l of work group b owns slots (b * SUM_SLOTS + s) * SUM_BLOCK + l of
// every rank.  Ranks are loaded SUM_RG at a time (all of a group's loads in
// flight together) and added in rank order.  Only the buffer's last slot
// can be short: it is read and written element by element.
template <typename TIn, bool MUL, bool MEAN>
__global__ __launch_bounds__(SUM_BLOCK) void k_sum_f32(const SArgs a) {
    constexpr int V = 16 / sizeof(TIn);
    const int64_t nslots = (a.n + V - 1) / V;
    const int64_t nfull = a.n / V;
    int64_t js[SUM_SLOTS];
#pragma unroll
    for (int s = 0; s < SUM_SLOTS; ++s)
        js[s] = (static_cast<int64_t>(blockIdx.x) * SUM_SLOTS + s) * SUM_BLOCK + threadIdx.x;
    float acc[SUM_SLOTS][V];
#pragma unroll
    for (int s = 0; s < SUM_SLOTS; ++s)
#pragma unroll
        for (int k = 0; k < V; ++k) acc[s][k] = 0.0f;
    for (int w0 = 0; w0 < a.W; w0 += SUM_RG) {
        uint4 raw[SUM_RG][SUM_SLOTS];
#pragma unroll
        for (int r = 0; r < SUM_RG; ++r) {
            if (w0 + r >= a.W) break;
            const uint4 *xv = static_cast<const uint4 *>(a.x[w0 + r]);
#pragma unroll
            for (int s = 0; s < SUM_SLOTS; ++s)
                raw[r][s] = js[s] < nfull ? load_stream(xv + js[s]) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < SUM_RG; ++r) {
            if (w0 + r >= a.W) break;
#pragma unroll
            for (int s = 0; s < SUM_SLOTS; ++s) {
                if (js[s] >= nfull && js[s] < nslots) {
                    // the short last slot: element by element
                    uint32_t w[4] = {0, 0, 0, 0};
                    for (int k = 0; k < V; ++k) {
                        const int64_t i = js[s] * V + k;
                        if (i >= a.n) break;
                        uint32_t bits;
                        if constexpr (V == 4)
                            bits = static_cast<const uint32_t *>(a.x[w0 + r])[i];
                        else
                            bits = static_cast<const uint16_t *>(a.x[w0 + r])[i];
                        const int sh = (V == 4) ? 0 : 16 * (k & 1);
                        const int wi = (V == 4) ? k : k >> 1;
                        w[wi] |= bits << sh;
                    }
                    raw[r][s] = make_uint4(w[0], w[1], w[2], w[3]);
                }
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    float g = slot_elem<TIn>(raw[r][s], k);
                    if (MUL) g = __fmul_rn(g, a.in_mul);
                    acc[s][k] = __fadd_rn(acc[s][k], g);
                }
            }
        }
    }
    const float wf = static_cast<float>(a.W);
#pragma unroll
    for (int s = 0; s < SUM_SLOTS; ++s) {
        if (js[s] >= nslots) continue;
        if (MEAN) {
#pragma unroll
            for (int k = 0; k < V; ++k) acc[s][k] = __fdiv_rn(acc[s][k], wf);
        }
        const int64_t i0 = js[s] * V;
        if (js[s] < nfull) {
#pragma unroll
            for (int k = 0; k < V / 4; ++k)
                store_stream(a.r + i0 + 4 * k, acc[s][4 * k], acc[s][4 * k + 1], acc[s][4 * k + 2],
                             acc[s][4 * k + 3]);
        } else {
            for (int k = 0; k < V; ++k)
                if (i0 + k < a.n) a.r[i0 + k] = acc[s][k];
        }
    }
}

// ---- error report -----------------------------------------------------------

struct Stats {
    uint64_t max_err, max_ref;  // |x| as binary64 bit patterns (NaN above inf)
    double err, ref, dd, rr, dr;
};

__device__ __forceinline__ uint64_t abs_bits64(double v) {
    return static_cast<uint64_t>(__double_as_longlong(v)) & kAbs64;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ double shfl_xor_d(double v, int o) {
    const long long b = __double_as_longlong(v);
    const int lo = __shfl_xor(static_cast<int>(b & 0xffffffff), o, 64);
    const int hi = __shfl_xor(static_cast<int>(b >> 32), o, 64);
    return __longlong_as_double((static_cast<long long>(hi) << 32) |
                                static_cast<long long>(static_cast<uint32_t>(lo)));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
    const int lo = __shfl_xor(static_cast<int>(v & 0xffffffffu), o, 64);
    const int hi = __shfl_xor(static_cast<int>(v >> 32), o, 64);
    return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// Butterfly over the wave: every lane ends with the same totals (IEEE
// addition is commutative, so partner lanes add the same two values).
__device__ __forceinline__ void wave_stats(Stats &s) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        s.max_err = umax64(s.max_err, shfl_xor_u64(s.max_err, o));
        s.max_ref = umax64(s.max_ref, shfl_xor_u64(s.max_ref, o));
        s.err = __dadd_rn(s.err, shfl_xor_d(s.err, o));
        s.ref = __dadd_rn(s.ref, shfl_xor_d(s.ref, o));
        s.dd = __dadd_rn(s.dd, shfl_xor_d(s.dd, o));
        s.rr = __dadd_rn(s.rr, shfl_xor_d(s.rr, o));
        s.dr = __dadd_rn(s.dr, shfl_xor_d(s.dr, o));
    }
}

// One reduce-table tile per work group; lane l takes the tile's 16-element
// slots l, l + REPORT_BLOCK, ... in order (one slot per lane for a narrow
// tile, two for a wide one).  The codes and the reference are 16-byte
// aligned buffers of n elements, so every slot but the buffer's last is
// read with whole 16-byte loads.
__global__ __launch_bounds__(REPORT_BLOCK) void k_report_tiles(const EArgs a) {
    __shared__ Stats sh[REPORT_BLOCK / 64];
    const Tile t = a.tiles[blockIdx.x];
    const int64_t j1 = (t.end + REPORT_V - 1) / REPORT_V;
    Stats st{0, 0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int64_t j = t.begin / REPORT_V + threadIdx.x; j < j1; j += REPORT_BLOCK) {
        const int64_t i0 = j * REPORT_V;
        int8_t qv[REPORT_V];
        float rv[REPORT_V];
        if (i0 + REPORT_V <= a.n) {
            const uint4 qw = *reinterpret_cast<const uint4 *>(a.q + i0);
            const uint32_t w4[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
            for (int k = 0; k < REPORT_V; ++k)
                qv[k] = static_cast<int8_t>((w4[k >> 2] >> (8 * (k & 3))) & 0xffu);
            const float4 *rp = reinterpret_cast<const float4 *>(a.ref + i0);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 f = rp[k];
                rv[4 * k] = f.x;
                rv[4 * k + 1] = f.y;
                rv[4 * k + 2] = f.z;
                rv[4 * k + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < REPORT_V; ++k) {
                const bool in = i0 + k < a.n;
                qv[k] = in ? a.q[i0 + k] : 0;
                rv[k] = in ? a.ref[i0 + k] : 0.0f;
            }
        }
        const float s = a.scale[t.unit];
#pragma unroll
        for (int k = 0; k < REPORT_V; ++k) {
            const int64_t i = i0 + k;
            if (i < t.begin || i >= t.end) continue;
            const double d = static_cast<double>(__fmul_rn(static_cast<float>(qv[k]), s));
            const double r = static_cast<double>(rv[k]);
            const double e = fabs(__dsub_rn(d, r));
            st.max_err = umax64(st.max_err, abs_bits64(e));
            st.max_ref = umax64(st.max_ref, abs_bits64(r));
            st.err = __dadd_rn(st.err, e);
            st.ref = __dadd_rn(st.ref, fabs(r));
            st.dd = __dadd_rn(st.dd, __dmul_rn(d, d));
            st.rr = __dadd_rn(st.rr, __dmul_rn(r, r));
            st.dr = __dadd_rn(st.dr, __dmul_rn(d, r));
        }
    }
    wave_stats(st);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = st;
    __syncthreads();
    if (threadIdx.x == 0) {
        Stats tot = sh[0];
        for (int w = 1; w < REPORT_BLOCK / 64; ++w) {
            tot.max_err = umax64(tot.max_err, sh[w].max_err);
            tot.max_ref = umax64(tot.max_ref, sh[w].max_ref);
            tot.err = __dadd_rn(tot.err, sh[w].err);
            tot.ref = __dadd_rn(tot.ref, sh[w].ref);
            tot.dd = __dadd_rn(tot.dd, sh[w].dd);
            tot.rr = __dadd_rn(tot.rr, sh[w].rr);
            tot.dr = __dadd_rn(tot.dr, sh[w].dr);
        }
        uint64_t *p = a.partial + static_cast<int64_t>(blockIdx.x) * kReportWords;
        p[0] = tot.max_err;
        p[1] = tot.max_ref;
        p[2] = static_cast<uint64_t>(__double_as_longlong(tot.err));
        p[3] = static_cast<uint64_t>(__double_as_longlong(tot.ref));
        p[4] = static_cast<uint64_t>(__double_as_longlong(tot.dd));
        p[5] = static_cast<uint64_t>(__double_as_longlong(tot.rr));
        p[6] = static_cast<uint64_t>(__double_as_longlong(tot.dr));
    }
}

__device__ __forceinline__ double ratio_or_zero(double x, double y) {
    return (x == 0.0 && y == 0.0) ? 0.0 : __ddiv_rn(x, y);
}

// One wave per unit: lane l combines the unit's tiles l, l + 64, ... in
// order, the wave butterfly combines the lanes (every lane ends with the
// same totals), then lane 0 takes the ratios (0/0 is 0) and the cosine (1
// for two zero vectors, 0 for one).  The order is fixed, so the result
// repeats bit for bit.
__global__ __launch_bounds__(256) void k_report_finalize(const EArgs a) {
    const int64_t u = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (u >= a.n_units) return;
    const int lane = threadIdx.x & 63;
    const int32_t t0 = a.unit_first[u], t1 = a.unit_first[u + 1];
    Stats st{0, 0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int32_t t = t0 + lane; t < t1; t += 64) {
        const uint64_t *p = a.partial + static_cast<int64_t>(t) * kReportWords;
        st.max_err = umax64(st.max_err, p[0]);
        st.max_ref = umax64(st.max_ref, p[1]);
        st.err = __dadd_rn(st.err, __longlong_as_double(static_cast<long long>(p[2])));
        st.ref = __dadd_rn(st.ref, __longlong_as_double(static_cast<long long>(p[3])));
        st.dd = __dadd_rn(st.dd, __longlong_as_double(static_cast<long long>(p[4])));
        st.rr = __dadd_rn(st.rr, __longlong_as_double(static_cast<long long>(p[5])));
        st.dr = __dadd_rn(st.dr, __longlong_as_double(static_cast<long long>(p[6])));
    }
    wave_stats(st);
    if (lane != 0) return;
    double *o = a.stats + u * GQ_STATS;
    const double me = __longlong_as_double(static_cast<long long>(st.max_err));
    const double mr = __longlong_as_double(static_cast<long long>(st.max_ref));
    o[GQ_STAT_MAX_ABS_ERR] = me;
    o[GQ_STAT_MAX_ABS_REF] = mr;
    o[GQ_STAT_MAX_REL_ERR] = ratio_or_zero(me, mr);
    o[GQ_STAT_SUM_ABS_ERR] = st.err;
    o[GQ_STAT_SUM_ABS_REF] = st.ref;
    o[GQ_STAT_MEAN_REL_ERR] = ratio_or_zero(st.err, st.ref);
    o[GQ_STAT_SUM_DD] = st.dd;
    o[GQ_STAT_SUM_RR] = st.rr;
    o[GQ_STAT_SUM_DR] = st.dr;
    double c;
    if (st.dd == 0.0 && st.rr == 0.0) c = 1.0;
    else if (st.dd == 0.0 || st.rr == 0.0) c = 0.0;
    else c = __ddiv_rn(st.dr, __dsqrt_rn(__dmul_rn(st.dd, st.rr)));
    o[GQ_STAT_COS] = c;
}

template <typename TIn, bool MUL>
hipError_t sum_typed(const SArgs &a, hipStream_t s) {
    constexpr int V = 16 / sizeof(TIn);
    const int64_t nslots = (a.n + V - 1) / V;
    const int64_t per_group = static_cast<int64_t>(SUM_BLOCK) * SUM_SLOTS;
    const int64_t groups = (nslots + per_group - 1) / per_group;
    if (groups < 1 || groups > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(groups));
    if (a.mean) hipLaunchKernelGGL((k_sum_f32<TIn, MUL, true>), grid, dim3(SUM_BLOCK), 0, s, a);
    else hipLaunchKernelGGL((k_sum_f32<TIn, MUL, false>), grid, dim3(SUM_BLOCK), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sum_f32(const SArgs &a, gq_dtype dt, hipStream_t s) {
    const bool mul = a.in_mul != 1.0f;
    if (dt == GQ_F16) return mul ? sum_typed<__half, true>(a, s) : sum_typed<__half, false>(a, s);
    return mul ? sum_typed<float, true>(a, s) : sum_typed<float, false>(a, s);
}

hipError_t launch_error_report(const EArgs &a, hipStream_t s) {
    if (a.n_tiles < 1 || a.n_tiles > 0x7fffffff || a.n_units < 1 || !a.tiles || !a.unit_first ||
        !a.partial)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_report_tiles, dim3(static_cast<unsigned>(a.n_tiles)), dim3(REPORT_BLOCK),
                       0, s, a);
    const int64_t groups = (a.n_units + 3) / 4;   // one wave per unit
    hipLaunchKernelGGL(k_report_finalize, dim3(static_cast<unsigned>(groups)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace gq
