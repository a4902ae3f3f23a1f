// gq_device.h -- device code shared by the gfx950 kernel files of libgq.so:
// the code arithmetic of the quantization (scale, int8 codes with the exact
// fast path), 16-byte input slots of fp32 or fp16 elements, streaming
// loads and stores, and work-group maxima.  Not part of the ABI.
//
// Numerics (bit-exact with the definition):
//   * g = x * in_mul is one rounded binary32 multiply (skipped when
//     in_mul == 1, which is exact);
//   * max|g| is an unsigned max over bit patterns with the sign cleared;
//   * the code is round-half-even of the IEEE quotient g / scale, clamped
//     to [-128, 127]; NaN quotients give 0 and a zero scale gives 0.  For a
//     normal scale (2^-126 <= s <= 2^126, so |g/s| <= 128) the quotient is
//     first estimated as q0 = fl(g * fl(1/s)), within 2^-16 of g/s; when q0
//     is more than 2^-15 away from every half-integer, fl(g/s) rounds to the
//     same integer as q0 and the division is skipped, otherwise it is done
//     exactly.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gq {
namespace {

constexpr uint32_t kAbsMask = 0x7fffffffu;
constexpr float kNearHalf = 0.5f - 0x1p-15f;   // fast-path guard band

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Streaming accesses.  The hot loops read every input byte once and write
// every output byte once, so their loads and stores carry the non-temporal
// hint (the nt bit of global_load/global_store), which keeps read-once and
// write-once data from competing with other lines in the caches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(int8_t *p, uint32_t w) {
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t *>(p));
}

__device__ __forceinline__ void store_stream(int8_t *p, uint32_t w0, uint32_t w1) {
    const u32x2 v = {w0, w1};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
}

__device__ __forceinline__ void store_stream(int8_t *p, uint4 w) {
    const u32x4 v = {w.x, w.y, w.z, w.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = umax(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64)));
    return v;
}

// Max over the work group; every thread gets it.  `sh` may be reused only
// after a __syncthreads().
template <int BLOCK>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t *sh) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = sh[0];
#pragma unroll
    for (int i = 1; i < BLOCK / 64; ++i) r = umax(r, sh[i]);
    return r;
}

// ---- codes --------------------------------------------------------------------

// Code of g for scale s by the definition (any s != 0, any g).
__device__ __forceinline__ int code_exact(float g, float s) {
    const float t = __fdiv_rn(g, s);
    float r = __builtin_rintf(t);
    r = fminf(fmaxf(r, -128.0f), 127.0f);
    return (t == t) ? static_cast<int>(r) : 0;
}

// Codes of four values in the fast mode (normal scale, |g| <= max), packed
// into the four bytes of a word.  Adding 1.5 * 2^23 to q0 = fl(g * r)
// rounds it to an integer half-to-even (|q0| < 2^22) and leaves that
// integer, as a two's-complement byte, in the low byte of the sum; if any of
// the four estimates lies within 2^-15 of a half-integer, the four codes
// are redone with exact division (rare).
__device__ __forceinline__ uint32_t codes4_fast(float g0, float g1, float g2, float g3, float s,
                                                float r) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    const float q0 = __fmul_rn(g0, r), q1 = __fmul_rn(g1, r);
    const float q2 = __fmul_rn(g2, r), q3 = __fmul_rn(g3, r);
    const float t0 = __fadd_rn(q0, kMagic), t1 = __fadd_rn(q1, kMagic);
    const float t2 = __fadd_rn(q2, kMagic), t3 = __fadd_rn(q3, kMagic);
    const float d0 = fabsf(__fsub_rn(q0, __fsub_rn(t0, kMagic)));
    const float d1 = fabsf(__fsub_rn(q1, __fsub_rn(t1, kMagic)));
    const float d2 = fabsf(__fsub_rn(q2, __fsub_rn(t2, kMagic)));
    const float d3 = fabsf(__fsub_rn(q3, __fsub_rn(t3, kMagic)));
    uint32_t b0 = __float_as_uint(t0), b1 = __float_as_uint(t1);
    uint32_t b2 = __float_as_uint(t2), b3 = __float_as_uint(t3);
    if (fmaxf(fmaxf(d0, d1), fmaxf(d2, d3)) >= kNearHalf) {
        b0 = static_cast<uint32_t>(code_exact(g0, s));
        b1 = static_cast<uint32_t>(code_exact(g1, s));
        b2 = static_cast<uint32_t>(code_exact(g2, s));
        b3 = static_cast<uint32_t>(code_exact(g3, s));
    }
    // low bytes of b0..b3 -> bytes 0..3 (selector 0x0c yields a zero byte)
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
    return lo | hi;
}

enum CodeMode { CM_ZERO = 0, CM_FAST = 1, CM_EXACT = 2 };

struct QuantParams {
    float s, r;
    int mode;
};

// `true_max`: the scale comes from the data's own max (fast path allowed).
__device__ __forceinline__ QuantParams quant_params(float s, bool true_max) {
    QuantParams p;
    p.s = s;
    p.r = 0.0f;
    if (s == 0.0f) {
        p.mode = CM_ZERO;
    } else if (true_max && s >= 0x1p-126f && s <= 0x1p126f) {
        p.mode = CM_FAST;
        p.r = __fdiv_rn(1.0f, s);
    } else {
        p.mode = CM_EXACT;
    }
    return p;
}

__device__ __forceinline__ uint32_t pack4(int c0, int c1, int c2, int c3) {
    return (static_cast<uint32_t>(c0) & 0xffu) | ((static_cast<uint32_t>(c1) & 0xffu) << 8) |
           ((static_cast<uint32_t>(c2) & 0xffu) << 16) | (static_cast<uint32_t>(c3) << 24);
}

// ---- input slots --------------------------------------------------------------
// A tile's slots are held raw (as loaded); elements outside the tile read as
// zero and are never loaded, stored or allowed into a max.

template <typename TIn>
struct In;

// Rare paths (the last slot of a buffer, slots cut by a unit boundary) are
// rolled loops, to keep the unrolled hot loops small.
__device__ __forceinline__ uint4 load_tail16(const void *base, int64_t byte0, int64_t nbytes) {
    const uint8_t *p = static_cast<const uint8_t *>(base);
    uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll 1
    for (int k = 0; k < 16; ++k) {
        if (byte0 + k >= nbytes) break;
        const uint32_t b = static_cast<uint32_t>(p[byte0 + k]) << (8 * (k & 3));
        const int wi = k >> 2;
        w0 |= wi == 0 ? b : 0u;
        w1 |= wi == 1 ? b : 0u;
        w2 |= wi == 2 ? b : 0u;
        w3 |= wi == 3 ? b : 0u;
    }
    return make_uint4(w0, w1, w2, w3);
}

// Keep the bytes [lo, hi) of a 16-byte slot, zero the others.
__device__ __forceinline__ uint4 keep_bytes(uint4 v, int lo, int hi) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t m = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int i = 4 * k + b;
            if (i >= lo && i < hi) m |= 0xffu << (8 * b);
        }
        w[k] &= m;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// 16-byte slot j of an element buffer of n elements of esz bytes, with the
// elements outside [b, e) zeroed.
__device__ __forceinline__ uint4 load_slot16(const void *x, int64_t j, int64_t b, int64_t e,
                                             int64_t n, int esz) {
    const int per = 16 / esz;
    const int64_t i0 = j * per;
    uint4 v;
    if (i0 + per <= n) v = *reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(x) + 16 * j);
    else v = load_tail16(x, 16 * j, n * esz);
    if (i0 < b || i0 + per > e) {
        const int lo = static_cast<int>((b > i0 ? b - i0 : 0) * esz);
        const int hi = static_cast<int>((e < i0 + per ? e - i0 : per) * esz);
        v = keep_bytes(v, lo, hi);
    }
    return v;
}

template <>
struct In<float> {
    static constexpr int V = 4;
    using Raw = uint4;
    static __device__ __forceinline__ Raw load(const void *x, int64_t j, int64_t b, int64_t e,
                                               int64_t n) {
        return load_slot16(x, j, b, e, n, 4);
    }
    static __device__ __forceinline__ uint32_t absmax(const Raw &r, uint32_t m) {
        m = umax(m, r.x & kAbsMask);
        m = umax(m, r.y & kAbsMask);
        m = umax(m, r.z & kAbsMask);
        return umax(m, r.w & kAbsMask);
    }
    // raw max bits -> max |g| (g = x * in_mul)
    static __device__ __forceinline__ float max_value(uint32_t mbits, float in_mul, bool mul) {
        const float m = __uint_as_float(mbits);
        return mul ? __fmul_rn(m, in_mul) : m;
    }
    static __device__ __forceinline__ float elem(const Raw &r, int k) {
        return __uint_as_float(k == 0 ? r.x : k == 1 ? r.y : k == 2 ? r.z : r.w);
    }
};

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(bits16)));
}

template <>
struct In<__half> {
    static constexpr int V = 8;
    using Raw = uint4;
    static __device__ __forceinline__ Raw load(const void *x, int64_t j, int64_t b, int64_t e,
                                               int64_t n) {
        return load_slot16(x, j, b, e, n, 2);
    }
    static __device__ __forceinline__ uint32_t absmax(const Raw &r, uint32_t m) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m = umax(m, w[k] & 0x7fffu);
            m = umax(m, (w[k] >> 16) & 0x7fffu);
        }
        return m;
    }
    static __device__ __forceinline__ float max_value(uint32_t mbits, float in_mul, bool mul) {
        const float m = h2f(mbits);
        return mul ? __fmul_rn(m, in_mul) : m;
    }
    static __device__ __forceinline__ float elem(const Raw &r, int k) {
        const uint32_t w = k < 2 ? r.x : k < 4 ? r.y : k < 6 ? r.z : r.w;
        return h2f((k & 1) ? (w >> 16) : (w & 0xffffu));
    }
};

// ---- output slots -------------------------------------------------------------

// Store the packed codes of elements [i0, i0+cnt) that fall inside [b, e).
__device__ __forceinline__ void store_codes_part(int8_t *q, int64_t i0, int cnt, int64_t b,
                                                 int64_t e, uint4 packed) {
#pragma unroll 1
    for (int k = 0; k < cnt; ++k) {
        const int64_t i = i0 + k;
        const uint32_t w = (k >> 2) == 0 ? packed.x : (k >> 2) == 1 ? packed.y
                         : (k >> 2) == 2 ? packed.z : packed.w;
        if (i >= b && i < e) q[i] = static_cast<int8_t>((w >> (8 * (k & 3))) & 0xffu);
    }
}

// Code of one element for the exact and zero modes (the fast mode codes
// four values at a time, codes4_fast).
template <int MODE>
__device__ __forceinline__ int code_of(float g, const QuantParams &p) {
    static_assert(MODE != CM_FAST, "the fast mode goes through codes4_fast");
    if constexpr (MODE == CM_EXACT) return code_exact(g, p.s);
    else return 0;
}

}  // namespace
}  // namespace gq
