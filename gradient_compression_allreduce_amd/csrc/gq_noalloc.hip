// gq_noalloc.hip -- gq_quantize_noalloc: the quantize stage (§2.2.1 of the
// pipelined HCCL AllReduce article, bjdmk.com.cn/news/6235379: scale =
// max|g| / 127 per unit and int8 codes; §6.1 unscale on load) for callers
// that cannot allocate device memory.  It needs no unit table: the caller
// passes the unit offsets, and the per-(rank, unit) maxima live in a
// fixed-size array of this file, `scratch`, that every call on a device
// shares.
//
// Three launches, none of whose work groups waits on another:
//   1. clear the W * n_units maxima in `scratch`;
//   2. per (rank, element range of a work group): the bit-pattern max of
//      |x| over each unit the range holds, merged into that unit's word by
//      an unsigned atomic max (maxima of non-negative floats order as their
//      bit patterns, and NaN above inf above every finite value);
//   3. per (rank, range) again: the scale of each unit from its word, and
//      the codes of the range's elements (the inputs are read a second
//      time).
// A work group covers a fixed element range, which may hold several units
// or part of one; it finds the unit of its first element with a 64-way
// search of the device offsets by one wave.
#include <mutex>

#include "gq_internal.h"
#include "gq_device.h"

// The maxima of the no-allocation quantize (GQ_NOALLOC_MAX_MAXIMA words,
// 4 MiB): one per (rank, unit) of the call in flight.  Host code takes its
// device address with hipGetSymbolAddress (per device, once) and passes that
// to the kernels; the array's name is not a device address on the host.
static __device__ __align__(256) uint32_t scratch[GQ_NOALLOC_MAX_MAXIMA];

namespace gq {
namespace {

constexpr int NA_BLOCK = 256;
constexpr int NA_SLOTS = 4;  // 16-byte slots per thread: 4096 fp32 or 8192 fp16 elements

struct NArgs {
    const void *x[GQ_MAX_RANKS];
    float *scale[GQ_MAX_RANKS];
    int8_t *q[GQ_MAX_RANKS];
    const int64_t *off;   // [n_units + 1] device offsets
    uint32_t *amax;       // [W][n_units] in scratch
    int64_t n_units;
    int64_t n;            // elements per rank (off[n_units])
    int64_t first;        // off[0]: elements before it belong to no unit
    int64_t base;         // first element of work group 0's range (slot-aligned)
    float in_mul;
    int32_t W;
};

__global__ __launch_bounds__(NA_BLOCK) void k_na_clear(uint32_t *amax, int64_t words) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * NA_BLOCK + threadIdx.x; i < words;
         i += static_cast<int64_t>(gridDim.x) * NA_BLOCK)
        amax[i] = 0u;
}

// The unit holding element e (off[0] <= e < off[U]), by wave 0 of the work
// group: each round, lane k looks at the offset `step` * (k + 1) past the
// current lower bound, and the lanes whose offset is <= e move the bound.
__device__ __forceinline__ int64_t find_unit(const int64_t *off, int64_t U, int64_t e) {
    const int lane = threadIdx.x & 63;
    int64_t lo = 0, hi = U;  // off[lo] <= e < off[hi]
    while (hi - lo > 1) {
        const int64_t step = (hi - lo + 64) / 65;
        const int64_t k = lo + step * (lane + 1);
        const bool le = k < hi && off[k] <= e;
        const uint64_t ball = __ballot(le);
        const int cnt = __popcll(ball);  // lanes 0 .. cnt-1 satisfy it (offsets increase)
        const int64_t nlo = lo + step * cnt;
        const int64_t nhi = cnt < 64 ? (lo + step * (cnt + 1) < hi ? lo + step * (cnt + 1) : hi) : hi;
        lo = nlo;
        hi = nhi;
    }
    return lo;
}

// The element range of this work group, [c0, c1) ∩ [first, n), and the unit
// of its first element (uniform over the work group); false if the range
// holds no unit's element.
template <int V>
__device__ __forceinline__ bool na_range(const NArgs &a, int64_t &c0, int64_t &c1, int64_t &lo,
                                         int64_t &u0, int64_t *s_u) {
    constexpr int64_t CH = static_cast<int64_t>(NA_BLOCK) * NA_SLOTS * V;
    c0 = a.base + static_cast<int64_t>(blockIdx.x) * CH;
    c1 = c0 + CH < a.n ? c0 + CH : a.n;
    lo = c0 > a.first ? c0 : a.first;
    if (lo >= c1) return false;
    if (threadIdx.x < 64) {
        const int64_t u = find_unit(a.off, a.n_units, lo);
        if (threadIdx.x == 0) *s_u = u;
    }
    __syncthreads();
    u0 = *s_u;
    return true;
}

// The thread's slots of the range (raw; zero past the buffer's end).
template <typename TIn>
__device__ __forceinline__ void na_load(const void *x, int64_t c0, int64_t n,
                                        typename In<TIn>::Raw (&raw)[NA_SLOTS]) {
    constexpr int V = In<TIn>::V;
#pragma unroll
    for (int s = 0; s < NA_SLOTS; ++s) {
        const int64_t i0 = c0 + static_cast<int64_t>(s * NA_BLOCK + threadIdx.x) * V;
        if (i0 + V <= n) raw[s] = load_stream(reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(x) + i0 * (16 / V)));
        else if (i0 < n) raw[s] = load_tail16(x, i0 * (16 / V), n * (16 / V));
        else raw[s] = make_uint4(0, 0, 0, 0);
    }
}

template <typename TIn>
__device__ __forceinline__ uint32_t elem_bits(const typename In<TIn>::Raw &r, int k) {
    if constexpr (In<TIn>::V == 4) {
        return (k == 0 ? r.x : k == 1 ? r.y : k == 2 ? r.z : r.w) & kAbsMask;
    } else {
        const uint32_t w = k < 2 ? r.x : k < 4 ? r.y : k < 6 ? r.z : r.w;
        return ((k & 1) ? (w >> 16) : w) & 0x7fffu;
    }
}

template <typename TIn>
__global__ __launch_bounds__(NA_BLOCK) void k_na_absmax(const NArgs a) {
    constexpr int V = In<TIn>::V;
    __shared__ uint32_t sh[NA_BLOCK / 64];
    __shared__ int64_t s_u;
    const int w = blockIdx.y;
    int64_t c0, c1, lo, u;
    if (!na_range<V>(a, c0, c1, lo, u, &s_u)) return;
    typename In<TIn>::Raw raw[NA_SLOTS];
    na_load<TIn>(a.x[w], c0, a.n, raw);
    for (;;) {
        const int64_t ua = a.off[u] > lo ? a.off[u] : lo;
        const int64_t ub = a.off[u + 1] < c1 ? a.off[u + 1] : c1;
        uint32_t m = 0;
#pragma unroll
        for (int s = 0; s < NA_SLOTS; ++s) {
            const int64_t i0 = c0 + static_cast<int64_t>(s * NA_BLOCK + threadIdx.x) * V;
            if (i0 >= ua && i0 + V <= ub) {
                m = In<TIn>::absmax(raw[s], m);
            } else if (i0 + V > ua && i0 < ub) {
#pragma unroll
                for (int k = 0; k < V; ++k)
                    if (i0 + k >= ua && i0 + k < ub) m = umax(m, elem_bits<TIn>(raw[s], k));
            }
        }
        m = block_max<NA_BLOCK>(m, sh);
        if (threadIdx.x == 0 && m != 0)
            __hip_atomic_fetch_max(&a.amax[static_cast<int64_t>(w) * a.n_units + u], m,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (ub >= c1 || u + 1 >= a.n_units) break;
        __syncthreads();  // sh is reused by the next unit's max
        ++u;
    }
}

template <typename TIn, bool MUL>
__global__ __launch_bounds__(NA_BLOCK) void k_na_quantize(const NArgs a) {
    constexpr int V = In<TIn>::V;
    __shared__ int64_t s_u;
    const int w = blockIdx.y;
    int64_t c0, c1, lo, u;
    if (!na_range<V>(a, c0, c1, lo, u, &s_u)) return;
    typename In<TIn>::Raw raw[NA_SLOTS];
    na_load<TIn>(a.x[w], c0, a.n, raw);
    uint32_t pk[NA_SLOTS][V / 4];
#pragma unroll
    for (int s = 0; s < NA_SLOTS; ++s)
#pragma unroll
        for (int k = 0; k < V / 4; ++k) pk[s][k] = 0u;
    for (;;) {
        const int64_t ustart = a.off[u];
        const int64_t ua = ustart > lo ? ustart : lo;
        const int64_t ub = a.off[u + 1] < c1 ? a.off[u + 1] : c1;
        const uint32_t mbits = a.amax[static_cast<int64_t>(w) * a.n_units + u];
        const float sc = __fdiv_rn(In<TIn>::max_value(mbits, a.in_mul, MUL), 127.0f);
        if (threadIdx.x == 0 && ustart >= c0) a.scale[w][u] = sc;  // the range of its first element
        const QuantParams p = quant_params(sc, true);
        const int mode = __builtin_amdgcn_readfirstlane(p.mode);
#pragma unroll
        for (int s = 0; s < NA_SLOTS; ++s) {
            const int64_t i0 = c0 + static_cast<int64_t>(s * NA_BLOCK + threadIdx.x) * V;
            float g[V];
#pragma unroll
            for (int k = 0; k < V; ++k) {
                g[k] = In<TIn>::elem(raw[s], k);
                if (MUL) g[k] = __fmul_rn(g[k], a.in_mul);
            }
            if (i0 >= ua && i0 + V <= ub) {  // the whole slot is in this unit
#pragma unroll
                for (int k = 0; k < V / 4; ++k) {
                    if (mode == CM_FAST)
                        pk[s][k] = codes4_fast(g[4 * k], g[4 * k + 1], g[4 * k + 2], g[4 * k + 3],
                                               p.s, p.r);
                    else if (mode == CM_EXACT)
                        pk[s][k] = pack4(code_exact(g[4 * k], p.s), code_exact(g[4 * k + 1], p.s),
                                         code_exact(g[4 * k + 2], p.s),
                                         code_exact(g[4 * k + 3], p.s));
                    else
                        pk[s][k] = 0u;
                }
            } else if (i0 + V > ua && i0 < ub) {  // a slot cut by a unit boundary
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    if (i0 + k >= ua && i0 + k < ub) {
                        const int c = mode == CM_ZERO ? 0 : code_exact(g[k], p.s);
                        const uint32_t sh8 = 8u * (k & 3);
                        pk[s][k >> 2] = (pk[s][k >> 2] & ~(0xffu << sh8)) |
                                        ((static_cast<uint32_t>(c) & 0xffu) << sh8);
                    }
                }
            }
        }
        if (ub >= c1 || u + 1 >= a.n_units) break;
        ++u;
    }
#pragma unroll
    for (int s = 0; s < NA_SLOTS; ++s) {
        const int64_t i0 = c0 + static_cast<int64_t>(s * NA_BLOCK + threadIdx.x) * V;
        if (i0 >= c1) continue;
        if (i0 >= lo && i0 + V <= c1) {
            if constexpr (V == 4) store_stream(a.q[w] + i0, pk[s][0]);
            else store_stream(a.q[w] + i0, pk[s][0], pk[s][1]);
        } else {
            store_codes_part(a.q[w] + i0, 0, V, lo - i0, c1 - i0,
                             make_uint4(pk[s][0], pk[s][(V / 4) - 1] & (V == 8 ? ~0u : 0u), 0u, 0u));
        }
    }
}

template <typename TIn, bool MUL>
hipError_t na_typed(const NArgs &a, hipStream_t st) {
    constexpr int V = In<TIn>::V;
    constexpr int64_t CH = static_cast<int64_t>(NA_BLOCK) * NA_SLOTS * V;
    const int64_t words = static_cast<int64_t>(a.W) * a.n_units;
    const int64_t clear_groups = (words + NA_BLOCK - 1) / NA_BLOCK;
    hipLaunchKernelGGL(k_na_clear, dim3(static_cast<unsigned>(clear_groups < 4096 ? clear_groups : 4096)),
                       dim3(NA_BLOCK), 0, st, a.amax, words);
    const dim3 grid(static_cast<unsigned>((a.n - a.base + CH - 1) / CH), static_cast<unsigned>(a.W));
    hipLaunchKernelGGL(k_na_absmax<TIn>, grid, dim3(NA_BLOCK), 0, st, a);
    hipLaunchKernelGGL((k_na_quantize<TIn, MUL>), grid, dim3(NA_BLOCK), 0, st, a);
    return hipGetLastError();
}

}  // namespace

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup failed.
void *noalloc_scratch(int device) {
    static std::mutex mu;
    static void *addr[GQ_NOALLOC_MAX_DEVICES] = {};
    if (device < 0 || device >= GQ_NOALLOC_MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        addr[device] = p;
    }
    return addr[device];
}

hipError_t launch_quantize_noalloc(const NoallocArgs &c, void *scratch_dev, hipStream_t st) {
    NArgs a;
    for (int w = 0; w < c.W; ++w) {
        a.x[w] = c.x[w];
        a.scale[w] = c.scale[w];
        a.q[w] = c.q[w];
    }
    a.off = c.d_off;
    a.amax = static_cast<uint32_t *>(scratch_dev);
    a.n_units = c.n_units;
    a.n = c.n;
    a.first = c.first;
    a.in_mul = c.in_mul;
    a.W = c.W;
    const int V = c.dt == GQ_F32 ? 4 : 8;
    a.base = (c.first / V) * V;
    const bool mul = c.in_mul != 1.0f;
    if (c.dt == GQ_F32) return mul ? na_typed<float, true>(a, st) : na_typed<float, false>(a, st);
    return mul ? na_typed<__half, true>(a, st) : na_typed<__half, false>(a, st);
}

}  // namespace gq
