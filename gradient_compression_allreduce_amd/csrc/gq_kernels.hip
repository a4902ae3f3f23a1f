// gq_kernels.hip -- gfx950 kernels of the INT8-compressed gradient AllReduce
// compute (pipelined HCCL AllReduce article, bjdmk.com.cn/news/6235379:
// §2.2.1 absmax scale, int8 codes and the INT8 AllReduce; §6.1 unscale).
//
// The work is bandwidth-bound streaming (no dense contraction, so no MFMA).
// Kernels walk host-built "tiles" (contiguous element ranges of one unit);
// a work group loads one tile of one rank at a time (and may hold one or
// two earlier tiles whose unit max it still needs).  A tile is read with
// 16-byte loads, one slot of V elements per lane per step, so a wave touches
// 1 KiB of contiguous memory per load instruction, and the tile stays on
// chip (registers, or LDS while it waits for its unit max) between the max
// and the code pass.
//
// The hot path is one persistent kernel per stage, launched with no more
// work groups (G) than the device keeps resident at once.  Work groups take
// tiles in order from a ticket counter (tickets run over rank 0's tiles in
// unit order, then rank 1's, and so on), so the tiles of one unit start at
// about the same time.  A unit larger than one tile combines its tiles'
// maxima in device memory (see "cross-work-group max" below) and each of
// its tiles waits, bounded, for the others, so every input byte is read
// from HBM once.  A work group
// blocks only in that wait, and by then it has published every tile it
// holds.  So if all running work groups were blocked, the earliest unit any
// of them waits on would have all of its taken tiles published and at least
// one tile untaken, which needs every running work group to hold one of its
// tiles.  The grid alone fits on the device, so every work group eventually
// runs (as soon as any other work on the device has finished); a work group
// takes tickets only once it runs, except that in the layer quantize and the
// reduce its first ticket is its own index (tickets below G), so once all
// run the taken tickets are again a prefix, and the wait ends for units of
// up to G tiles.  Larger units take a two-launch fallback (per-tile maxima,
// then a re-reading quantize pass).  The argument needs the other work on
// the device to finish without waiting on this grid: two such persistent
// kernels side by side could each hold compute units the other needs, so
// where two stages may overlap (the bucket pipeline) one of them runs in
// its wait-free form.  Every wait is bounded: if one ever gives up (the
// device did not run the grid), the table's fault counter records it and
// the launch's results are invalid.  While that count is nonzero, every
// wait on the table gives up at its first unsatisfied look, so no later
// launch waits a second per tile; the host clears the count.
//
// Numerics (must match the CPU oracle bit for bit):
//   * g = x * in_mul is one rounded binary32 multiply (skipped when
//     in_mul == 1, which is exact);
//   * max|g| is an unsigned max over bit patterns with the sign cleared,
//     taken on the raw inputs and scaled once (rounding is monotonic, so
//     max_i fl(|x_i| m) = fl(max_i |x_i| m));
//   * scale = max / 127 is an IEEE division;
//   * the code is round-half-even of the IEEE quotient g / scale, clamped
//     to [-128, 127]; NaN quotients give 0 and a zero scale gives 0.  For a
//     normal scale (2^-126 <= s <= 2^126, so |g/s| <= 128) the quotient is
//     first estimated as q0 = fl(g * fl(1/s)), within 2^-16 of g/s; when q0
//     is more than 2^-15 away from every half-integer, fl(g/s) rounds to the
//     same integer as q0 and the division is skipped, otherwise it is done
//     exactly;
//   * the reduction adds fl(q_w * s_w) to a +0 accumulator in rank order
//     with separate rounded multiplies and adds (never contracted).
#include <hip/hip_fp16.h>

#include "gq_internal.h"
#include "gq_device.h"

namespace gq {
namespace {

constexpr uint32_t kSpinLimit = 1u << 20;       // bounded wait (about a second)

// threadIdx.x as a value the compiler cannot see through, so that per-lane
// index arithmetic is not hoisted out of the persistent loops (hoisted
// values stay live across the whole loop and cost registers).
// With GROUP == 64 one wave works on a tile alone: the lane index.
template <int GROUP>
__device__ __forceinline__ int64_t opaque_tid() {
    int v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"(static_cast<int>(threadIdx.x)));
    return GROUP == 64 ? (v & 63) : v;
}

// The slot j of a tile when it is not a whole slot inside the tile: zero
// past the tile, the buffer's last (short) slot byte by byte, and the
// elements outside [b, e) cleared.  Rare; kept out of the issue loop.
template <typename TIn>
__device__ __forceinline__ uint4 fix_slot(const void *x, int64_t j, int64_t j1, int64_t b,
                                          int64_t e, int64_t n) {
    if (j >= j1) return make_uint4(0, 0, 0, 0);
    return load_slot16(x, j, b, e, n, 16 / In<TIn>::V);
}

// Rows of BLOCK slots that tile t covers (uniform over the work group).
template <typename TIn, int BLOCK>
__device__ __forceinline__ int tile_rows(const Tile &t) {
    constexpr int V = In<TIn>::V;
    const int64_t j0 = t.begin / V, j1 = (t.end + V - 1) / V;
    return __builtin_amdgcn_readfirstlane(static_cast<int>((j1 - j0 + BLOCK - 1) / BLOCK));
}

// Issue the loads of the S slots of tile t, at indices clamped into the
// buffer and without branches, so that all S loads are in flight together.
// With ROWS (tiles often much shorter than S rows, such as the short units
// that one wave takes), rows past the tile are not loaded.
template <typename TIn, int S, int BLOCK, bool ROWS = false>
__device__ __forceinline__ void issue_tile(const void *x, const Tile &t, int64_t n,
                                           typename In<TIn>::Raw (&raw)[S]) {
    constexpr int V = In<TIn>::V;
    const int64_t tid = opaque_tid<BLOCK>();
    const int64_t j0 = t.begin / V, j1 = (t.end + V - 1) / V;
    const int64_t nfull = n / V;
    // last slot to touch: the tile's last slot, at most the buffer's last
    // whole slot (lanes past the tile all load that one address, which the
    // memory pipeline merges)
    const int64_t jmax = (j1 < nfull ? j1 : nfull) - 1;
    const int rows = ROWS ? tile_rows<TIn, BLOCK>(t) : S;
    const uint4 *xv = static_cast<const uint4 *>(x);
    if (jmax >= 0) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int64_t j = j0 + static_cast<int64_t>(s) * BLOCK + tid;
            if (!ROWS || s < rows) raw[s] = load_stream(xv + (j < jmax ? j : jmax));
        }
    }
}

// Redo the few slots that are not whole slots inside the tile (slots past
// the tile, loaded or not, become zero), and return the max |x| bits of the
// tile.
template <typename TIn, int S, int BLOCK>
__device__ __forceinline__ uint32_t fix_tile(const void *x, const Tile &t, int64_t n,
                                             typename In<TIn>::Raw (&raw)[S]) {
    constexpr int V = In<TIn>::V;
    const int64_t tid = opaque_tid<BLOCK>();
    const int64_t j0 = t.begin / V, j1 = (t.end + V - 1) / V;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t j = j0 + static_cast<int64_t>(s) * BLOCK + tid;
        const bool inner = j < j1 && j * V >= t.begin && j * V + V <= t.end;
        if (!inner) raw[s] = fix_slot<TIn>(x, j, j1, t.begin, t.end, n);
    }
    uint32_t m = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) m = In<TIn>::absmax(raw[s], m);
    return m;
}

template <typename TIn, int S, int BLOCK, bool ROWS = false>
__device__ __forceinline__ uint32_t load_tile(const void *x, const Tile &t, int64_t n,
                                              typename In<TIn>::Raw (&raw)[S]) {
    issue_tile<TIn, S, BLOCK, ROWS>(x, t, n, raw);
    return fix_tile<TIn, S, BLOCK>(x, t, n, raw);
}

// Store the sums of elements [i0, i0+16) that fall inside [b, e).
__device__ __forceinline__ void store_sum_part(float *r, int64_t i0, int64_t b, int64_t e,
                                               float4 a0, float4 a1, float4 a2, float4 a3) {
#pragma unroll 1
    for (int k = 0; k < 16; ++k) {
        const int64_t i = i0 + k;
        const float4 v = (k >> 2) == 0 ? a0 : (k >> 2) == 1 ? a1 : (k >> 2) == 2 ? a2 : a3;
        const float f = (k & 3) == 0 ? v.x : (k & 3) == 1 ? v.y : (k & 3) == 2 ? v.z : v.w;
        if (i >= b && i < e) r[i] = f;
    }
}

// Codes of one slot j of tile t (V elements held raw), for one code mode.
template <typename TIn, bool MUL, int MODE>
__device__ __forceinline__ void quantize_slot(const typename In<TIn>::Raw &raw, int64_t j,
                                              const Tile &t, float in_mul, const QuantParams &p,
                                              int8_t *q) {
    constexpr int V = In<TIn>::V;
    float g[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        g[k] = In<TIn>::elem(raw, k);
        if (MUL) g[k] = __fmul_rn(g[k], in_mul);
    }
    uint32_t pk[V / 4];
#pragma unroll
    for (int k = 0; k < V / 4; ++k) {
        if constexpr (MODE == CM_FAST) {
            pk[k] = codes4_fast(g[4 * k], g[4 * k + 1], g[4 * k + 2], g[4 * k + 3], p.s, p.r);
        } else {
            pk[k] = pack4(code_of<MODE>(g[4 * k], p), code_of<MODE>(g[4 * k + 1], p),
                          code_of<MODE>(g[4 * k + 2], p), code_of<MODE>(g[4 * k + 3], p));
        }
    }
    const int64_t i0 = j * V;
    if constexpr (V == 4) {
        const uint32_t p0 = pk[0];
        if (i0 >= t.begin && i0 + V <= t.end) store_stream(q + i0, p0);
        else store_codes_part(q, i0, V, t.begin, t.end, make_uint4(p0, 0, 0, 0));
    } else {
        const uint32_t p0 = pk[0], p1 = pk[1];
        if (i0 >= t.begin && i0 + V <= t.end) store_stream(q + i0, p0, p1);
        else store_codes_part(q, i0, V, t.begin, t.end, make_uint4(p0, p1, 0, 0));
    }
}

// Codes of the S held slots of tile t, for one code mode.
template <typename TIn, int S, int BLOCK, bool MUL, int MODE>
__device__ __forceinline__ void quantize_tile_mode(const typename In<TIn>::Raw (&raw)[S],
                                                   const Tile &t, float in_mul,
                                                   const QuantParams &p, int8_t *q) {
    constexpr int V = In<TIn>::V;
    const int64_t tid = opaque_tid<BLOCK>();
    const int64_t j0 = t.begin / V, j1 = (t.end + V - 1) / V;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t j = j0 + static_cast<int64_t>(s) * BLOCK + tid;
        if (j >= j1) continue;
        quantize_slot<TIn, MUL, MODE>(raw[s], j, t, in_mul, p, q);
    }
}

// The same for a tile parked in LDS (slot s of lane l at park[s][l]); each
// lane reads back only what it parked.
template <typename TIn, int S, int BLOCK, bool MUL, int MODE>
__device__ __forceinline__ void quantize_parked_mode(const typename In<TIn>::Raw (*park)[BLOCK],
                                                     const Tile &t, float in_mul,
                                                     const QuantParams &p, int8_t *q) {
    constexpr int V = In<TIn>::V;
    const int64_t tid = opaque_tid<BLOCK>();
    const int64_t j0 = t.begin / V, j1 = (t.end + V - 1) / V;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t j = j0 + static_cast<int64_t>(s) * BLOCK + tid;
        if (j >= j1) continue;
        const typename In<TIn>::Raw r = park[s][threadIdx.x];
        quantize_slot<TIn, MUL, MODE>(r, j, t, in_mul, p, q);
    }
}

// The code mode is uniform over the work group: branch once per tile.
template <typename TIn, int S, int BLOCK, bool MUL>
__device__ __forceinline__ void quantize_tile(const typename In<TIn>::Raw (&raw)[S], const Tile &t,
                                              float in_mul, const QuantParams &p, int8_t *q) {
    const int mode = __builtin_amdgcn_readfirstlane(p.mode);
    if (mode == CM_FAST) quantize_tile_mode<TIn, S, BLOCK, MUL, CM_FAST>(raw, t, in_mul, p, q);
    else if (mode == CM_EXACT) quantize_tile_mode<TIn, S, BLOCK, MUL, CM_EXACT>(raw, t, in_mul, p, q);
    else quantize_tile_mode<TIn, S, BLOCK, MUL, CM_ZERO>(raw, t, in_mul, p, q);
}

// ---- cross-work-group max of a multi-tile unit ----------------------------------
// Each tile of a multi-tile unit publishes its max in its own 64-bit word,
// tagged with the launch's tag in the high half, then counts itself in on
// the unit's arrival counter.  The tile that completes a multiple of the
// unit's tile count is the last to arrive: it reads every tile word of the
// unit (waiting for any not yet visible), and publishes the unit max in the
// unit's tagged result word, which the other tiles poll.  All accesses are
// relaxed device-scope atomics on the words that carry the data, so no
// acquire/release fences (which would write back or invalidate the L2) are
// needed, and nothing has to be cleared between launches: a word holding an
// earlier launch's tag reads as "not yet published", and every launch adds
// exactly the tile count to each unit's counter.
//
// The tag is the table's launch epoch with the top bit set (never the
// initial zero); the last work group to leave a launch advances the epoch.
// A stale word could only pass for a fresh one after 2^31 launches of the
// table without that word being rewritten.

__device__ __forceinline__ uint32_t launch_tag(const uint32_t *ctl) {
    return __hip_atomic_load(&ctl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) | 0x80000000u;
}

// Thread 0: take the next ticket (every work group takes tickets until one
// is past the end, or none where its first ticket is static and the grid has
// a work group per tile; the last work group to leave clears the counter).  Where
// each work group's first ticket is its own index (no atomic at the start:
// the reduce and the layer quantize, whose start then costs no contended
// round trip), the counter hands out tickets from base = G on.  The chunk
// quantize takes its first ticket from the counter (base 0): its work
// groups, which never wait for one another, then start staggered, and were
// 1% slower on 128 KiB chunks with static first tickets.
__device__ __forceinline__ uint32_t take_ticket(uint32_t *ctl, uint32_t base = 0) {
    return base + __hip_atomic_fetch_add(&ctl[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread of the work group, once, at the end of a persistent kernel.
__device__ __forceinline__ void launch_exit(uint32_t *ctl) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(&ctl[1], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(&ctl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ctl[2], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&ctl[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Poll `word` (by lane 0) until it carries `tag`; returns its low half.
__device__ __forceinline__ uint32_t wait_tagged(const uint64_t *word, uint32_t tag, bool give_up,
                                                uint32_t *faults) {
    uint64_t v = 0;
    for (uint32_t it = 0;; ++it) {
        v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (static_cast<uint32_t>(v >> 32) == tag) break;
        if (give_up || it >= kSpinLimit) {
            __hip_atomic_fetch_add(faults, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(4);
    }
    return static_cast<uint32_t>(v);
}

// Wave 0: publish this tile's max m and count the tile in.  Returns (in
// lane 0) the unit's arrival count after this tile; a multiple of the tile
// count means this tile was the unit's last to arrive.
__device__ __forceinline__ uint64_t unit_publish(uint64_t *pub, uint64_t *cnt, int32_t tix,
                                                 uint32_t m, uint32_t tag) {
    uint64_t arrived = 0;
    if (threadIdx.x == 0) {
        __hip_atomic_store(&pub[tix], (static_cast<uint64_t>(tag) << 32) | m, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        arrived = __hip_atomic_fetch_add(cnt, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
    }
    return arrived;
}

// Wave 0: the unit max.  The unit's last arrival gathers every tile's max
// and publishes the unit max in the result word; the others poll that word.
__device__ __forceinline__ uint32_t unit_max(uint64_t *pub, uint64_t *res, int32_t tix,
                                             int32_t first, int32_t count, uint32_t m,
                                             uint64_t arrived_lane0, uint32_t tag,
                                             uint32_t *faults) {
    const int lane = threadIdx.x;
    const uint64_t arrived = __shfl(arrived_lane0, 0, 64);
    // once a wait on the table has given up (a nonzero count), later waits
    // do not wait again until the host clears the count
    const bool give_up = __hip_atomic_load(faults, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    if (arrived % static_cast<uint64_t>(count) != 0) {
        uint32_t um = 0;
        if (lane == 0) um = wait_tagged(res, tag, give_up, faults);
        return static_cast<uint32_t>(__shfl(static_cast<int>(um), 0, 64));
    }
    uint32_t mx = m;
    for (int i = lane; i < count; i += 64) {
        if (first + i == tix) continue;
        mx = umax(mx, wait_tagged(&pub[first + i], tag, give_up, faults));
    }
    mx = wave_max(mx);
    if (lane == 0)
        __hip_atomic_store(res, (static_cast<uint64_t>(tag) << 32) | mx, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return mx;
}

// Pack descriptors, likewise (the same for the whole wave).
__device__ __forceinline__ Pack load_pack(const Pack *packs, int64_t i) {
    using ConstPack = __attribute__((address_space(4))) const Pack;
    const ConstPack *p = (const ConstPack *)(packs + i);
    Pack k;
    k.first = p->first;
    k.count = p->count;
    k.lanes = p->lanes;
    k.pad = 0;
    return k;
}

// Tile descriptors are read-only: load them through the scalar cache.
__device__ __forceinline__ Tile load_desc(const Tile *tiles, int64_t i) {
    using ConstTile = __attribute__((address_space(4))) const Tile;
    const ConstTile *p = (const ConstTile *)(tiles + i);
    Tile t;
    t.begin = p->begin;
    t.end = p->end;
    t.unit = p->unit;
    t.first = p->first;
    t.count = p->count;
    t.slot = p->slot;
    return t;
}

// ---- quantize kernels -------------------------------------------------------------

// Small units: one wave per (rank, unit), no tile exchange and no ticket.
template <typename TIn, int SS, bool MUL>
__device__ __forceinline__ void quantize_wave_unit(const QArgs &a, int w, const Tile &t) {
    using Raw = typename In<TIn>::Raw;
    Raw raw[SS];
    const uint32_t m = wave_max(load_tile<TIn, SS, 64, true>(a.x[w], t, a.n, raw));
    const float sc = __fdiv_rn(In<TIn>::max_value(m, a.in_mul, MUL), 127.0f);
    if ((threadIdx.x & 63) == 0) a.scale[w][t.unit] = sc;
    quantize_tile<TIn, SS, 64, MUL>(raw, t, a.in_mul, quant_params(sc, true), a.q[w]);
}

// `item` runs over ranks, then small units.
template <typename TIn, int SS, bool MUL>
__device__ __forceinline__ void quantize_small_unit(const QArgs &a, int64_t item) {
    const int w = static_cast<int>(item / a.n_small);
    quantize_wave_unit<TIn, SS, MUL>(a, w, load_desc(a.small, item - static_cast<int64_t>(w) * a.n_small));
}

// The lane's group of a pack of lanes < 64 (group g = lane / lanes takes
// the pack's unit g, if there is one): its unit's tile (a vector load, the
// units differing across the wave), its lane within the group, and whether
// it has a unit.
struct PackLane {
    Tile t;
    int li;
    bool live;
};
__device__ __forceinline__ PackLane pack_lane(const Tile *units, const Pack &pk) {
    PackLane pl;
    const int lane = threadIdx.x & 63;
    const int lg = __builtin_ctz(static_cast<unsigned>(pk.lanes));
    const int g = lane >> lg;
    pl.li = lane & (pk.lanes - 1);
    pl.live = g < pk.count;
    pl.t = Tile{0, 0, 0, 0, 0, -1};
    if (pl.live) pl.t = units[pk.first + g];
    return pl;
}

// Max over each group of `lanes` lanes (a power of two): the xor partners
// of offsets below `lanes` stay within the group.
__device__ __forceinline__ uint32_t group_max(uint32_t v, int lanes) {
    for (int o = lanes >> 1; o > 0; o >>= 1)
        v = umax(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64)));
    return v;
}

// A pack of lanes < 64 of a short quantize table: each group of lanes
// quantizes its unit, one slot per lane.
template <typename TIn, bool MUL>
__device__ __forceinline__ void quantize_pack(const QArgs &a, int w, const Pack &pk) {
    constexpr int V = In<TIn>::V;
    const PackLane pl = pack_lane(a.small, pk);
    const Tile &t = pl.t;
    const int64_t j = t.begin / V + pl.li, j1 = (t.end + V - 1) / V;
    const bool in = pl.live && j < j1;
    typename In<TIn>::Raw raw{};
    if (in) raw = In<TIn>::load(a.x[w], j, t.begin, t.end, a.n);
    const uint32_t m = group_max(In<TIn>::absmax(raw, 0u), pk.lanes);
    const float sc = __fdiv_rn(In<TIn>::max_value(m, a.in_mul, MUL), 127.0f);
    if (pl.live && pl.li == 0) a.scale[w][t.unit] = sc;
    if (in) {
        const QuantParams qp = quant_params(sc, true);
        if (qp.mode == CM_FAST) quantize_slot<TIn, MUL, CM_FAST>(raw, j, t, a.in_mul, qp, a.q[w]);
        else if (qp.mode == CM_EXACT) quantize_slot<TIn, MUL, CM_EXACT>(raw, j, t, a.in_mul, qp, a.q[w]);
        else quantize_slot<TIn, MUL, CM_ZERO>(raw, j, t, a.in_mul, qp, a.q[w]);
    }
}

// The small units' phase of the persistent kernels: wave v of work group g
// takes the small items v + waves * (g + G * k).  Ends with a work-group
// barrier.  The quantize kernels and the narrow reduce run it after their
// ticket loop, so that it fills the ragged end of the tile phase instead of
// holding back the first tiles; the wide reduce runs it first (run last,
// it made that kernel slower).
template <int BLOCK, typename F>
__device__ __forceinline__ void small_phase(int64_t items, F &&one) {
    constexpr int WPG = BLOCK / 64;
    const int64_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t item = static_cast<int64_t>(blockIdx.x) * WPG + wave; item < items;
         item += static_cast<int64_t>(gridDim.x) * WPG)
        one(item);
    __syncthreads();
}

// Hot path, SCHED_CHUNK: every tile of every rank, one read of the input.
// Per tile, a work group: issues the loads of its next tile; writes the
// codes of its current tile (whose unit max it already has), so the loads
// are in flight during the code pass; takes the next tile's max, publishes
// it and waits for that unit's max; then moves on to a new ticket.  When the
// next tile ends its unit (a 128 KiB chunk is one tile), the ticket after it
// is taken before that tile's loads are issued, so the ticket's round trip
// overlaps them instead of following them.  Such a tile never waits for
// another, and the early ticket lies in a later unit than any the work group
// may then wait on; so a work group blocks only while holding no
// unpublished tile and no ticket of the unit it waits on or of an earlier
// one (the scheduling note above then still applies: tickets are taken in
// order, so the earliest unit anyone waits on has all its tiles taken and
// published, or an untaken tile and every running work group holding one of
// its tiles).
template <typename TIn, int S, int BLOCK, bool MUL>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
void k_quantize_chunk(const QArgs a) {
    using Raw = typename In<TIn>::Raw;
    __shared__ uint32_t sh[BLOCK / 64];
    __shared__ uint32_t s_val[2];  // unit max, ticket
    __shared__ uint32_t s_tk[2];   // early tickets, by iteration parity
    const int64_t total = static_cast<int64_t>(a.W) * a.n_tiles;
    const uint32_t tag = launch_tag(a.ctl);
    Raw cur[S], nxt[S];

    // ticket -> (rank, tile index, descriptor)
    auto next_ticket = [&]() -> int64_t {
        if (threadIdx.x == 0) s_val[1] = take_ticket(a.ctl);
        __syncthreads();
        const int64_t t = s_val[1];
        __syncthreads();
        return t;
    };
    // max of a loaded tile, published and combined into its unit max
    // (blocks until the unit is complete)
    auto tile_max = [&](Raw (&buf)[S], const Tile &t, int w, int32_t tix) -> uint32_t {
        uint32_t m = block_max<BLOCK>(fix_tile<TIn, S, BLOCK>(a.x[w], t, a.n, buf), sh);
        if (t.count > 1) {
            if (threadIdx.x < 64) {
                uint64_t *pub = a.pub + static_cast<int64_t>(w) * a.n_tiles;
                const int64_t u = static_cast<int64_t>(w) * a.n_multi_units + t.slot;
                const uint64_t arr = unit_publish(pub, a.cnt + u, tix, m, tag);
                const uint32_t um = unit_max(pub, a.res + u, tix, t.first, t.count, m, arr, tag,
                                             a.faults);
                if (threadIdx.x == 0) s_val[0] = um;
            }
            __syncthreads();
            m = s_val[0];
        }
        return m;
    };

    int64_t tk = next_ticket();
    if (tk < total) {
        int wc = static_cast<int>(tk / a.n_tiles);
        int32_t tix = static_cast<int32_t>(tk - static_cast<int64_t>(wc) * a.n_tiles);
        Tile tc = load_desc(a.tiles, tix);
        // a tile that ends its unit: take the next ticket while its loads fly
        bool early = tix == tc.first + tc.count - 1;
        uint32_t pend = 0;
        if (early && threadIdx.x == 0) pend = take_ticket(a.ctl);
        issue_tile<TIn, S, BLOCK>(a.x[wc], tc, a.n, cur);
        uint32_t mc = tile_max(cur, tc, wc, tix);
        auto ticket_after = [&]() -> int64_t {
            if (!early) return next_ticket();
            if (threadIdx.x == 0) s_val[1] = pend;
            __syncthreads();
            const int64_t t = s_val[1];
            __syncthreads();
            return t;
        };
        int64_t tn = ticket_after();
        int par = 0;
        for (;;) {
            const bool more = tn < total;
            int wn = 0;
            int32_t tixn = 0;
            Tile tnx{};
            early = false;
            if (more) {
                wn = static_cast<int>(tn / a.n_tiles);
                tixn = static_cast<int32_t>(tn - static_cast<int64_t>(wn) * a.n_tiles);
                tnx = load_desc(a.tiles, tixn);
                early = tixn == tnx.first + tnx.count - 1;
                if (early && threadIdx.x == 0) pend = take_ticket(a.ctl);
                issue_tile<TIn, S, BLOCK>(a.x[wn], tnx, a.n, nxt);
            }
            const float sc = __fdiv_rn(In<TIn>::max_value(mc, a.in_mul, MUL), 127.0f);
            if (threadIdx.x == 0 && tix == tc.first) a.scale[wc][tc.unit] = sc;
            quantize_tile<TIn, S, BLOCK, MUL>(cur, tc, a.in_mul, quant_params(sc, true), a.q[wc]);
            if (!more) break;
            // an early ticket reaches the work group through LDS at the
            // block-max barrier inside tile_max, with no barriers of its
            // own; slots alternate by parity, since the next write to a slot
            // follows another tile_max barrier, after every read of it
            if (early && threadIdx.x == 0) s_tk[par] = pend;
            mc = tile_max(nxt, tnx, wn, tixn);
#pragma unroll
            for (int s = 0; s < S; ++s) cur[s] = nxt[s];
            tc = tnx;
            wc = wn;
            tix = tixn;
            tn = early ? static_cast<int64_t>(s_tk[par]) : next_ticket();
            par ^= 1;
        }
    }
    small_phase<BLOCK>(static_cast<int64_t>(a.W) * a.n_small, [&](int64_t item) {
        quantize_small_unit<TIn, SMALL_SLOTS_Q, MUL>(a, item);
    });
    launch_exit(a.ctl);
}

// Hot path, SCHED_LAYER: every tile of every rank, one read of the input.
// A work group holds up to two published tiles whose unit max it may still
// need: C in registers and P, the older one, parked in LDS (64 KiB).  Per
// ticket it: takes the ticket (and polls P's unit result word once, in the
// same round trip); issues the new tile N's loads; codes P from LDS while
// they fly if P's unit max is known; takes N's max and publishes it; only
// then, if P is still open, waits for P's unit max and codes P; parks C in
// LDS as the next P and keeps N in registers as the next C.  A tile's unit
// max is thus first asked for two tiles after the tile was published, when
// it is usually known, and the work group blocks only with every tile it
// holds published (see the scheduling note above).
template <typename TIn, int S, int BLOCK, bool MUL>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
void k_quantize_layer(const QArgs a) {
    using Raw = typename In<TIn>::Raw;
    __shared__ uint32_t sh[BLOCK / 64];
    __shared__ uint32_t s_val[3];  // unit max, ticket, polled-ready flag
    __shared__ Raw park[S][BLOCK];
    const int64_t total = static_cast<int64_t>(a.W) * a.n_tiles;
    const uint32_t tag = launch_tag(a.ctl);
    const int lane = threadIdx.x;
    // held tiles C (slots in A) and P (slots parked): ticket, rank,
    // descriptor, max (the unit max once known) and arrival count
    Raw A[S], B[S];
    bool has_c = false, known_c = false, has_p = false, known_p = false;
    Tile tc{}, tp{};
    int wc = 0, wp = 0;
    int64_t kc = 0, kp = 0;
    uint32_t mc = 0, mp = 0;
    uint64_t arr_c = 0, arr_p = 0;
    // max of a loaded tile, its publication, and the gather if it was its
    // unit's last arrival; returns whether m is the unit max
    auto finish_tile = [&](int64_t t_k, Raw (&buf)[S], const Tile &t, int w, uint32_t &m,
                           uint64_t &arr) -> bool {
        const int32_t tix = static_cast<int32_t>(t_k - static_cast<int64_t>(w) * a.n_tiles);
        m = block_max<BLOCK>(fix_tile<TIn, S, BLOCK>(a.x[w], t, a.n, buf), sh);
        if (t.count == 1) return true;
        if (threadIdx.x < 64) {
            uint64_t *pub = a.pub + static_cast<int64_t>(w) * a.n_tiles;
            const int64_t u = static_cast<int64_t>(w) * a.n_multi_units + t.slot;
            arr = unit_publish(pub, a.cnt + u, tix, m, tag);
            uint32_t last = 0;
            if (__shfl(arr, 0, 64) % static_cast<uint64_t>(t.count) == 0) {
                const uint32_t um = unit_max(pub, a.res + u, tix, t.first, t.count, m, arr, tag,
                                             a.faults);
                last = 1;
                if (threadIdx.x == 0) s_val[0] = um;
            }
            if (threadIdx.x == 0) s_val[2] = last;
        }
        __syncthreads();
        const bool known = s_val[2] != 0;
        if (known) m = s_val[0];
        __syncthreads();
        return known;
    };
    auto code_parked = [&]() {
        const int32_t tix = static_cast<int32_t>(kp - static_cast<int64_t>(wp) * a.n_tiles);
        const float sc = __fdiv_rn(In<TIn>::max_value(mp, a.in_mul, MUL), 127.0f);
        if (threadIdx.x == 0 && tix == tp.first) a.scale[wp][tp.unit] = sc;
        const QuantParams qp = quant_params(sc, true);
        const int mode = __builtin_amdgcn_readfirstlane(qp.mode);
        if (mode == CM_FAST)
            quantize_parked_mode<TIn, S, BLOCK, MUL, CM_FAST>(park, tp, a.in_mul, qp, a.q[wp]);
        else if (mode == CM_EXACT)
            quantize_parked_mode<TIn, S, BLOCK, MUL, CM_EXACT>(park, tp, a.in_mul, qp, a.q[wp]);
        else
            quantize_parked_mode<TIn, S, BLOCK, MUL, CM_ZERO>(park, tp, a.in_mul, qp, a.q[wp]);
    };
    // with a grid of at least one work group per tile, the static first
    // tickets cover every tile: no dynamic ticket (and no round trip for it)
    bool tickets_left = static_cast<int64_t>(gridDim.x) < total;
    {
        const int64_t tk = blockIdx.x;
        if (tk < total) {
            wc = static_cast<int>(tk / a.n_tiles);
            tc = load_desc(a.tiles, static_cast<int32_t>(tk - static_cast<int64_t>(wc) * a.n_tiles));
            issue_tile<TIn, S, BLOCK>(a.x[wc], tc, a.n, A);
            known_c = finish_tile(tk, A, tc, wc, mc, arr_c);
            kc = tk;
            has_c = true;
        } else {
            tickets_left = false;
        }
    }
    while (has_c || has_p) {
        // one round trip: the next ticket, and one look at P's result word
        const int64_t up = static_cast<int64_t>(wp) * a.n_multi_units + tp.slot;
        if (threadIdx.x == 0) {
            if (tickets_left) s_val[1] = take_ticket(a.ctl, gridDim.x);
            uint32_t ready = 0;
            if (has_p && !known_p) {
                const uint64_t v = __hip_atomic_load(a.res + up, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                if (static_cast<uint32_t>(v >> 32) == tag) {
                    ready = 1;
                    s_val[0] = static_cast<uint32_t>(v);
                }
            }
            s_val[2] = ready;
        }
        __syncthreads();
        const int64_t tn = tickets_left ? static_cast<int64_t>(s_val[1]) : total;
        if (has_p && !known_p && s_val[2] != 0) {
            known_p = true;
            mp = s_val[0];
        }
        __syncthreads();
        const bool more = tn < total;
        if (!more) tickets_left = false;
        Tile tnx{};
        int wn = 0;
        if (more) {
            wn = static_cast<int>(tn / a.n_tiles);
            tnx = load_desc(a.tiles, static_cast<int32_t>(tn - static_cast<int64_t>(wn) * a.n_tiles));
            issue_tile<TIn, S, BLOCK>(a.x[wn], tnx, a.n, B);
        }
        if (has_p && known_p) {  // while N's loads fly
            code_parked();
            has_p = false;
        }
        uint32_t mn = 0;
        uint64_t arr_n = 0;
        bool known_n = false;
        if (more) known_n = finish_tile(tn, B, tnx, wn, mn, arr_n);
        if (has_p) {  // every held tile is published: safe to wait
            if (threadIdx.x < 64) {
                const int32_t tix = static_cast<int32_t>(kp - static_cast<int64_t>(wp) * a.n_tiles);
                const uint32_t um = unit_max(a.pub + static_cast<int64_t>(wp) * a.n_tiles, a.res + up,
                                             tix, tp.first, tp.count, mp, arr_p, tag, a.faults);
                if (threadIdx.x == 0) s_val[0] = um;
            }
            __syncthreads();
            mp = s_val[0];
            __syncthreads();
            code_parked();
            has_p = false;
        }
        if (has_c) {  // C becomes P
#pragma unroll
            for (int s = 0; s < S; ++s) park[s][lane] = A[s];
            tp = tc;
            wp = wc;
            kp = kc;
            mp = mc;
            known_p = known_c;
            arr_p = arr_c;
            has_p = true;
            has_c = false;
        }
        if (more) {  // N becomes C
#pragma unroll
            for (int s = 0; s < S; ++s) A[s] = B[s];
            tc = tnx;
            wc = wn;
            kc = tn;
            mc = mn;
            known_c = known_n;
            arr_c = arr_n;
            has_c = true;
        }
    }
    small_phase<BLOCK>(static_cast<int64_t>(a.W) * a.n_small, [&](int64_t item) {
        quantize_small_unit<TIn, SMALL_SLOTS_Q, MUL>(a, item);
    });
    launch_exit(a.ctl);
}

// Fallback pass 1 (and gq_absmax): per-tile max of the listed tiles.
template <typename TIn, int S, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_tile_absmax(const QArgs a) {
    __shared__ uint32_t sh[BLOCK / 64];
    const int w = blockIdx.y;
    const int32_t tix = a.list ? a.list[blockIdx.x] : static_cast<int32_t>(blockIdx.x);
    const Tile t = load_desc(a.tiles, tix);
    typename In<TIn>::Raw raw[S];
    const uint32_t m = block_max<BLOCK>(load_tile<TIn, S, BLOCK>(a.x[w], t, a.n, raw), sh);
    if (threadIdx.x == 0) a.partial[static_cast<int64_t>(w) * a.n_tiles + tix] = m;
}

// gq_absmax: one max per (rank, unit) from the per-tile maxima.
template <typename TIn>
__global__ void k_absmax_finalize(const QArgs a, bool mul) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= static_cast<int64_t>(a.W) * a.n_units) return;
    const int64_t w = idx / a.n_units, u = idx - w * a.n_units;
    const uint32_t *p = a.partial + w * a.n_tiles;
    uint32_t m = 0;
    for (int32_t i = a.unit_first[u]; i < a.unit_first[u + 1]; ++i) m = umax(m, p[i]);
    a.amax_out[idx] = __float_as_uint(In<TIn>::max_value(m, a.in_mul, mul)) & kAbsMask;
}

enum QMode { Q_FUSED = 0, Q_GIVEN = 1 };

// Fallback pass 2 (Q_FUSED: maxima from pass 1 for multi-tile units) and
// the quantize-with-given-maxima entry (Q_GIVEN).  One tile per work group.
template <typename TIn, int S, int BLOCK, bool MUL, int MODE>
__global__ __launch_bounds__(BLOCK) void k_quantize(const QArgs a) {
    __shared__ uint32_t sh[BLOCK / 64];
    const int w = blockIdx.y;
    const int32_t tix = static_cast<int32_t>(blockIdx.x);
    const Tile t = load_desc(a.tiles, tix);
    typename In<TIn>::Raw raw[S];
    const uint32_t own = load_tile<TIn, S, BLOCK>(a.x[w], t, a.n, raw);
    float maxv;
    if (MODE == Q_GIVEN) {
        maxv = __uint_as_float(a.amax[static_cast<int64_t>(w) * a.n_units + t.unit]);
    } else {
        uint32_t m;
        if (t.count == 1) {
            m = block_max<BLOCK>(own, sh);
        } else {
            const uint32_t *p = a.partial + static_cast<int64_t>(w) * a.n_tiles + t.first;
            uint32_t pm = 0;
            for (int i = threadIdx.x; i < t.count; i += BLOCK) pm = umax(pm, p[i]);
            m = block_max<BLOCK>(pm, sh);
        }
        maxv = In<TIn>::max_value(m, a.in_mul, MUL);
    }
    const float sc = __fdiv_rn(maxv, 127.0f);
    if (threadIdx.x == 0 && tix == t.first) a.scale[w][t.unit] = sc;
    quantize_tile<TIn, S, BLOCK, MUL>(raw, t, a.in_mul, quant_params(sc, MODE == Q_FUSED), a.q[w]);
}

// ---- reduce kernels ----------------------------------------------------------------

constexpr int RV = 16;  // codes per reduce slot

// Rank w's scale of unit u, through the scalar cache (the same for every
// lane of a work group).  A vector load here would join the code loads'
// in-order completion count, so that waiting for the scale would also wait
// for every code load issued before it (the ranks loaded ahead included).
// The scales are inputs, written before the launch (the launch's acquire
// makes them visible to the scalar cache) and never written by it.
__device__ __forceinline__ float rank_scale(const RArgs &a, int w, int32_t u) {
    using ConstF = __attribute__((address_space(4))) const float;
    return ((ConstF *)(a.scale[w]))[u];
}

// acc += fl(q * sw) for the 16 codes of each held slot: each code is
// converted from its signed byte (one instruction with a byte-select source
// operand) and multiplied by sw with one rounding, then added.
template <int S>
__device__ __forceinline__ void accumulate(const uint4 (&v)[S], float sw, float (&acc)[S][RV]) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint32_t wd[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
        for (int k = 0; k < RV; ++k) {
            const int c = static_cast<int8_t>((wd[k >> 2] >> (8 * (k & 3))) & 0xffu);
            acc[s][k] = __fadd_rn(acc[s][k], __fmul_rn(static_cast<float>(c), sw));
        }
    }
}

// Rank-order dequant-accumulate of the S slots of tile t into acc.  With
// OFF32, a lane's loads are addressed from the tile's first slot by a 32-bit
// offset (a tile spans at most S * BLOCK slots), which saves registers.
// WT > 0: the rank count is WT (= a.W), known when compiling, and the rank
// loop unrolls fully (no loop-carried buffers for the compiler to copy).
template <int S, int BLOCK, int RG = 4, bool OFF32 = false, int WT = 0>
__device__ __forceinline__ void reduce_tile(const RArgs &a, const Tile &t, float (&acc)[S][RV]) {
    const int W = WT > 0 ? WT : a.W;
    const int64_t tid = opaque_tid<BLOCK>();
    const int64_t j0 = t.begin / RV, j1 = (t.end + RV - 1) / RV;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int k = 0; k < RV; ++k) acc[s][k] = 0.0f;

    // Codes are loaded RG ranks at a time into two buffers in turn: the
    // next group's loads are issued before the current group is
    // accumulated, and no buffer is copied into the other (a copy would
    // wait for the loads just issued).  Every load is issued on every path,
    // and no loaded value is replaced on some lanes only (the merge would be
    // a copy), so that the hardware's in-order load count tells each
    // group's wait exactly; a rank past the last one loads the last rank's
    // first slot again (one cache line, never used).  Loads are issued at
    // indices clamped into the buffer, without branches.  Slots past the
    // tile are summed from those clamped loads and their sums cleared below;
    // a slot at the buffer's short end (n not a multiple of 16) is summed
    // again afterwards from its bytes.  Whole 16-byte slots are read even
    // where a unit boundary cuts them (the bytes belong to the rank's
    // buffer); sums of elements outside the tile are cleared below.
    const int64_t nfull = a.n / RV;
    const int64_t jmax = (j1 < nfull ? j1 : nfull) - 1;
    // slot jb + o, o = min(lane's slot - jb, jmax - jb), jb = min(j0, jmax)
    const int64_t jb = j0 < jmax ? j0 : jmax;
    const uint32_t lim = static_cast<uint32_t>(jmax - jb);
    const uint32_t o0 = static_cast<uint32_t>(j0 - jb) + static_cast<uint32_t>(tid);
    uint4 bufA[RG][S], bufB[RG][S];
    auto issue = [&](int w0, uint4 (&v)[RG][S]) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const bool past = w0 + r >= W;
            const int w = past ? W - 1 : w0 + r;
            if constexpr (OFF32) {
                const uint4 *qv = reinterpret_cast<const uint4 *>(a.q[w]) + jb;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const uint32_t o = o0 + static_cast<uint32_t>(s * BLOCK);
                    v[r][s] = load_stream(qv + (past ? 0u : (o < lim ? o : lim)));
                }
            } else {
                const uint4 *qv = reinterpret_cast<const uint4 *>(a.q[w]);
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const int64_t j = j0 + static_cast<int64_t>(s) * BLOCK + tid;
                    v[r][s] = load_stream(qv + (past ? jb : (j < jmax ? j : jmax)));
                }
            }
        }
    };
    auto consume = [&](int w0, uint4 (&v)[RG][S]) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int w = w0 + r;
            if (w >= W) break;
            accumulate<S>(v[r], rank_scale(a, w, t.unit), acc);
        }
    };
    if (jmax >= 0) {  // (else the buffer is one short slot, summed below)
        issue(0, bufA);
        if constexpr (WT > 0) {
#pragma unroll
            for (int w0 = 0; w0 < WT; w0 += 2 * RG) {
                issue(w0 + RG, bufB);
                consume(w0, bufA);
                if (w0 + 2 * RG < WT) issue(w0 + 2 * RG, bufA);
                consume(w0 + RG, bufB);
            }
        } else {
            for (int w0 = 0; w0 < a.W; w0 += 2 * RG) {
                issue(w0 + RG, bufB);
                consume(w0, bufA);
                issue(w0 + 2 * RG, bufA);
                consume(w0 + RG, bufB);
            }
        }
    }
    // the buffer's short last slot, from its bytes, in rank order
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t j = j0 + static_cast<int64_t>(s) * BLOCK + tid;
        if (j < j1 && j >= nfull) {
            float part[1][RV];
#pragma unroll
            for (int k = 0; k < RV; ++k) part[0][k] = 0.0f;
            for (int w = 0; w < a.W; ++w) {
                const uint4 c[1] = {load_tail16(a.q[w], j * RV, a.n)};
                accumulate<1>(c, rank_scale(a, w, t.unit), part);
            }
#pragma unroll
            for (int k = 0; k < RV; ++k) acc[s][k] = part[0][k];
        }
    }
    // elements outside the tile never reach a max or a store (0 * inf = NaN)
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t j = j0 + static_cast<int64_t>(s) * BLOCK + tid;
        const int64_t i0 = j * RV;
        if (!(j < j1 && i0 >= t.begin && i0 + RV <= t.end)) {
#pragma unroll
            for (int k = 0; k < RV; ++k) {
                const int64_t i = i0 + k;
                if (!(j < j1 && i >= t.begin && i < t.end)) acc[s][k] = 0.0f;
            }
        }
    }
}

template <int S>
__device__ __forceinline__ uint32_t acc_absmax(const float (&acc)[S][RV]) {
    uint32_t m = 0;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int k = 0; k < RV; ++k) m = umax(m, __float_as_uint(acc[s][k]) & kAbsMask);
    return m;
}

// The 16 sums of slot j of tile t (acc, one slot's sums), stored where they
// fall inside the tile.
__device__ __forceinline__ void store_sum_slot(int64_t j, const Tile &t, const float *acc,
                                               float *r) {
    const int64_t i0 = j * RV;
    float4 f[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        f[k] = make_float4(acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]);
    if (i0 >= t.begin && i0 + RV <= t.end) {
        float4 *rp = reinterpret_cast<float4 *>(r + i0);
#pragma unroll
        for (int k = 0; k < 4; ++k) rp[k] = f[k];
    } else {
        store_sum_part(r, i0, t.begin, t.end, f[0], f[1], f[2], f[3]);
    }
}

template <int S, int BLOCK>
__device__ __forceinline__ void store_sum(const Tile &t, const float (&acc)[S][RV], float *r) {
    const int64_t tid = opaque_tid<BLOCK>();
    const int64_t j0 = t.begin / RV, j1 = (t.end + RV - 1) / RV;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t j = j0 + static_cast<int64_t>(s) * BLOCK + tid;
        if (j >= j1) continue;
        store_sum_slot(j, t, acc[s], r);
    }
}

// Codes of the 16 sums of slot j of tile t (acc, one slot's sums), stored
// where they fall inside the tile.
template <int MODE>
__device__ __forceinline__ void requantize_slot(int64_t j, const Tile &t, const float *acc,
                                                const QuantParams &p, int8_t *q) {
    uint32_t w4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float *g = acc + 4 * k;
        if constexpr (MODE == CM_FAST) {
            w4[k] = codes4_fast(g[0], g[1], g[2], g[3], p.s, p.r);
        } else {
            w4[k] = pack4(code_of<MODE>(g[0], p), code_of<MODE>(g[1], p),
                          code_of<MODE>(g[2], p), code_of<MODE>(g[3], p));
        }
    }
    const int64_t i0 = j * RV;
    const uint4 pk = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    if (i0 >= t.begin && i0 + RV <= t.end) store_stream(q + i0, pk);
    else store_codes_part(q, i0, RV, t.begin, t.end, pk);
}

template <int S, int BLOCK, int MODE>
__device__ __forceinline__ void requantize_tile_mode(const Tile &t, const float (&acc)[S][RV],
                                                     const QuantParams &p, int8_t *q) {
    const int64_t tid = opaque_tid<BLOCK>();
    const int64_t j0 = t.begin / RV, j1 = (t.end + RV - 1) / RV;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t j = j0 + static_cast<int64_t>(s) * BLOCK + tid;
        if (j >= j1) continue;
        requantize_slot<MODE>(j, t, acc[s], p, q);
    }
}

template <int S, int BLOCK>
__device__ __forceinline__ void requantize_tile(const Tile &t, const float (&acc)[S][RV],
                                                const QuantParams &p, int8_t *q) {
    const int mode = __builtin_amdgcn_readfirstlane(p.mode);
    if (mode == CM_FAST) requantize_tile_mode<S, BLOCK, CM_FAST>(t, acc, p, q);
    else if (mode == CM_EXACT) requantize_tile_mode<S, BLOCK, CM_EXACT>(t, acc, p, q);
    else requantize_tile_mode<S, BLOCK, CM_ZERO>(t, acc, p, q);
}

// Small units: one wave per unit.  A unit of at most 64 slots takes one
// slot per lane and more ranks in flight.  With HALVES (narrow reduce
// tables), a unit of up to twice the wave's 64 * SR slots is summed in two
// halves, the first half's sums parked meanwhile in this wave's 8 KiB of
// LDS (slot group g of lane l at wpark[g * 64 + l]; each lane reads back
// only its own), and both halves are requantized with the whole unit's
// scale.  Multi-slot units load one rank ahead (the persistent kernels'
// registers are sized for whole tiles).
template <int SR, bool HALVES>
__device__ __forceinline__ void reduce_small_unit(const RArgs &a, int64_t item, float4 *wpark) {
    const Tile t = load_desc(a.small, item);
    float acc[SR][RV];
    const int64_t half_end = (t.begin / RV + 64 * SR) * RV;
    if (HALVES && t.end > half_end) {
        const int lane = threadIdx.x & 63;
        uint32_t m = 0;
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            Tile th = t;
            if (h == 0) th.end = half_end;
            else th.begin = half_end;
            reduce_tile<SR, 64, 1>(a, th, acc);
            if (a.r) store_sum<SR, 64>(th, acc, a.r);
            m = umax(m, acc_absmax<SR>(acc));
            if (h == 0) {
#pragma unroll
                for (int s = 0; s < SR; ++s)
#pragma unroll
                    for (int g = 0; g < RV / 4; ++g)
                        wpark[(s * (RV / 4) + g) * 64 + lane] = make_float4(
                            acc[s][4 * g], acc[s][4 * g + 1], acc[s][4 * g + 2], acc[s][4 * g + 3]);
            }
        }
        m = wave_max(m);
        const float sc = __fdiv_rn(__uint_as_float(m), 127.0f);
        if (lane == 0) a.scale_out[t.unit] = sc;
        const QuantParams qp = quant_params(sc, true);
#pragma unroll 1
        for (int h = 1; h >= 0; --h) {  // the second half is still in registers
            Tile th = t;
            if (h == 0) {
                th.end = half_end;
#pragma unroll
                for (int s = 0; s < SR; ++s)
#pragma unroll
                    for (int g = 0; g < RV / 4; ++g) {
                        const float4 v = wpark[(s * (RV / 4) + g) * 64 + lane];
                        acc[s][4 * g] = v.x;
                        acc[s][4 * g + 1] = v.y;
                        acc[s][4 * g + 2] = v.z;
                        acc[s][4 * g + 3] = v.w;
                    }
            } else {
                th.begin = half_end;
            }
            requantize_tile<SR, 64>(th, acc, qp, a.q_out);
        }
        return;
    }
    if ((t.end + RV - 1) / RV - t.begin / RV <= 64) {
        // one slot per lane: registers for the ranks' loads four at a time,
        // eight in flight, instead of one or two
        float acc1[1][RV];
        reduce_tile<1, 64, 4>(a, t, acc1);
        if (a.r) store_sum<1, 64>(t, acc1, a.r);
        const uint32_t m = wave_max(acc_absmax<1>(acc1));
        const float sc = __fdiv_rn(__uint_as_float(m), 127.0f);
        if ((threadIdx.x & 63) == 0) a.scale_out[t.unit] = sc;
        requantize_tile<1, 64>(t, acc1, quant_params(sc, true), a.q_out);
        return;
    }
    reduce_tile<SR, 64, 1>(a, t, acc);
    if (a.r) store_sum<SR, 64>(t, acc, a.r);
    const uint32_t m = wave_max(acc_absmax<SR>(acc));
    const float sc = __fdiv_rn(__uint_as_float(m), 127.0f);
    if ((threadIdx.x & 63) == 0) a.scale_out[t.unit] = sc;
    requantize_tile<SR, 64>(t, acc, quant_params(sc, true), a.q_out);
}

// Hot path for narrow tiles (one slot per lane): reduce + requantize of
// every tile, one read of the codes.  A work group sums its next tile (and
// publishes that tile's max) before it waits for the current tile's unit
// max, so the wait overlaps a whole tile of memory traffic; both tiles'
// sums are in registers.
template <int S, int BLOCK>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
void k_reduce_coop(const RArgs a) {
    // the small phase's half-unit sums: 8 KiB per wave
    __shared__ float4 spark[(BLOCK / 64) * SMALL_SLOTS_R * (RV / 4) * 64];
    float4 *wpark = spark + (threadIdx.x >> 6) * (SMALL_SLOTS_R * (RV / 4) * 64);
    __shared__ uint32_t sh[BLOCK / 64];
    __shared__ uint32_t s_val[2];  // unit max, next ticket
    const int64_t total = a.n_tiles;
    const uint32_t tag = launch_tag(a.ctl);
    int64_t tk = blockIdx.x;
    float acc_c[S][RV], acc_n[S][RV];
    Tile tc{};
    uint32_t mc = 0;
    uint64_t arr_c = 0;
    if (tk < total) {
        tc = load_desc(a.tiles, tk);
        reduce_tile<S, BLOCK>(a, tc, acc_c);
        if (a.r) store_sum<S, BLOCK>(tc, acc_c, a.r);
        mc = block_max<BLOCK>(acc_absmax<S>(acc_c), sh);
        if (tc.count > 1 && threadIdx.x < 64)
            arr_c = unit_publish(a.pub, a.cnt + tc.slot, static_cast<int32_t>(tk), mc, tag);
    }
    while (tk < total) {
        if (threadIdx.x == 0)  // (no dynamic ticket if the static ones cover every tile)
            s_val[1] = static_cast<int64_t>(gridDim.x) < total ? take_ticket(a.ctl, gridDim.x)
                                                               : static_cast<uint32_t>(total);
        __syncthreads();
        const int64_t tn = s_val[1];
        const bool more = tn < total;
        Tile tnx{};
        uint32_t mn = 0;
        uint64_t arr_n = 0;
        if (more) {
            tnx = load_desc(a.tiles, tn);
            reduce_tile<S, BLOCK>(a, tnx, acc_n);
            if (a.r) store_sum<S, BLOCK>(tnx, acc_n, a.r);
            mn = block_max<BLOCK>(acc_absmax<S>(acc_n), sh);
            if (tnx.count > 1 && threadIdx.x < 64) {
                arr_n = unit_publish(a.pub, a.cnt + tnx.slot, static_cast<int32_t>(tn), mn, tag);
                if (__shfl(arr_n, 0, 64) % static_cast<uint64_t>(tnx.count) == 0)  // last: gather now
                    (void)unit_max(a.pub, a.res + tnx.slot, static_cast<int32_t>(tn), tnx.first,
                                   tnx.count, mn, arr_n, tag, a.faults);
            }
        }
        uint32_t m = mc;
        if (tc.count > 1) {
            if (threadIdx.x < 64) {
                const uint32_t um = unit_max(a.pub, a.res + tc.slot, static_cast<int32_t>(tk),
                                             tc.first, tc.count, mc, arr_c, tag, a.faults);
                if (threadIdx.x == 0) s_val[0] = um;
            }
            __syncthreads();
            m = s_val[0];
        }
        const float sc = __fdiv_rn(__uint_as_float(m), 127.0f);
        if (threadIdx.x == 0 && tk == tc.first) a.scale_out[tc.unit] = sc;
        requantize_tile<S, BLOCK>(tc, acc_c, quant_params(sc, true), a.q_out);
        __syncthreads();
        if (!more) break;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int k = 0; k < RV; ++k) acc_c[s][k] = acc_n[s][k];
        tc = tnx;
        mc = mn;
        arr_c = arr_n;
        tk = tn;
    }
    small_phase<BLOCK>(a.n_small,
                       [&](int64_t item) { reduce_small_unit<SMALL_SLOTS_R, true>(a, item, wpark); });
    launch_exit(a.ctl);
}

// Hot path for wide tiles (two slots per lane): as k_reduce_coop, but the
// held tile's sums wait in LDS while the next tile is summed in registers.
// Each lane parks its own sums (as 16-byte words, lane-contiguous, so the
// stores and loads are free of bank conflicts) and reads back only its own,
// so parking needs no barrier.  Two tiles of sums would not fit in
// registers next to a tile's loads; in LDS they take 128 bytes per lane
// (64 KiB for 512 lanes, 128 KiB for the 1024 lanes of a chunk-wide tile).
// WT > 0: built for exactly WT ranks (8 and 16 are), the tiles' rank loop
// unrolled.
template <int S, int BLOCK, int WT = 0>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
void k_reduce_coop_wide(const RArgs a) {
    small_phase<BLOCK>(a.n_small,
                       [&](int64_t item) { reduce_small_unit<SMALL_SLOTS_R, false>(a, item, nullptr); });
    __shared__ uint32_t sh[BLOCK / 64];
    __shared__ uint32_t s_val[2];  // unit max, next ticket
    __shared__ float4 park[S * RV / 4][BLOCK];
    const int64_t total = a.n_tiles;
    const uint32_t tag = launch_tag(a.ctl);
    const int lane = threadIdx.x;
    auto put = [&](const float (&acc)[S][RV]) {
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int g = 0; g < RV / 4; ++g)
                park[s * (RV / 4) + g][lane] = make_float4(acc[s][4 * g], acc[s][4 * g + 1],
                                                           acc[s][4 * g + 2], acc[s][4 * g + 3]);
    };
    auto get = [&](float (&acc)[S][RV]) {
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int g = 0; g < RV / 4; ++g) {
                const float4 v = park[s * (RV / 4) + g][lane];
                acc[s][4 * g] = v.x;
                acc[s][4 * g + 1] = v.y;
                acc[s][4 * g + 2] = v.z;
                acc[s][4 * g + 3] = v.w;
            }
    };
    int64_t tk = blockIdx.x;
    Tile tc{};
    uint32_t mc = 0;
    uint64_t arr_c = 0;
    if (tk < total) {
        float acc[S][RV];
        tc = load_desc(a.tiles, tk);
        reduce_tile<S, BLOCK, 1, true, WT>(a, tc, acc);
        if (a.r) store_sum<S, BLOCK>(tc, acc, a.r);
        mc = block_max<BLOCK>(acc_absmax<S>(acc), sh);
        if (tc.count > 1 && threadIdx.x < 64)
            arr_c = unit_publish(a.pub, a.cnt + tc.slot, static_cast<int32_t>(tk), mc, tag);
        put(acc);
    }
    while (tk < total) {
        if (threadIdx.x == 0)  // (no dynamic ticket if the static ones cover every tile)
            s_val[1] = static_cast<int64_t>(gridDim.x) < total ? take_ticket(a.ctl, gridDim.x)
                                                               : static_cast<uint32_t>(total);
        __syncthreads();
        const int64_t tn = s_val[1];
        const bool more = tn < total;
        Tile tnx{};
        uint32_t mn = 0;
        uint64_t arr_n = 0;
        float acc_n[S][RV];
        if (more) {
            tnx = load_desc(a.tiles, tn);
            reduce_tile<S, BLOCK, 1, true, WT>(a, tnx, acc_n);
            if (a.r) store_sum<S, BLOCK>(tnx, acc_n, a.r);
            mn = block_max<BLOCK>(acc_absmax<S>(acc_n), sh);
            if (tnx.count > 1 && threadIdx.x < 64) {
                arr_n = unit_publish(a.pub, a.cnt + tnx.slot, static_cast<int32_t>(tn), mn, tag);
                if (__shfl(arr_n, 0, 64) % static_cast<uint64_t>(tnx.count) == 0)  // last: gather now
                    (void)unit_max(a.pub, a.res + tnx.slot, static_cast<int32_t>(tn), tnx.first,
                                   tnx.count, mn, arr_n, tag, a.faults);
            }
        }
        uint32_t m = mc;
        if (tc.count > 1) {
            if (threadIdx.x < 64) {
                const uint32_t um = unit_max(a.pub, a.res + tc.slot, static_cast<int32_t>(tk),
                                             tc.first, tc.count, mc, arr_c, tag, a.faults);
                if (threadIdx.x == 0) s_val[0] = um;
            }
            __syncthreads();
            m = s_val[0];
        }
        const float sc = __fdiv_rn(__uint_as_float(m), 127.0f);
        if (threadIdx.x == 0 && tk == tc.first) a.scale_out[tc.unit] = sc;
        {
            float acc_c[S][RV];
            get(acc_c);
            requantize_tile<S, BLOCK>(tc, acc_c, quant_params(sc, true), a.q_out);
        }
        __syncthreads();
        if (!more) break;
        put(acc_n);
        tc = tnx;
        mc = mn;
        arr_c = arr_n;
        tk = tn;
    }
    launch_exit(a.ctl);
}

// Tables whose units all fit one tile and whose small units hold most of
// the elements (many short tensors) run both stages as plain launches whose
// work groups never wait on each other: the quantize takes one wave per
// (rank, unit) item for units of up to 64 * SHORT_SLOTS_Q slots
// (k_quantize_small), the reduce one wave per piece of 64 slots
// (k_reduce_pieces), and the few other units one work group per tile
// (k_quantize, k_reduce).  With no tile path beside them, these kernels need
// fewer registers than the persistent ones, so more waves are resident, and
// each wave's work is its only item (none waits for the one before it on
// the same wave).
// Two waves per work group in the quantize: a group leaves only when its
// slowest unit is done, and the units of one group may differ in length a
// thousandfold.
constexpr int SMALL_BLOCK = 128;

template <typename TIn, bool MUL>
__global__ __launch_bounds__(SMALL_BLOCK) void k_quantize_small(const QArgs a) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) * (SMALL_BLOCK / 64) +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= static_cast<int64_t>(a.W) * a.n_packs) return;
    const int w = static_cast<int>(item / a.n_packs);
    const Pack pk = load_pack(a.packs, item - static_cast<int64_t>(w) * a.n_packs);
    if (pk.lanes == 64) quantize_wave_unit<TIn, SHORT_SLOTS_Q, MUL>(a, w, load_desc(a.small, pk.first));
    else quantize_pack<TIn, MUL>(a, w, pk);
}

// Rank-order dequant-accumulate of one wave's piece (at most 64 slots, one
// per lane), eight ranks at a time: the eight ranks' code pointers are read
// together (one scalar load), then all eight ranks' loads are issued, each
// lane addressing its slot by a 32-bit offset from the piece's first slot,
// before any is accumulated.  As in reduce_tile, a slot at the buffer's
// short end is summed again from its bytes, and sums of elements outside
// the piece are cleared.
__device__ __forceinline__ void reduce_piece(const RArgs &a, const Tile &t, float (&acc)[1][RV]) {
    const int64_t lane = opaque_tid<64>();
    const int64_t j0 = t.begin / RV, j1 = (t.end + RV - 1) / RV;
#pragma unroll
    for (int k = 0; k < RV; ++k) acc[0][k] = 0.0f;
    const int64_t nfull = a.n / RV;
    const int64_t jmax = (j1 < nfull ? j1 : nfull) - 1;
    const int64_t j = j0 + lane;
    // slot jb + o, o = min(j - jb, jmax - jb), jb = min(j0, jmax)
    const int64_t jb = j0 < jmax ? j0 : jmax;
    const uint32_t lim = static_cast<uint32_t>(jmax - jb);
    const uint32_t o = static_cast<uint32_t>(j - jb) < lim ? static_cast<uint32_t>(j - jb) : lim;
    for (int w0 = 0; w0 < a.W; w0 += 8) {
        const int nr = a.W - w0 < 8 ? a.W - w0 : 8;
        // past the last rank, rank w0's slot again (loaded, never used): the
        // loads stay unconditional, so none waits for the ones before it
        const int8_t *qp[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int8_t *q = a.q[w0 + r];  // w0 + 8 <= GQ_MAX_RANKS
            qp[r] = r < nr ? q : a.q[w0];
        }
        uint4 v[8];
        if (jmax >= 0) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                v[r] = load_stream(reinterpret_cast<const uint4 *>(qp[r]) + jb + o);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (r >= nr) break;
            const uint4 c[1] = {v[r]};
            accumulate<1>(c, rank_scale(a, w0 + r, t.unit), acc);
        }
    }
    if (j < j1 && j >= nfull) {
        // the buffer's short last slot, from its bytes, in rank order
#pragma unroll
        for (int k = 0; k < RV; ++k) acc[0][k] = 0.0f;
        for (int w = 0; w < a.W; ++w) {
            const uint4 c[1] = {load_tail16(a.q[w], j * RV, a.n)};
            accumulate<1>(c, rank_scale(a, w, t.unit), acc);
        }
    }
    const int64_t i0 = j * RV;
    if (!(j < j1 && i0 >= t.begin && i0 + RV <= t.end)) {
#pragma unroll
        for (int k = 0; k < RV; ++k) {
            const int64_t i = i0 + k;
            if (!(j < j1 && i >= t.begin && i < t.end)) acc[0][k] = 0.0f;
        }
    }
}

// A pack's wave of a short reduce table: each group of lanes sums and
// requantizes its unit, one slot per lane, four ranks at a time (fewer
// registers than the pieces' eight, which would cost the kernel
// occupancy).  The ranks' scales differ across the wave (one unit per
// group), so they are vector loads, issued before the ranks' code loads
// (the in-order load count then lets each rank wait for its own loads
// only).  Lanes without a slot load rank 0's first slot (in every buffer,
// never used).
__device__ __forceinline__ void reduce_pack(const RArgs &a, const Pack &pk) {
    const PackLane pl = pack_lane(a.pack_units, pk);
    const Tile &t = pl.t;
    const int64_t j = t.begin / RV + pl.li, j1 = (t.end + RV - 1) / RV;
    const bool in = pl.live && j < j1;
    const int64_t nfull = a.n / RV;
    const int64_t js = (in && j < nfull) ? j : 0;
    const int32_t u = pl.live ? t.unit : 0;
    float sums[1][RV];
    float *acc = sums[0];
#pragma unroll
    for (int k = 0; k < RV; ++k) acc[k] = 0.0f;
    constexpr int PR = 4;
    for (int w0 = 0; w0 < a.W; w0 += PR) {
        const int nr = a.W - w0 < PR ? a.W - w0 : PR;
        float sw[PR];
#pragma unroll
        for (int r = 0; r < PR; ++r) sw[r] = a.scale[r < nr ? w0 + r : w0][u];
        uint4 v[PR];
        if (nfull > 0) {
#pragma unroll
            for (int r = 0; r < PR; ++r)
                v[r] = load_stream(reinterpret_cast<const uint4 *>(a.q[r < nr ? w0 + r : w0]) + js);
        }
#pragma unroll
        for (int r = 0; r < PR; ++r) {
            if (r >= nr) break;
            const uint4 c[1] = {v[r]};
            accumulate<1>(c, sw[r], sums);
        }
    }
    if (in && j >= nfull) {
        // the buffer's short last slot, from its bytes, in rank order
#pragma unroll
        for (int k = 0; k < RV; ++k) acc[k] = 0.0f;
        for (int w = 0; w < a.W; ++w) {
            const uint4 c[1] = {load_tail16(a.q[w], j * RV, a.n)};
            accumulate<1>(c, a.scale[w][u], sums);
        }
    }
    // elements outside the unit never reach a max or a store
#pragma unroll
    for (int k = 0; k < RV; ++k) {
        const int64_t i = j * RV + k;
        if (!(in && i >= t.begin && i < t.end)) acc[k] = 0.0f;
    }
    if (in && a.r) store_sum_slot(j, t, acc, a.r);
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < RV; ++k) m = umax(m, __float_as_uint(acc[k]) & kAbsMask);
    m = group_max(m, pk.lanes);
    const float sc = __fdiv_rn(__uint_as_float(m), 127.0f);
    if (pl.live && pl.li == 0) a.scale_out[t.unit] = sc;
    if (in) {
        const QuantParams qp = quant_params(sc, true);
        if (qp.mode == CM_FAST) requantize_slot<CM_FAST>(j, t, acc, qp, a.q_out);
        else if (qp.mode == CM_EXACT) requantize_slot<CM_EXACT>(j, t, acc, qp, a.q_out);
        else requantize_slot<CM_ZERO>(j, t, acc, qp, a.q_out);
    }
}

// Short reduce tables: one wave per piece of PIECE_SLOTS slots (eight
// ranks' loads in flight, reduce_piece), the waves of a unit in one work
// group.  Each wave's max goes through LDS to the unit's other waves, and
// every wave requantizes its own piece with the unit's scale.  Against one
// wave per unit (the unit summed in two halves of 128 slots, one parked in
// LDS), a unit's slots are summed by several waves at once, with fewer
// registers per wave.
__global__ __launch_bounds__(PIECE_WAVES * 64) void k_reduce_pieces(const RArgs a) {
    __shared__ uint32_t wmax[PIECE_WAVES];
    const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Tile p = load_desc(a.small, static_cast<int64_t>(blockIdx.x) * PIECE_WAVES + v);
    static_assert(PIECE_SLOTS == 64, "reduce_piece takes one slot per lane");
    if (p.slot == PACK_WAVE) {  // a pack: no unit shared with another wave
        reduce_pack(a, load_pack(a.packs, p.first));
        __syncthreads();  // the group's one barrier, as the piece waves'
        return;
    }
    float acc[1][RV];
    uint32_t m = 0;
    if (p.count > 0) {
        reduce_piece(a, p, acc);
        if (a.r) store_sum<1, 64>(p, acc, a.r);
        m = wave_max(acc_absmax<1>(acc));
    }
    if ((threadIdx.x & 63) == 0) wmax[v] = m;
    __syncthreads();
    if (p.count == 0) return;
    uint32_t um = 0;
    for (int i = 0; i < p.count; ++i) um = umax(um, wmax[p.first + i]);
    const float sc = __fdiv_rn(__uint_as_float(um), 127.0f);
    if (v == p.first && (threadIdx.x & 63) == 0) a.scale_out[p.unit] = sc;
    requantize_tile<1, 64>(p, acc, quant_params(sc, true), a.q_out);
}

enum RMode { R_SUM = 0, R_PASS1 = 1, R_FUSED = 2 };

// Non-persistent reduce: the plain sum (R_SUM), and the two-launch form
// whose work groups never wait on each other (R_PASS1 writes per-tile
// maxima, R_FUSED recomputes the sum and requantizes), used for units with
// more tiles than resident work groups and where another kernel may share
// the device.
template <int S, int BLOCK, int MODE>
__global__ __launch_bounds__(BLOCK) void k_reduce(const RArgs a) {
    __shared__ uint32_t sh[BLOCK / 64];
    const int32_t tix = (MODE == R_PASS1) ? a.list[blockIdx.x] : static_cast<int32_t>(blockIdx.x);
    const Tile t = load_desc(a.tiles, tix);
    float acc[S][RV];
    if constexpr (S == 1) reduce_tile<S, BLOCK>(a, t, acc);
    else reduce_tile<S, BLOCK, 1, true>(a, t, acc);
    if (a.r != nullptr && (MODE != R_FUSED || t.count == 1)) store_sum<S, BLOCK>(t, acc, a.r);
    if (MODE == R_SUM) return;
    uint32_t m;
    if (MODE == R_PASS1) {
        m = block_max<BLOCK>(acc_absmax<S>(acc), sh);
        if (threadIdx.x == 0) a.partial[tix] = m;
        return;
    }
    if (t.count == 1) {
        m = block_max<BLOCK>(acc_absmax<S>(acc), sh);
    } else {
        const uint32_t *p = a.partial + t.first;
        uint32_t pm = 0;
        for (int i = threadIdx.x; i < t.count; i += BLOCK) pm = umax(pm, p[i]);
        m = block_max<BLOCK>(pm, sh);
    }
    const float sc = __fdiv_rn(__uint_as_float(m), 127.0f);
    if (threadIdx.x == 0 && tix == t.first) a.scale_out[t.unit] = sc;
    requantize_tile<S, BLOCK>(t, acc, quant_params(sc, true), a.q_out);
}

// Copy of a table's fault count into a caller's buffer, ordered on the
// caller's stream (a kernel rather than a memory copy, so that it can also
// be captured into a graph).
__global__ void k_copy_word(const uint32_t *src, uint32_t *dst) {
    if (threadIdx.x == 0) dst[0] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- launch helpers -------------------------------------------------------------------

struct DeviceInfo {
    int cus = 0;
};

DeviceInfo device_info() {
    static thread_local int cached_dev = -1;
    static thread_local DeviceInfo info;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev != cached_dev) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) info.cus = prop.multiProcessorCount;
        cached_dev = dev;
    }
    return info;
}

// Resident work groups of kernel K on the current device (0 on error),
// cached per kernel and device.
template <auto K>
int64_t resident_groups(int block) {
    static thread_local int cached_dev = -1;
    static thread_local int64_t cached = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev == cached_dev) return cached;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, block, 0) != hipSuccess)
        return 0;
    cached = static_cast<int64_t>(per_cu) * device_info().cus;
    cached_dev = dev;
    return cached;
}

// A persistent kernel: `groups` never exceeds the resident capacity.  (A
// cooperative launch would also guarantee co-residency, but with the ROCm
// runtime it costs about 20 us of extra queue synchronization per launch,
// and the schedule above needs only that the grid fits.)
template <typename K, typename A>
hipError_t launch_persistent(K kernel, int64_t groups, int block, const A &args, hipStream_t s) {
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(groups)), dim3(block), 0, s, args);
    return hipGetLastError();
}

template <typename TIn, int BLOCK, int S, bool MUL>
constexpr auto coop_quantize_kernel() {
    if constexpr (BLOCK == Q_BLOCK_CHUNK) return k_quantize_chunk<TIn, S, BLOCK, MUL>;
    else return k_quantize_layer<TIn, S, BLOCK, MUL>;
}

template <typename TIn, int BLOCK, int S, bool MUL>
hipError_t quantize_geom(const QArgs &a, const Table &t, hipStream_t s, int64_t cap) {
    const dim3 block(BLOCK);
    const dim3 grid(static_cast<unsigned>(t.n_tiles), static_cast<unsigned>(a.W));
    if (a.amax != nullptr) {
        hipLaunchKernelGGL((k_quantize<TIn, S, BLOCK, MUL, Q_GIVEN>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    if (short_table(t)) {
        // many short tensors: no exchange needed (see k_quantize_small)
        if (t.n_packs > 0) {
            QArgs c = a;
            c.small = t.d_short;
            c.n_small = t.n_short;
            c.packs = t.d_packs;
            c.n_packs = t.n_packs;
            const int64_t items = static_cast<int64_t>(a.W) * t.n_packs;
            hipLaunchKernelGGL((k_quantize_small<TIn, MUL>),
                               dim3(static_cast<unsigned>((items + SMALL_BLOCK / 64 - 1) / (SMALL_BLOCK / 64))),
                               dim3(SMALL_BLOCK), 0, s, c);
        }
        if (t.n_rest > 0) {
            QArgs c = a;
            c.tiles = t.d_rest;
            c.n_tiles = t.n_rest;
            hipLaunchKernelGGL((k_quantize<TIn, S, BLOCK, MUL, Q_FUSED>),
                               dim3(static_cast<unsigned>(t.n_rest), static_cast<unsigned>(a.W)), block, 0, s, c);
        }
        return hipGetLastError();
    }
    constexpr auto coop = coop_quantize_kernel<TIn, BLOCK, S, MUL>();
    int64_t resident = resident_groups<coop>(BLOCK);
    if (cap > 0 && cap < resident) resident = cap;
    if (resident >= t.big_max_count) {
        // one launch: the tiles of the other units through the ticket
        // counter, then the small units (one wave each)
        QArgs c = a;
        c.tiles = t.d_big;
        c.n_tiles = t.n_big;
        const int64_t small_groups =
            (static_cast<int64_t>(a.W) * t.n_small + BLOCK / 64 - 1) / (BLOCK / 64);
        int64_t groups = static_cast<int64_t>(a.W) * t.n_big;
        if (small_groups > groups) groups = small_groups;
        return launch_persistent(coop, groups < resident ? groups : resident, BLOCK, c, s);
    }
    // a unit with more tiles than resident work groups: two launches
    QArgs p = a;
    p.list = t.d_multi;
    hipLaunchKernelGGL((k_tile_absmax<TIn, S, BLOCK>),
                       dim3(static_cast<unsigned>(t.n_multi), static_cast<unsigned>(a.W)), block, 0, s, p);
    hipLaunchKernelGGL((k_quantize<TIn, S, BLOCK, MUL, Q_FUSED>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <typename TIn, bool MUL>
hipError_t quantize_typed(const QArgs &a0, const Table &t, hipStream_t s, int64_t cap) {
    QArgs a = a0;
    a.partial = t.d_partial;
    a.tiles = t.d_tiles;
    a.pub = t.d_pub;
    a.res = t.d_res;
    a.cnt = t.d_cnt;
    a.ctl = t.d_ctl;
    a.n_multi_units = t.n_multi_units;
    a.small = t.d_small;
    a.n_small = t.n_small;
    if (t.block == Q_BLOCK_CHUNK && t.slots == Q_SLOTS_CHUNK_SHORT)
        return quantize_geom<TIn, Q_BLOCK_CHUNK, Q_SLOTS_CHUNK_SHORT, MUL>(a, t, s, cap);
    if (t.block == Q_BLOCK_CHUNK) return quantize_geom<TIn, Q_BLOCK_CHUNK, Q_SLOTS_CHUNK, MUL>(a, t, s, cap);
    return quantize_geom<TIn, Q_BLOCK_LAYER, Q_SLOTS_LAYER, MUL>(a, t, s, cap);
}

template <typename TIn, int BLOCK, int S>
void absmax_geom(const QArgs &a, const Table &t, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(t.n_tiles), static_cast<unsigned>(a.W));
    hipLaunchKernelGGL((k_tile_absmax<TIn, S, BLOCK>), grid, dim3(BLOCK), 0, s, a);
}

}  // namespace

// ---- launchers ----------------------------------------------------------------------------

// The quantize table geometries the launchers are built for.
static bool quantize_geometry(const Table &t) {
    if (t.block == Q_BLOCK_LAYER) return t.slots == Q_SLOTS_LAYER;
    return t.block == Q_BLOCK_CHUNK && (t.slots == Q_SLOTS_CHUNK || t.slots == Q_SLOTS_CHUNK_SHORT);
}

hipError_t launch_absmax(const QArgs &a0, gq_dtype dt, const Table &t, hipStream_t s) {
    if (!table_ready(t, a0.n_units) || !quantize_geometry(t)) return hipErrorInvalidValue;
    QArgs a = a0;
    a.list = nullptr;
    a.partial = t.d_partial;
    a.unit_first = t.d_unit_first;
    a.tiles = t.d_tiles;
    const bool mul = a.in_mul != 1.0f;
    const int64_t total = static_cast<int64_t>(a.W) * a.n_units;
    const unsigned nb = static_cast<unsigned>((total + 255) / 256);
    const bool chunk = t.block == Q_BLOCK_CHUNK;
    const bool rows8 = chunk && t.slots == Q_SLOTS_CHUNK_SHORT;
    if (dt == GQ_F32) {
        if (rows8) absmax_geom<float, Q_BLOCK_CHUNK, Q_SLOTS_CHUNK_SHORT>(a, t, s);
        else if (chunk) absmax_geom<float, Q_BLOCK_CHUNK, Q_SLOTS_CHUNK>(a, t, s);
        else absmax_geom<float, Q_BLOCK_LAYER, Q_SLOTS_LAYER>(a, t, s);
        hipLaunchKernelGGL(k_absmax_finalize<float>, dim3(nb), dim3(256), 0, s, a, mul);
    } else {
        if (rows8) absmax_geom<__half, Q_BLOCK_CHUNK, Q_SLOTS_CHUNK_SHORT>(a, t, s);
        else if (chunk) absmax_geom<__half, Q_BLOCK_CHUNK, Q_SLOTS_CHUNK>(a, t, s);
        else absmax_geom<__half, Q_BLOCK_LAYER, Q_SLOTS_LAYER>(a, t, s);
        hipLaunchKernelGGL(k_absmax_finalize<__half>, dim3(nb), dim3(256), 0, s, a, mul);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(const QArgs &a, gq_dtype dt, const Table &t, hipStream_t s,
                           int64_t cap) {
    if (!table_ready(t, a.n_units) || !quantize_geometry(t)) return hipErrorInvalidValue;
    const bool mul = a.in_mul != 1.0f;
    if (dt == GQ_F32)
        return mul ? quantize_typed<float, true>(a, t, s, cap)
                   : quantize_typed<float, false>(a, t, s, cap);
    return mul ? quantize_typed<__half, true>(a, t, s, cap)
               : quantize_typed<__half, false>(a, t, s, cap);
}

template <int S, int BLOCK, int WT = 0>
constexpr auto coop_reduce_kernel() {
    if constexpr (S == R_SLOTS_WIDE) return k_reduce_coop_wide<S, BLOCK, WT>;
    else return k_reduce_coop<S, BLOCK>;
}

template <int S, int BLOCK, int WT>
hipError_t reduce_persistent(const RArgs &a, const Table &t, int64_t cap, hipStream_t s,
                             bool &launched) {
    constexpr auto coop = coop_reduce_kernel<S, BLOCK, WT>();
    int64_t resident = resident_groups<coop>(BLOCK);
    if (cap > 0 && cap < resident) resident = cap;
    launched = false;
    if (resident < t.big_max_count) return hipSuccess;
    RArgs c = a;
    c.small = t.d_small;
    c.n_small = t.n_small;
    c.tiles = t.d_big;
    c.n_tiles = t.n_big;
    const int64_t small_groups = (t.n_small + BLOCK / 64 - 1) / (BLOCK / 64);
    const int64_t groups = t.n_big > small_groups ? t.n_big : small_groups;
    launched = true;
    return launch_persistent(coop, groups < resident ? groups : resident, BLOCK, c, s);
}

template <int S, int BLOCK>
hipError_t reduce_geom(RArgs a, const Table &t, bool requantize, bool wait_free, hipStream_t s,
                       int64_t cap) {
    const dim3 block(BLOCK);
    if (!requantize) {
        a.list = nullptr;
        hipLaunchKernelGGL((k_reduce<S, BLOCK, R_SUM>), dim3(static_cast<unsigned>(t.n_tiles)),
                           block, 0, s, a);
        return hipGetLastError();
    }
    if (requantize && short_table(t)) {
        // many short tensors: no exchange needed (see k_reduce_pieces)
        if (t.n_short > 0) {
            RArgs c = a;
            c.small = t.d_short;
            c.n_small = t.n_short;
            c.packs = t.d_packs;
            c.pack_units = t.d_pack_units;
            hipLaunchKernelGGL(k_reduce_pieces, dim3(static_cast<unsigned>(t.n_short / PIECE_WAVES)),
                               dim3(PIECE_WAVES * 64), 0, s, c);
        }
        if (t.n_rest > 0) {
            RArgs c = a;
            c.tiles = t.d_rest;
            c.n_tiles = t.n_rest;
            hipLaunchKernelGGL((k_reduce<S, BLOCK, R_FUSED>), dim3(static_cast<unsigned>(t.n_rest)), block, 0, s, c);
        }
        return hipGetLastError();
    }
    if (!wait_free) {
        bool launched = false;
        hipError_t e;
        if (S == R_SLOTS_WIDE && a.W == 8) e = reduce_persistent<S, BLOCK, 8>(a, t, cap, s, launched);
        else if (S == R_SLOTS_WIDE && a.W == 16) e = reduce_persistent<S, BLOCK, 16>(a, t, cap, s, launched);
        else e = reduce_persistent<S, BLOCK, 0>(a, t, cap, s, launched);
        if (launched || e != hipSuccess) return e;
    }
    if (t.n_multi > 0) {
        RArgs p = a;
        p.list = t.d_multi;
        hipLaunchKernelGGL((k_reduce<S, BLOCK, R_PASS1>), dim3(static_cast<unsigned>(t.n_multi)),
                           block, 0, s, p);
    }
    a.list = nullptr;
    hipLaunchKernelGGL((k_reduce<S, BLOCK, R_FUSED>), dim3(static_cast<unsigned>(t.n_tiles)),
                       block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_copy_word(const uint32_t *src, uint32_t *dst, hipStream_t s) {
    hipLaunchKernelGGL(k_copy_word, dim3(1), dim3(64), 0, s, src, dst);
    return hipGetLastError();
}

template <typename TIn, bool MUL>
int64_t quantize_resident_typed(const Table &t) {
    if (t.block == Q_BLOCK_CHUNK && t.slots == Q_SLOTS_CHUNK_SHORT)
        return resident_groups<coop_quantize_kernel<TIn, Q_BLOCK_CHUNK, Q_SLOTS_CHUNK_SHORT, MUL>()>(
            Q_BLOCK_CHUNK);
    if (t.block == Q_BLOCK_CHUNK)
        return resident_groups<coop_quantize_kernel<TIn, Q_BLOCK_CHUNK, Q_SLOTS_CHUNK, MUL>()>(
            Q_BLOCK_CHUNK);
    return resident_groups<coop_quantize_kernel<TIn, Q_BLOCK_LAYER, Q_SLOTS_LAYER, MUL>()>(
        Q_BLOCK_LAYER);
}

int64_t quantize_resident(gq_dtype dt, bool mul, const Table &t) {
    if (dt == GQ_F32)
        return mul ? quantize_resident_typed<float, true>(t) : quantize_resident_typed<float, false>(t);
    return mul ? quantize_resident_typed<__half, true>(t) : quantize_resident_typed<__half, false>(t);
}

template <int BLOCK>
int64_t wide_resident() {
    int64_t r = resident_groups<coop_reduce_kernel<R_SLOTS_WIDE, BLOCK, 0>()>(BLOCK);
    const int64_t r8 = resident_groups<coop_reduce_kernel<R_SLOTS_WIDE, BLOCK, 8>()>(BLOCK);
    const int64_t r16 = resident_groups<coop_reduce_kernel<R_SLOTS_WIDE, BLOCK, 16>()>(BLOCK);
    if (r8 < r) r = r8;
    if (r16 < r) r = r16;
    return r;
}

int64_t reduce_resident(const Table &t) {
    if (t.block == R_BLOCK_CHUNK) return wide_resident<R_BLOCK_CHUNK>();
    if (t.slots == R_SLOTS_WIDE) return wide_resident<R_BLOCK>();
    return resident_groups<coop_reduce_kernel<R_SLOTS_NARROW, R_BLOCK>()>(R_BLOCK);
}

int64_t device_cus() { return device_info().cus; }

bool quantize_waits(gq_dtype dt, bool mul, const Table &t, int64_t cap) {
    if (short_table(t) || t.big_max_count <= 1) return false;
    int64_t resident = quantize_resident(dt, mul, t);
    if (cap > 0 && cap < resident) resident = cap;
    return resident >= t.big_max_count;
}

bool reduce_waits(const Table &t, int64_t cap) {
    if (short_table(t) || t.big_max_count <= 1) return false;
    int64_t resident = reduce_resident(t);
    if (cap > 0 && cap < resident) resident = cap;
    return resident >= t.big_max_count;
}

hipError_t launch_reduce(const RArgs &a0, const Table &t, bool requantize, bool wait_free,
                         hipStream_t s, int64_t cap) {
    if (!table_ready(t, 1)) return hipErrorInvalidValue;
    const bool chunk = t.block == R_BLOCK_CHUNK && t.slots == R_SLOTS_WIDE;
    if (!chunk && (t.block != R_BLOCK || (t.slots != R_SLOTS_NARROW && t.slots != R_SLOTS_WIDE)))
        return hipErrorInvalidValue;
    RArgs a = a0;
    a.tiles = t.d_tiles;
    a.partial = t.d_partial;
    a.n_tiles = t.n_tiles;
    a.pub = t.d_pub;
    a.res = t.d_res;
    a.cnt = t.d_cnt;
    a.ctl = t.d_ctl;
    if (chunk) return reduce_geom<R_SLOTS_WIDE, R_BLOCK_CHUNK>(a, t, requantize, wait_free, s, cap);
    if (t.slots == R_SLOTS_WIDE)
        return reduce_geom<R_SLOTS_WIDE, R_BLOCK>(a, t, requantize, wait_free, s, cap);
    return reduce_geom<R_SLOTS_NARROW, R_BLOCK>(a, t, requantize, wait_free, s, cap);
}

}  // namespace gq
