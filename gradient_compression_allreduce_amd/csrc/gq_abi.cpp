// gq_abi.cpp -- the extern "C" boundary of libgq.so: argument checks, the
// chunk planner, unit tables, error strings and kernel dispatch.
// Declarations and the contract of every entry point: include/gq.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "gq_internal.h"

namespace {

thread_local std::string g_last_error;

gq_status fail(gq_status code, const char *op, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = std::string(op) + ": " + buf;
    return code;
}

gq_status ok() {
    g_last_error.clear();
    return GQ_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The work tables of one slot geometry (see gq::Tile).
void build_tiles(const std::vector<int64_t> &off, int V, int64_t cap_slots,
                 std::vector<gq::Tile> &tiles, std::vector<int32_t> &multi,
                 std::vector<int32_t> &unit_first, int64_t &n_multi_units, int32_t &max_count) {
    const int64_t U = static_cast<int64_t>(off.size()) - 1;
    unit_first.resize(U + 1);
    n_multi_units = 0;
    max_count = 1;
    for (int64_t u = 0; u < U; ++u) {
        const int64_t a = off[u], b = off[u + 1];
        const int64_t first_slot = a / V, end_slot = (b + V - 1) / V;
        const int64_t slots = end_slot - first_slot;
        const int32_t first = static_cast<int32_t>(tiles.size());
        unit_first[u] = first;
        if (slots <= cap_slots) {
            tiles.push_back({a, b, static_cast<int32_t>(u), first, 1, -1});
            continue;
        }
        // as few tiles as the capacity allows, of sizes differing by at
        // most one slot (so that no tile of the unit is a sliver the others
        // wait on): tile m starts at slot floor(m * slots / cnt)
        const int64_t cnt = (slots + cap_slots - 1) / cap_slots;
        const int64_t q = slots / cnt, r = slots % cnt;
        auto start = [&](int64_t m) { return first_slot + m * q + (m * r) / cnt; };
        const int32_t slot = static_cast<int32_t>(n_multi_units++);
        if (cnt > max_count) max_count = static_cast<int32_t>(cnt);
        for (int64_t m = 0; m < cnt; ++m) {
            const int64_t sb = start(m) * V;
            const int64_t se = start(m + 1) * V;
            multi.push_back(static_cast<int32_t>(tiles.size()));
            tiles.push_back({sb > a ? sb : a, se < b ? se : b, static_cast<int32_t>(u), first,
                             static_cast<int32_t>(cnt), slot});
        }
    }
    unit_first[U] = static_cast<int32_t>(tiles.size());
}

// Lanes per unit of a pack for a unit spanning `slots` slots: the smallest
// power of two from PACK_MIN_LANES up that holds them, or 64 above 32.
int pack_lanes(int64_t slots) {
    int g = gq::PACK_MIN_LANES;
    while (g < 64 && g < slots) g *= 2;
    return g;
}

// Packs of the units `us` (all of `lanes` lanes each, in the given order),
// 64 / lanes units to a pack, appended to packs and their unit tiles to
// units (first: the unit's index in that list).
void add_packs(const std::vector<int64_t> &off, const std::vector<int64_t> &us, int lanes,
               std::vector<gq::Pack> &packs, std::vector<gq::Tile> &units) {
    const size_t per = static_cast<size_t>(64 / lanes);
    for (size_t i = 0; i < us.size(); i += per) {
        const size_t cnt = std::min(per, us.size() - i);
        packs.push_back({static_cast<int32_t>(units.size()), static_cast<int32_t>(cnt), lanes, 0});
        for (size_t k = 0; k < cnt; ++k) {
            const int64_t u = us[i + k];
            units.push_back({off[u], off[u + 1], static_cast<int32_t>(u),
                             static_cast<int32_t>(units.size()), 1, -1});
        }
    }
}

// The per-wave work of a short reduce table (see gq::Table::d_short).  A unit
// of at most 32 slots goes into a pack (several to a wave).  A unit of more
// than 32 and at most PIECE_WAVES * PIECE_SLOTS slots is cut into pieces of
// PIECE_SLOTS slots from its first slot.  Pieces and packs' waves are
// packed, each unit's pieces whole, into work groups of PIECE_WAVES waves,
// best fit in decreasing order of piece count (units are independent, so
// their order is free, and a work group with idle waves would hold
// resident slots for nothing).  The other units keep their one tile each (a
// short table has no multi-tile unit).
void build_pieces(const std::vector<int64_t> &off, int V, const std::vector<gq::Tile> &tiles,
                  const std::vector<int32_t> &unit_first, std::vector<gq::Tile> &pieces,
                  std::vector<gq::Pack> &packs, std::vector<gq::Tile> &pack_units,
                  std::vector<gq::Tile> &rest) {
    constexpr int PW = gq::PIECE_WAVES;
    constexpr int64_t PS = gq::PIECE_SLOTS;
    const int64_t U = static_cast<int64_t>(off.size()) - 1;
    auto span = [&](int64_t u) { return (off[u + 1] + V - 1) / V - off[u] / V; };
    // units by piece count, most first (counting sort, unit order within);
    // packs of the smallest units, one wave each
    std::vector<std::vector<int64_t>> by_k(PW + 1);
    std::vector<std::vector<int64_t>> by_lanes(7);  // index log2(lanes)
    for (int64_t u = 0; u < U; ++u) {
        const int64_t sl = span(u);
        const int64_t k = (sl + PS - 1) / PS;
        if (k > PW) {
            gq::Tile tl = tiles[unit_first[u]];
            tl.first = static_cast<int32_t>(rest.size());
            rest.push_back(tl);
        } else if (sl <= 32) {
            by_lanes[__builtin_ctz(static_cast<unsigned>(pack_lanes(sl)))].push_back(u);
        } else {
            by_k[k].push_back(u);
        }
    }
    for (int lg = 5; lg >= 2; --lg) add_packs(off, by_lanes[lg], 1 << lg, packs, pack_units);
    std::vector<std::vector<gq::Tile>> groups;
    std::vector<std::vector<int64_t>> with_free(PW);  // groups by free waves (1 .. PW-1)
    auto place = [&](int k) -> std::vector<gq::Tile> & {
        int c = k;
        while (c < PW && with_free[c].empty()) ++c;
        int64_t g;
        if (c < PW) {
            g = with_free[c].back();
            with_free[c].pop_back();
        } else {
            g = static_cast<int64_t>(groups.size());
            groups.emplace_back();
            c = PW;
        }
        if (c - k > 0) with_free[c - k].push_back(g);
        return groups[g];
    };
    for (int k = PW; k >= 1; --k) {
        for (const int64_t u : by_k[k]) {
            std::vector<gq::Tile> &grp = place(k);
            const int32_t first = static_cast<int32_t>(grp.size());
            const int64_t a = off[u], b = off[u + 1], j0 = a / V;
            for (int i = 0; i < k; ++i) {
                const int64_t pb = (j0 + PS * i) * V, pe = (j0 + PS * (i + 1)) * V;
                grp.push_back({pb > a ? pb : a, pe < b ? pe : b, static_cast<int32_t>(u), first, k,
                               -1});
            }
        }
        if (k == 1) {
            for (size_t i = 0; i < packs.size(); ++i)
                place(1).push_back({0, 0, -1, static_cast<int32_t>(i), 1, gq::PACK_WAVE});
        }
    }
    const gq::Tile empty = {0, 0, -1, 0, 0, -1};
    pieces.reserve(groups.size() * PW);
    for (const std::vector<gq::Tile> &grp : groups) {
        pieces.insert(pieces.end(), grp.begin(), grp.end());
        for (size_t i = grp.size(); i < static_cast<size_t>(PW); ++i) pieces.push_back(empty);
    }
}

// The per-wave work of a short quantize table: packs of the units of at
// most cap_slots slots (a unit of more than 32 slots alone in a pack of 64
// lanes; those first, the larger ones taking longer), their units in pack
// order; the other units keep their one tile each.
void build_short_units(const std::vector<int64_t> &off, int V, int64_t cap_slots,
                       const std::vector<gq::Tile> &tiles, const std::vector<int32_t> &unit_first,
                       std::vector<gq::Pack> &packs, std::vector<gq::Tile> &units,
                       std::vector<gq::Tile> &rest) {
    const int64_t U = static_cast<int64_t>(off.size()) - 1;
    std::vector<std::vector<int64_t>> by_lanes(7);  // index log2(lanes)
    for (int64_t u = 0; u < U; ++u) {
        const int64_t sl = (off[u + 1] + V - 1) / V - off[u] / V;
        if (sl <= cap_slots) {
            by_lanes[__builtin_ctz(static_cast<unsigned>(pack_lanes(sl)))].push_back(u);
        } else {
            gq::Tile tl = tiles[unit_first[u]];
            tl.first = static_cast<int32_t>(rest.size());
            rest.push_back(tl);
        }
    }
    for (int lg = 6; lg >= 2; --lg) add_packs(off, by_lanes[lg], 1 << lg, packs, units);
}

template <typename T>
hipError_t upload(T **dst, const std::vector<T> &src) {
    *dst = nullptr;
    if (src.empty()) return hipSuccess;
    hipError_t e = hipMalloc(reinterpret_cast<void **>(dst), src.size() * sizeof(T));
    if (e != hipSuccess) return e;
    return hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
}

void free_table(gq::Table &t) {
    if (t.d_tiles) (void)hipFree(t.d_tiles);
    if (t.d_small) (void)hipFree(t.d_small);
    if (t.d_big) (void)hipFree(t.d_big);
    if (t.d_multi) (void)hipFree(t.d_multi);
    if (t.d_partial) (void)hipFree(t.d_partial);
    if (t.d_unit_first) (void)hipFree(t.d_unit_first);
    if (t.d_pub) (void)hipFree(t.d_pub);
    if (t.d_ctl) (void)hipFree(t.d_ctl);
    if (t.d_res) (void)hipFree(t.d_res);
    if (t.d_cnt) (void)hipFree(t.d_cnt);
    if (t.d_short) (void)hipFree(t.d_short);
    if (t.d_packs) (void)hipFree(t.d_packs);
    if (t.d_pack_units) (void)hipFree(t.d_pack_units);
    if (t.d_rest) (void)hipFree(t.d_rest);
    t = gq::Table{};
}

gq_status check_units(const char *op, const gq_units *u) {
    if (!u) return fail(GQ_ERR_INVALID, op, "unit table is NULL");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(GQ_ERR_HIP, op, "hipGetDevice failed");
    if (dev != u->device)
        return fail(GQ_ERR_DEVICE, op, "current device %d, unit table lives on device %d", dev,
                    u->device);
    return GQ_OK;
}

gq_status check_ranks(const char *op, int32_t W) {
    if (W < 1 || W > GQ_MAX_RANKS)
        return fail(GQ_ERR_INVALID, op, "W = %d outside [1, %d]", W, GQ_MAX_RANKS);
    return GQ_OK;
}

template <typename P>
gq_status check_ptr_array(const char *op, const char *name, P const *arr, int32_t W,
                          uintptr_t align) {
    if (!arr) return fail(GQ_ERR_INVALID, op, "%s is NULL", name);
    for (int32_t w = 0; w < W; ++w) {
        if (!arr[w]) return fail(GQ_ERR_INVALID, op, "%s[%d] is NULL", name, w);
        if (!aligned(arr[w], align))
            return fail(GQ_ERR_ALIGN, op, "%s[%d] = %p is not %d-byte aligned", name, w,
                        static_cast<const void *>(arr[w]), static_cast<int>(align));
    }
    return GQ_OK;
}

gq_status check_ptr(const char *op, const char *name, const void *p, uintptr_t align) {
    if (!p) return fail(GQ_ERR_INVALID, op, "%s is NULL", name);
    if (!aligned(p, align))
        return fail(GQ_ERR_ALIGN, op, "%s = %p is not %d-byte aligned", name, p,
                    static_cast<int>(align));
    return GQ_OK;
}

gq_status launch_status(const char *op, hipError_t e) {
    if (e != hipSuccess) return fail(GQ_ERR_HIP, op, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

gq::TableId q_table(gq_dtype dt) { return dt == GQ_F32 ? gq::TAB_Q32 : gq::TAB_Q16; }

#define GQ_TRY(expr)                      \
    do {                                  \
        gq_status st_ = (expr);           \
        if (st_ != GQ_OK) return st_;     \
    } while (0)

}  // namespace

// A pipelined step plan: one unit table per bucket, with offsets relative to
// a 16-element boundary at or before the bucket's first element (so that
// every per-bucket buffer base stays 16-byte aligned), a second stream, and
// the events that order the two streams.
struct gq_pipe {
    int device = -1;
    int64_t n = 0;
    int64_t n_units = 0;
    int64_t n_buckets = 0;
    std::vector<int64_t> base;    // element offset of each bucket's tables
    std::vector<int64_t> u0;      // first unit of each bucket
    std::vector<gq_units *> tab;  // per-bucket unit tables
    int64_t slot_elems = 0;
    int64_t slot_units = 0;
    int32_t mode = GQ_PIPE_OVERLAP;
    hipStream_t aux = nullptr;
    hipEvent_t ev_q[2] = {nullptr, nullptr};
    hipEvent_t ev_r[2] = {nullptr, nullptr};
    hipEvent_t ev_done = nullptr;
};

extern "C" {

// Error reporting for the library's other host files (hidden, not part of
// the ABI): GQ_OK clears the text.
__attribute__((visibility("hidden"))) gq_status gq_set_error_internal(gq_status code,
                                                                      const char *op,
                                                                      const char *what) {
    if (code == GQ_OK) return ok();
    return fail(code, op, "%s", what);
}

const char *gq_last_error(void) { return g_last_error.c_str(); }

const char *gq_version(void) { return "gq 0.1 (gfx950)"; }

gq_status gq_plan_chunks(int64_t numel, int32_t elem_bytes, int64_t chunk_bytes,
                         int32_t align_bytes, int64_t *off_out, int64_t cap,
                         int64_t *count_out) {
    const char *op = "gq_plan_chunks";
    if (!count_out) return fail(GQ_ERR_INVALID, op, "count_out is NULL");
    if (numel < 1) return fail(GQ_ERR_INVALID, op, "numel = %lld < 1", (long long)numel);
    if (elem_bytes < 1 || chunk_bytes < 1 || align_bytes < 1)
        return fail(GQ_ERR_INVALID, op, "elem_bytes, chunk_bytes and align_bytes must be >= 1");
    const int64_t divisor = chunk_bytes - chunk_bytes % align_bytes;
    if (divisor < 1)
        return fail(GQ_ERR_INVALID, op, "chunk_bytes %lld rounds down to 0 at alignment %d",
                    (long long)chunk_bytes, align_bytes);
    if (numel > (INT64_MAX / 8) / elem_bytes)
        return fail(GQ_ERR_INVALID, op, "numel * elem_bytes overflows");
    int64_t k = numel * elem_bytes / divisor;
    if (k < 1) k = 1;
    const int64_t piece = (numel + k - 1) / k;      // torch.chunk split size
    const int64_t count = (numel + piece - 1) / piece;
    *count_out = count;
    if (cap < count + 1 || !off_out)
        return fail(GQ_ERR_CAPACITY, op, "need %lld offsets, capacity %lld",
                    (long long)(count + 1), (long long)cap);
    for (int64_t j = 0; j < count; ++j) off_out[j] = j * piece;
    off_out[count] = numel;
    return ok();
}

gq_status gq_units_create(const int64_t *h_off, int64_t n_units, gq_units **out) {
    const char *op = "gq_units_create";
    if (!out) return fail(GQ_ERR_INVALID, op, "out is NULL");
    *out = nullptr;
    if (!h_off) return fail(GQ_ERR_INVALID, op, "h_off is NULL");
    if (n_units < 1 || n_units >= GQ_MAX_TILES)
        return fail(GQ_ERR_INVALID, op, "n_units = %lld outside [1, %d]", (long long)n_units,
                    GQ_MAX_TILES - 1);
    if (h_off[0] < 0) return fail(GQ_ERR_INVALID, op, "h_off[0] = %lld < 0", (long long)h_off[0]);
    for (int64_t u = 0; u < n_units; ++u)
        if (h_off[u + 1] <= h_off[u])
            return fail(GQ_ERR_INVALID, op, "h_off not strictly increasing at unit %lld",
                        (long long)u);
    const int64_t n = h_off[n_units];
    if (n > (int64_t(1) << 40)) return fail(GQ_ERR_INVALID, op, "n = %lld above 2^40", (long long)n);

    gq_units *U = new (std::nothrow) gq_units;
    if (!U) return fail(GQ_ERR_INVALID, op, "out of host memory");
    if (hipGetDevice(&U->device) != hipSuccess) {
        delete U;
        return fail(GQ_ERR_HIP, op, "hipGetDevice failed");
    }
    U->n = n;
    U->n_units = n_units;
    std::vector<int64_t> off(h_off, h_off + n_units + 1);
    hipError_t e = hipMalloc(reinterpret_cast<void **>(&U->d_faults), sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(U->d_faults, 0, sizeof(uint32_t));
    for (int ti = 0; ti < gq::TAB_COUNT && e == hipSuccess; ++ti) {
        const int V = gq::kSlotElems[ti];
        gq::Table &t = U->tab[ti];
        int64_t small_cap =
            64 * static_cast<int64_t>(ti == gq::TAB_R ? gq::SMALL_SLOTS_R : gq::SMALL_SLOTS_Q);
        auto span = [&](int64_t u) { return (off[u + 1] + V - 1) / V - off[u] / V; };
        if (ti == gq::TAB_R) {
            // wide tiles when most elements of the non-small units sit in
            // units wider than a narrow tile; chunk-wide ones when most sit
            // in units that fill one chunk-wide tile but not one wide tile
            const int64_t narrow = static_cast<int64_t>(gq::R_BLOCK) * gq::R_SLOTS_NARROW;
            const int64_t wide = static_cast<int64_t>(gq::R_BLOCK) * gq::R_SLOTS_WIDE;
            const int64_t chunk = static_cast<int64_t>(gq::R_BLOCK_CHUNK) * gq::R_SLOTS_WIDE;
            int64_t in_wide = 0, in_chunk = 0, in_big = 0;
            for (int64_t u = 0; u < n_units; ++u) {
                if (span(u) <= small_cap) continue;
                in_big += off[u + 1] - off[u];
                if (span(u) > narrow) in_wide += off[u + 1] - off[u];
                if (span(u) > wide && span(u) <= chunk) in_chunk += off[u + 1] - off[u];
            }
            t.sched = gq::SCHED_LAYER;
            t.block = (2 * in_chunk >= in_big && in_big > 0) ? gq::R_BLOCK_CHUNK : gq::R_BLOCK;
            t.slots = (2 * in_wide >= in_big) ? gq::R_SLOTS_WIDE : gq::R_SLOTS_NARROW;
            // the narrow kernel's waves also take units of up to twice their
            // slots, in two halves
            if (t.slots == gq::R_SLOTS_NARROW) small_cap *= 2;
        } else {
            // chunk schedule when most elements of the non-small units sit
            // in units that fill one chunk tile but not one layer tile (a
            // shorter unit would leave most of a chunk tile's lanes idle),
            // or when small units hold most elements (their per-wave phase
            // runs faster in the chunk kernel); the layer schedule otherwise
            const int64_t cap = static_cast<int64_t>(gq::Q_BLOCK_CHUNK) * gq::Q_SLOTS_CHUNK;
            const int64_t layer_cap = static_cast<int64_t>(gq::Q_BLOCK_LAYER) * gq::Q_SLOTS_LAYER;
            int64_t in_chunk = 0, in_big = 0;
            for (int64_t u = 0; u < n_units; ++u) {
                if (span(u) <= small_cap) continue;
                in_big += off[u + 1] - off[u];
                if (span(u) > layer_cap && span(u) <= cap) in_chunk += off[u + 1] - off[u];
            }
            const bool mostly_small = 2 * in_big < off[n_units] - off[0];
            t.sched = (mostly_small || 2 * in_chunk >= in_big) ? gq::SCHED_CHUNK : gq::SCHED_LAYER;
            t.block = t.sched == gq::SCHED_CHUNK ? gq::Q_BLOCK_CHUNK : gq::Q_BLOCK_LAYER;
            t.slots = t.sched == gq::SCHED_CHUNK ? gq::Q_SLOTS_CHUNK : gq::Q_SLOTS_LAYER;
            if (t.sched == gq::SCHED_CHUNK) {
                // 8-row chunk tiles where that adds no tile to any unit
                const int64_t short_cap =
                    static_cast<int64_t>(gq::Q_BLOCK_CHUNK) * gq::Q_SLOTS_CHUNK_SHORT;
                bool same = true;
                for (int64_t u = 0; u < n_units && same; ++u)
                    if (span(u) > small_cap)
                        same = (span(u) + short_cap - 1) / short_cap == (span(u) + cap - 1) / cap;
                if (same) t.slots = gq::Q_SLOTS_CHUNK_SHORT;
            }
        }
        std::vector<gq::Tile> tiles;
        std::vector<int32_t> multi, unit_first;
        build_tiles(off, V, static_cast<int64_t>(t.block) * t.slots, tiles, multi, unit_first,
                    t.n_multi_units, t.max_count);
        if (static_cast<int64_t>(tiles.size()) >= GQ_MAX_TILES) {
            (void)gq_units_destroy(U);
            return fail(GQ_ERR_INVALID, op, "table of %lld work tiles (limit %d): too many units "
                        "or elements", (long long)tiles.size(), GQ_MAX_TILES - 1);
        }
        // hot-path split: small units, and the tiles of the others
        std::vector<gq::Tile> small, big;
        int32_t big_max = 1;
        for (int64_t u = 0; u < n_units; ++u) {
            if (span(u) <= small_cap) {
                small.push_back({off[u], off[u + 1], static_cast<int32_t>(u),
                                 static_cast<int32_t>(small.size()), 1, -1});
                continue;
            }
            const int32_t first_big = static_cast<int32_t>(big.size());
            for (int32_t k = unit_first[u]; k < unit_first[u + 1]; ++k) {
                gq::Tile tl = tiles[k];
                tl.first = first_big;
                big.push_back(tl);
            }
            big_max = std::max(big_max, unit_first[u + 1] - unit_first[u]);
        }
        t.n_tiles = static_cast<int64_t>(tiles.size());
        t.n_multi = static_cast<int64_t>(multi.size());
        t.n_small = static_cast<int64_t>(small.size());
        t.n_big = static_cast<int64_t>(big.size());
        t.big_max_count = big_max;
        {
            int64_t in_small = 0;
            for (const gq::Tile &x : small) in_small += x.end - x.begin;
            t.small_dominant = 2 * in_small > off[n_units] - off[0];
        }
        if (gq::short_table(t)) {
            std::vector<gq::Tile> work, pack_units, rest;
            std::vector<gq::Pack> packs;
            if (ti == gq::TAB_R)
                build_pieces(off, V, tiles, unit_first, work, packs, pack_units, rest);
            else
                build_short_units(off, V, 64 * gq::SHORT_SLOTS_Q, tiles, unit_first, packs, work,
                                  rest);
            t.n_short = static_cast<int64_t>(work.size());
            t.n_packs = static_cast<int64_t>(packs.size());
            t.n_pack_units = static_cast<int64_t>(pack_units.size());
            t.n_rest = static_cast<int64_t>(rest.size());
            e = upload(&t.d_short, work);
            if (e == hipSuccess) e = upload(&t.d_packs, packs);
            if (e == hipSuccess) e = upload(&t.d_pack_units, pack_units);
            if (e == hipSuccess) e = upload(&t.d_rest, rest);
        }
        if (e == hipSuccess) e = upload(&t.d_tiles, tiles);
        if (e == hipSuccess) e = upload(&t.d_multi, multi);
        if (e == hipSuccess) e = upload(&t.d_unit_first, unit_first);
        if (e == hipSuccess) e = upload(&t.d_small, small);
        if (e == hipSuccess) e = upload(&t.d_big, big);
        const size_t partial_bytes = sizeof(uint32_t) * GQ_MAX_RANKS * static_cast<size_t>(t.n_tiles);
        if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&t.d_partial), partial_bytes);
        if (e == hipSuccess) e = hipMemset(t.d_partial, 0, partial_bytes);
        if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&t.d_ctl), 4 * sizeof(uint32_t));
        if (e == hipSuccess) e = hipMemset(t.d_ctl, 0, 4 * sizeof(uint32_t));
        if (e == hipSuccess && t.n_multi_units > 0) {
            const size_t pub_bytes = sizeof(uint64_t) * GQ_MAX_RANKS * static_cast<size_t>(t.n_big);
            const size_t unit_bytes =
                sizeof(uint64_t) * GQ_MAX_RANKS * static_cast<size_t>(t.n_multi_units);
            e = hipMalloc(reinterpret_cast<void **>(&t.d_pub), pub_bytes);
            if (e == hipSuccess) e = hipMemset(t.d_pub, 0, pub_bytes);
            if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&t.d_res), unit_bytes);
            if (e == hipSuccess) e = hipMemset(t.d_res, 0, unit_bytes);
            if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&t.d_cnt), unit_bytes);
            if (e == hipSuccess) e = hipMemset(t.d_cnt, 0, unit_bytes);
        }
    }
    if (e != hipSuccess) {
        (void)gq_units_destroy(U);
        return fail(GQ_ERR_HIP, op, "device allocation failed: %s", hipGetErrorString(e));
    }
    for (int ti = 0; ti < gq::TAB_COUNT; ++ti) {
        if (!gq::table_ready(U->tab[ti], n_units)) {
            (void)gq_units_destroy(U);
            return fail(GQ_ERR_HIP, op, "internal error: work table %d incomplete", ti);
        }
    }
    if (hipDeviceSynchronize() != hipSuccess) {
        (void)gq_units_destroy(U);
        return fail(GQ_ERR_HIP, op, "synchronize failed");
    }
    *out = U;
    return ok();
}

gq_status gq_units_destroy(gq_units *u) {
    if (!u) return ok();
    for (int k = 0; k < gq::TAB_COUNT; ++k) free_table(u->tab[k]);
    if (u->d_faults) (void)hipFree(u->d_faults);
    delete u;
    return ok();
}

gq_status gq_units_schedule(const gq_units *u, gq_dtype dt, int32_t *sched) {
    const char *op = "gq_units_schedule";
    if (!u) return fail(GQ_ERR_INVALID, op, "unit table is NULL");
    if (!sched) return fail(GQ_ERR_INVALID, op, "sched is NULL");
    if (dt != GQ_F32 && dt != GQ_F16) return fail(GQ_ERR_INVALID, op, "unknown dtype %d", (int)dt);
    *sched = u->tab[q_table(dt)].sched;
    return ok();
}

gq_status gq_units_quantize_tile(const gq_units *u, gq_dtype dt, int64_t *elems) {
    const char *op = "gq_units_quantize_tile";
    if (!u) return fail(GQ_ERR_INVALID, op, "unit table is NULL");
    if (!elems) return fail(GQ_ERR_INVALID, op, "elems is NULL");
    if (dt != GQ_F32 && dt != GQ_F16) return fail(GQ_ERR_INVALID, op, "unknown dtype %d", (int)dt);
    const gq::Table &t = u->tab[q_table(dt)];
    *elems = static_cast<int64_t>(t.block) * t.slots * gq::kSlotElems[q_table(dt)];
    return ok();
}

gq_status gq_units_reduce_tile(const gq_units *u, int64_t *elems) {
    const char *op = "gq_units_reduce_tile";
    if (!u) return fail(GQ_ERR_INVALID, op, "unit table is NULL");
    if (!elems) return fail(GQ_ERR_INVALID, op, "elems is NULL");
    const gq::Table &t = u->tab[gq::TAB_R];
    *elems = static_cast<int64_t>(t.block) * t.slots * gq::kSlotElems[gq::TAB_R];
    return ok();
}

gq_status gq_units_faults(const gq_units *u, uint64_t *count) {
    const char *op = "gq_units_faults";
    if (!count) return fail(GQ_ERR_INVALID, op, "count is NULL");
    GQ_TRY(check_units(op, u));
    uint32_t v = 0;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&v, u->d_faults, sizeof v, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(GQ_ERR_HIP, op, "reading the fault counter failed");
    *count = v;
    return ok();
}

// Writes the fault count (after the device is idle).
static gq_status set_faults(const char *op, gq_units *u, bool force) {
    GQ_TRY(check_units(op, u));
    uint32_t v = 0;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&v, u->d_faults, sizeof v, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(GQ_ERR_HIP, op, "reading the fault counter failed");
    v = force ? (v == 0 ? 1u : v) : 0u;
    if (hipMemcpy(u->d_faults, &v, sizeof v, hipMemcpyHostToDevice) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
        return fail(GQ_ERR_HIP, op, "writing the fault counter failed");
    return ok();
}

gq_status gq_units_faults_async(const gq_units *u, uint32_t *count_out, gq_stream stream) {
    const char *op = "gq_units_faults_async";
    GQ_TRY(check_ptr(op, "count_out", count_out, 4));
    GQ_TRY(check_units(op, u));
    return launch_status(op, gq::launch_copy_word(u->d_faults, count_out,
                                                  static_cast<hipStream_t>(stream)));
}

gq_status gq_units_launch_plan(const gq_units *u, gq_dtype dt, float in_mul, int64_t *q_groups,
                               int32_t *q_form, int64_t *r_groups, int32_t *r_form) {
    const char *op = "gq_units_launch_plan";
    if (dt != GQ_F32 && dt != GQ_F16) return fail(GQ_ERR_INVALID, op, "unknown dtype %d", (int)dt);
    if (!std::isfinite(in_mul) || !(in_mul > 0.0f))
        return fail(GQ_ERR_INVALID, op, "in_mul = %g must be finite and > 0", (double)in_mul);
    GQ_TRY(check_units(op, u));
    const gq::Table &tq = u->tab[q_table(dt)];
    const gq::Table &tr = u->tab[gq::TAB_R];
    const int64_t qg = gq::quantize_resident(dt, in_mul != 1.0f, tq);
    const int64_t rg = gq::reduce_resident(tr);
    if (qg < 1 || rg < 1) return fail(GQ_ERR_HIP, op, "occupancy query failed");
    auto form = [](const gq::Table &t, int64_t groups) {
        if (gq::short_table(t)) return GQ_FORM_SHORT_UNITS;
        return groups >= t.big_max_count ? GQ_FORM_PERSISTENT : GQ_FORM_TWO_PASS;
    };
    if (q_groups) *q_groups = qg;
    if (q_form) *q_form = form(tq, qg);
    if (r_groups) *r_groups = rg;
    if (r_form) *r_form = form(tr, rg);
    return ok();
}

gq_status gq_units_clear_faults(gq_units *u) { return set_faults("gq_units_clear_faults", u, false); }

gq_status gq_units_force_timeout(gq_units *u) { return set_faults("gq_units_force_timeout", u, true); }

gq_status gq_units_info(const gq_units *u, int64_t *n, int64_t *n_units) {
    if (!u) return fail(GQ_ERR_INVALID, "gq_units_info", "unit table is NULL");
    if (n) *n = u->n;
    if (n_units) *n_units = u->n_units;
    return ok();
}

static gq_status fill_qargs(const char *op, const void *const *x, int32_t W, gq_dtype dt,
                            float in_mul, gq::QArgs &a) {
    GQ_TRY(check_ranks(op, W));
    if (dt != GQ_F32 && dt != GQ_F16) return fail(GQ_ERR_INVALID, op, "unknown dtype %d", (int)dt);
    if (!std::isfinite(in_mul) || !(in_mul > 0.0f))
        return fail(GQ_ERR_INVALID, op, "in_mul = %g must be finite and > 0", (double)in_mul);
    GQ_TRY(check_ptr_array(op, "x", x, W, 16));
    std::memset(&a, 0, sizeof a);
    for (int32_t w = 0; w < W; ++w) a.x[w] = x[w];
    a.W = W;
    a.in_mul = in_mul;
    return GQ_OK;
}

// Unit-table check (last, after every pointer check) and the table fields.
static gq_status bind_qtable(const char *op, const gq_units *u, gq_dtype dt, gq::QArgs &a) {
    GQ_TRY(check_units(op, u));
    a.n_units = u->n_units;
    a.n = u->n;
    const gq::Table &t = u->tab[q_table(dt)];
    a.tiles = t.d_tiles;
    a.n_tiles = t.n_tiles;
    a.faults = u->d_faults;
    return GQ_OK;
}

gq_status gq_absmax(const void *const *x, int32_t W, gq_dtype dt, float in_mul,
                    const gq_units *u, uint32_t *amax_bits, gq_stream stream) {
    const char *op = "gq_absmax";
    gq::QArgs a;
    GQ_TRY(fill_qargs(op, x, W, dt, in_mul, a));
    GQ_TRY(check_ptr(op, "amax_bits", amax_bits, 4));
    GQ_TRY(bind_qtable(op, u, dt, a));
    a.amax_out = amax_bits;
    const gq::Table &t = u->tab[q_table(dt)];
    return launch_status(op, gq::launch_absmax(a, dt, t, static_cast<hipStream_t>(stream)));
}

gq_status gq_quantize(const void *const *x, int32_t W, gq_dtype dt, float in_mul,
                      const gq_units *u, const uint32_t *amax_bits, float *const *scale_out,
                      int8_t *const *q_out, gq_stream stream) {
    const char *op = "gq_quantize";
    gq::QArgs a;
    GQ_TRY(fill_qargs(op, x, W, dt, in_mul, a));
    if (amax_bits) GQ_TRY(check_ptr(op, "amax_bits", amax_bits, 4));
    GQ_TRY(check_ptr_array(op, "scale_out", scale_out, W, 4));
    GQ_TRY(check_ptr_array(op, "q_out", q_out, W, 16));
    GQ_TRY(bind_qtable(op, u, dt, a));
    for (int32_t w = 0; w < W; ++w) {
        a.scale[w] = scale_out[w];
        a.q[w] = q_out[w];
    }
    a.amax = amax_bits;
    const gq::Table &t = u->tab[q_table(dt)];
    return launch_status(op, gq::launch_quantize(a, dt, t, static_cast<hipStream_t>(stream)));
}

gq_status gq_quantize_noalloc(const void *const *x, int32_t W, gq_dtype dt, float in_mul,
                              const int64_t *h_off, const int64_t *d_off, int64_t n_units,
                              float *const *scale_out, int8_t *const *q_out, gq_stream stream) {
    const char *op = "gq_quantize_noalloc";
    gq::QArgs a;
    GQ_TRY(fill_qargs(op, x, W, dt, in_mul, a));
    GQ_TRY(check_ptr_array(op, "scale_out", scale_out, W, 4));
    GQ_TRY(check_ptr_array(op, "q_out", q_out, W, 16));
    GQ_TRY(check_ptr(op, "d_off", d_off, 8));
    if (!h_off) return fail(GQ_ERR_INVALID, op, "h_off is NULL");
    if (n_units < 1) return fail(GQ_ERR_INVALID, op, "n_units = %lld < 1", (long long)n_units);
    if (n_units > GQ_NOALLOC_MAX_MAXIMA / W)
        return fail(GQ_ERR_INVALID, op, "W * n_units = %d * %lld maxima, above the limit of %d",
                    W, (long long)n_units, GQ_NOALLOC_MAX_MAXIMA);
    if (h_off[0] < 0) return fail(GQ_ERR_INVALID, op, "h_off[0] = %lld < 0", (long long)h_off[0]);
    for (int64_t u = 0; u < n_units; ++u)
        if (h_off[u + 1] <= h_off[u])
            return fail(GQ_ERR_INVALID, op, "h_off not strictly increasing at unit %lld",
                        (long long)u);
    if (h_off[n_units] > (int64_t(1) << 40))
        return fail(GQ_ERR_INVALID, op, "n = %lld above 2^40", (long long)h_off[n_units]);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GQ_ERR_HIP, op, "hipGetDevice failed");
    void *sp = gq::noalloc_scratch(dev);
    if (!sp) return fail(GQ_ERR_HIP, op, "looking up the maxima array on device %d failed", dev);
    gq::NoallocArgs c;
    c.x = x;
    c.scale = scale_out;
    c.q = q_out;
    c.d_off = d_off;
    c.n_units = n_units;
    c.n = h_off[n_units];
    c.first = h_off[0];
    c.in_mul = in_mul;
    c.dt = dt;
    c.W = W;
    return launch_status(op, gq::launch_quantize_noalloc(c, sp, static_cast<hipStream_t>(stream)));
}

static gq_status fill_rargs(const char *op, const int8_t *const *q, const float *const *scale,
                            int32_t W, gq::RArgs &a) {
    GQ_TRY(check_ranks(op, W));
    GQ_TRY(check_ptr_array(op, "q", q, W, 16));
    GQ_TRY(check_ptr_array(op, "scale", scale, W, 4));
    std::memset(&a, 0, sizeof a);
    for (int32_t w = 0; w < W; ++w) {
        a.q[w] = q[w];
        a.scale[w] = scale[w];
    }
    a.W = W;
    return GQ_OK;
}

gq_status gq_reduce_dequant(const int8_t *const *q, const float *const *scale, int32_t W,
                            const gq_units *u, float *r_out, gq_stream stream) {
    const char *op = "gq_reduce_dequant";
    gq::RArgs a;
    GQ_TRY(fill_rargs(op, q, scale, W, a));
    GQ_TRY(check_ptr(op, "r_out", r_out, 16));
    GQ_TRY(check_units(op, u));
    a.r = r_out;
    a.faults = u->d_faults;
    a.n = u->n;
    return launch_status(op, gq::launch_reduce(a, u->tab[gq::TAB_R], false, false,
                                               static_cast<hipStream_t>(stream)));
}

gq_status gq_requantize(const float *r, const gq_units *u, float *scale_out, int8_t *q_out,
                        gq_stream stream) {
    const char *op = "gq_requantize";
    const void *x[1] = {r};
    gq::QArgs a;
    GQ_TRY(fill_qargs(op, x, 1, GQ_F32, 1.0f, a));
    GQ_TRY(check_ptr(op, "scale_out", scale_out, 4));
    GQ_TRY(check_ptr(op, "q_out", q_out, 16));
    GQ_TRY(bind_qtable(op, u, GQ_F32, a));
    a.scale[0] = scale_out;
    a.q[0] = q_out;
    a.amax = nullptr;
    return launch_status(op, gq::launch_quantize(a, GQ_F32, u->tab[gq::TAB_Q32],
                                                 static_cast<hipStream_t>(stream)));
}

gq_status gq_reduce_requantize(const int8_t *const *q, const float *const *scale, int32_t W,
                               const gq_units *u, float *r_out, float *scale_out, int8_t *q_out,
                               gq_stream stream) {
    const char *op = "gq_reduce_requantize";
    gq::RArgs a;
    GQ_TRY(fill_rargs(op, q, scale, W, a));
    if (r_out) GQ_TRY(check_ptr(op, "r_out", r_out, 16));
    GQ_TRY(check_ptr(op, "scale_out", scale_out, 4));
    GQ_TRY(check_ptr(op, "q_out", q_out, 16));
    GQ_TRY(check_units(op, u));
    a.r = r_out;
    a.faults = u->d_faults;
    a.n = u->n;
    a.scale_out = scale_out;
    a.q_out = q_out;
    return launch_status(op, gq::launch_reduce(a, u->tab[gq::TAB_R], true, false,
                                               static_cast<hipStream_t>(stream)));
}

gq_status gq_pipe_destroy(gq_pipe *p) {
    if (!p) return ok();
    for (gq_units *u : p->tab) (void)gq_units_destroy(u);
    for (int k = 0; k < 2; ++k) {
        if (p->ev_q[k]) (void)hipEventDestroy(p->ev_q[k]);
        if (p->ev_r[k]) (void)hipEventDestroy(p->ev_r[k]);
    }
    if (p->ev_done) (void)hipEventDestroy(p->ev_done);
    if (p->aux) (void)hipStreamDestroy(p->aux);
    delete p;
    return ok();
}

gq_status gq_pipe_create(const int64_t *h_off, int64_t n_units, const int64_t *bucket_units,
                         int64_t n_buckets, int32_t mode, gq_pipe **out) {
    const char *op = "gq_pipe_create";
    if (!out) return fail(GQ_ERR_INVALID, op, "out is NULL");
    *out = nullptr;
    if (mode != GQ_PIPE_OVERLAP && mode != GQ_PIPE_SERIAL)
        return fail(GQ_ERR_INVALID, op, "unknown mode %d", mode);
    if (!h_off || !bucket_units) return fail(GQ_ERR_INVALID, op, "h_off or bucket_units is NULL");
    if (n_units < 1 || n_units >= GQ_MAX_TILES)
        return fail(GQ_ERR_INVALID, op, "n_units = %lld outside [1, %d]", (long long)n_units,
                    GQ_MAX_TILES - 1);
    if (h_off[0] != 0) return fail(GQ_ERR_INVALID, op, "h_off[0] = %lld, must be 0", (long long)h_off[0]);
    for (int64_t u = 0; u < n_units; ++u)
        if (h_off[u + 1] <= h_off[u])
            return fail(GQ_ERR_INVALID, op, "h_off not strictly increasing at unit %lld", (long long)u);
    if (h_off[n_units] > (int64_t(1) << 40))
        return fail(GQ_ERR_INVALID, op, "n = %lld above 2^40", (long long)h_off[n_units]);
    if (n_buckets < 1 || n_buckets > n_units)
        return fail(GQ_ERR_INVALID, op, "n_buckets = %lld outside [1, n_units]", (long long)n_buckets);
    if (bucket_units[0] != 0 || bucket_units[n_buckets] != n_units)
        return fail(GQ_ERR_INVALID, op, "bucket_units must run from 0 to n_units");
    for (int64_t b = 0; b < n_buckets; ++b)
        if (bucket_units[b + 1] <= bucket_units[b])
            return fail(GQ_ERR_INVALID, op, "bucket_units not strictly increasing at bucket %lld",
                        (long long)b);
    gq_pipe *P = new (std::nothrow) gq_pipe;
    if (!P) return fail(GQ_ERR_INVALID, op, "out of host memory");
    if (hipGetDevice(&P->device) != hipSuccess) {
        delete P;
        return fail(GQ_ERR_HIP, op, "hipGetDevice failed");
    }
    P->n = h_off[n_units];
    P->n_units = n_units;
    P->n_buckets = n_buckets;
    P->mode = mode;
    for (int64_t b = 0; b < n_buckets; ++b) {
        const int64_t ua = bucket_units[b], ub = bucket_units[b + 1];
        const int64_t base = h_off[ua] & ~int64_t{15};
        std::vector<int64_t> local(static_cast<size_t>(ub - ua + 1));
        for (int64_t u = ua; u <= ub; ++u) local[static_cast<size_t>(u - ua)] = h_off[u] - base;
        gq_units *t = nullptr;
        const gq_status st = gq_units_create(local.data(), ub - ua, &t);
        if (st != GQ_OK) {
            (void)gq_pipe_destroy(P);
            return st;  // gq_units_create set the error text
        }
        P->tab.push_back(t);
        P->base.push_back(base);
        P->u0.push_back(ua);
        P->slot_elems = std::max(P->slot_elems, h_off[ub] - base);
        P->slot_units = std::max(P->slot_units, ub - ua);
    }
    hipError_t e = hipStreamCreateWithFlags(&P->aux, hipStreamNonBlocking);
    for (int k = 0; k < 2 && e == hipSuccess; ++k) {
        e = hipEventCreateWithFlags(&P->ev_q[k], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&P->ev_r[k], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&P->ev_done, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)gq_pipe_destroy(P);
        return fail(GQ_ERR_HIP, op, "stream or event creation failed: %s", hipGetErrorString(e));
    }
    *out = P;
    return ok();
}

gq_status gq_pipe_slots(const gq_pipe *p, int64_t *slot_elems, int64_t *slot_units) {
    if (!p) return fail(GQ_ERR_INVALID, "gq_pipe_slots", "plan is NULL");
    if (slot_elems) *slot_elems = p->slot_elems;
    if (slot_units) *slot_units = p->slot_units;
    return ok();
}

gq_status gq_pipe_faults(const gq_pipe *p, uint64_t *count) {
    const char *op = "gq_pipe_faults";
    if (!p) return fail(GQ_ERR_INVALID, op, "plan is NULL");
    if (!count) return fail(GQ_ERR_INVALID, op, "count is NULL");
    uint64_t total = 0;
    for (gq_units *u : p->tab) {
        uint64_t c = 0;
        GQ_TRY(gq_units_faults(u, &c));
        total += c;
    }
    *count = total;
    return ok();
}

gq_status gq_pipe_clear_faults(gq_pipe *p) {
    const char *op = "gq_pipe_clear_faults";
    if (!p) return fail(GQ_ERR_INVALID, op, "plan is NULL");
    for (gq_units *u : p->tab) GQ_TRY(gq_units_clear_faults(u));
    return ok();
}

// Overlap schedules of gq_pipe_step.  Kernels of two buckets run side by
// side, so their forms must not strand each other's work groups:
//  ALTERNATE  buckets alternate between the two streams, each bucket's
//             reduce right after its quantize on the same stream (code slot
//             b % 2 is then always used by one stream, and no event orders
//             the streams inside the step).  Any kernel of one stream may
//             run beside any kernel of the other, so every kernel that waits
//             on its own work groups gets a grid of at most the compute unit
//             count; this needs each such kernel to fit at least two work
//             groups per compute unit (one of each of two such kernels then
//             fits in any compute unit that holds fewer than two, and
//             together they never exceed what the device holds at once).  A
//             kernel that never waits always finishes and frees its compute
//             units.
//  EVENTS     otherwise: quantize on the caller's stream, reduce on the
//             second stream after an event, so that only bucket b's reduce
//             and bucket b+1's quantize meet; per such pair, both run in
//             their full forms if one of them never waits, and else the
//             reduce takes its form that never waits.
static bool pipe_alternates(const gq_pipe *p, gq_dtype dt, bool mul, int64_t cus) {
    for (size_t b = 0; b < p->tab.size(); ++b) {
        const gq::Table &q = p->tab[b]->tab[q_table(dt)];
        const gq::Table &r = p->tab[b]->tab[gq::TAB_R];
        if (gq::quantize_waits(dt, mul, q, 0) && gq::quantize_resident(dt, mul, q) < 2 * cus)
            return false;
        if (gq::reduce_waits(r, 0) && gq::reduce_resident(r) < 2 * cus) return false;
    }
    return true;
}

gq_status gq_pipe_schedule(const gq_pipe *p, gq_dtype dt, float in_mul, int32_t *schedule) {
    const char *op = "gq_pipe_schedule";
    if (!p) return fail(GQ_ERR_INVALID, op, "plan is NULL");
    if (!schedule) return fail(GQ_ERR_INVALID, op, "schedule is NULL");
    if (dt != GQ_F32 && dt != GQ_F16) return fail(GQ_ERR_INVALID, op, "unknown dtype %d", (int)dt);
    if (!std::isfinite(in_mul) || !(in_mul > 0.0f))
        return fail(GQ_ERR_INVALID, op, "in_mul = %g must be finite and > 0", (double)in_mul);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GQ_ERR_HIP, op, "hipGetDevice failed");
    if (dev != p->device)
        return fail(GQ_ERR_DEVICE, op, "current device %d, plan lives on device %d", dev, p->device);
    if (p->mode == GQ_PIPE_SERIAL) {
        *schedule = GQ_PIPE_SCHED_SERIAL;
        return ok();
    }
    const int64_t cus = gq::device_cus();
    if (cus < 1) return fail(GQ_ERR_HIP, op, "device query failed");
    *schedule = pipe_alternates(p, dt, in_mul != 1.0f, cus) ? GQ_PIPE_SCHED_ALTERNATE
                                                            : GQ_PIPE_SCHED_EVENTS;
    return ok();
}

gq_status gq_pipe_step(gq_pipe *p, const void *const *x, int32_t W, gq_dtype dt, float in_mul,
                       int8_t *const *q_slot, float *const *scale_slot, float *scale_out,
                       int8_t *q_out, gq_stream stream) {
    const char *op = "gq_pipe_step";
    gq::QArgs qa;
    GQ_TRY(fill_qargs(op, x, W, dt, in_mul, qa));
    GQ_TRY(check_ptr_array(op, "q_slot", q_slot, 2 * W, 16));
    GQ_TRY(check_ptr_array(op, "scale_slot", scale_slot, 2 * W, 4));
    GQ_TRY(check_ptr(op, "scale_out", scale_out, 4));
    GQ_TRY(check_ptr(op, "q_out", q_out, 16));
    if (!p) return fail(GQ_ERR_INVALID, op, "plan is NULL");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GQ_ERR_HIP, op, "hipGetDevice failed");
    if (dev != p->device)
        return fail(GQ_ERR_DEVICE, op, "current device %d, plan lives on device %d", dev, p->device);
    const hipStream_t s_main = static_cast<hipStream_t>(stream);
    const bool serial = p->mode == GQ_PIPE_SERIAL;
    const int64_t esz = dt == GQ_F32 ? 4 : 2;
    const bool mul = in_mul != 1.0f;
    const int64_t B = p->n_buckets;
    auto tq = [&](int64_t b) -> const gq::Table & {
        return p->tab[static_cast<size_t>(b)]->tab[q_table(dt)];
    };
    auto tr = [&](int64_t b) -> const gq::Table & {
        return p->tab[static_cast<size_t>(b)]->tab[gq::TAB_R];
    };
    const int64_t cus = serial ? 0 : gq::device_cus();
    if (!serial && cus < 1) return fail(GQ_ERR_HIP, op, "device query failed");
    const bool alternate = !serial && pipe_alternates(p, dt, mul, cus);
    hipError_t e = hipSuccess;
    if (alternate) {
        // the second stream starts after the caller's stream's earlier work
        e = hipEventRecord(p->ev_q[0], s_main);
        if (e == hipSuccess) e = hipStreamWaitEvent(p->aux, p->ev_q[0], 0);
        if (e != hipSuccess) return launch_status(op, e);
    }
    for (int64_t b = 0; b < B; ++b) {
        const int s = static_cast<int>(b & 1);
        const gq_units *t = p->tab[static_cast<size_t>(b)];
        const int64_t base = p->base[static_cast<size_t>(b)];
        const hipStream_t s_q = (alternate && s == 1) ? p->aux : s_main;
        const hipStream_t s_r = serial ? s_main : alternate ? s_q : p->aux;
        int64_t q_cap = 0, r_cap = 0;
        bool r_wait_free = false;
        if (alternate) {
            q_cap = gq::quantize_waits(dt, mul, tq(b), 0) ? cus : 0;
            r_cap = gq::reduce_waits(tr(b), 0) ? cus : 0;
        } else if (!serial && b + 1 < B) {
            // EVENTS: this reduce meets the next bucket's quantize
            r_wait_free = gq::quantize_waits(dt, mul, tq(b + 1), 0) && gq::reduce_waits(tr(b), 0);
        }
        // quantize bucket b into slot s (EVENTS: once the reduce of bucket
        // b-2 has released it)
        if (!serial && !alternate && b >= 2 && hipStreamWaitEvent(s_main, p->ev_r[s], 0) != hipSuccess)
            return fail(GQ_ERR_HIP, op, "hipStreamWaitEvent failed");
        gq::QArgs a = qa;
        for (int32_t w = 0; w < W; ++w) {
            a.x[w] = static_cast<const uint8_t *>(x[w]) + base * esz;
            a.scale[w] = scale_slot[s * W + w];
            a.q[w] = q_slot[s * W + w];
        }
        a.amax = nullptr;
        GQ_TRY(bind_qtable(op, t, dt, a));
        e = gq::launch_quantize(a, dt, t->tab[q_table(dt)], s_q, q_cap);
        if (!serial && !alternate) {
            if (e == hipSuccess) e = hipEventRecord(p->ev_q[s], s_main);
            if (e == hipSuccess) e = hipStreamWaitEvent(p->aux, p->ev_q[s], 0);
        }
        if (e != hipSuccess) return launch_status(op, e);
        // reduce + requantize bucket b
        gq::RArgs r;
        GQ_TRY(fill_rargs(op, q_slot + s * W, scale_slot + s * W, W, r));
        r.r = nullptr;
        r.faults = t->d_faults;
        r.n = t->n;
        r.scale_out = scale_out + p->u0[static_cast<size_t>(b)];
        r.q_out = q_out + base;
        e = gq::launch_reduce(r, t->tab[gq::TAB_R], true, r_wait_free, s_r, r_cap);
        if (!serial && !alternate && e == hipSuccess) e = hipEventRecord(p->ev_r[s], p->aux);
        if (e != hipSuccess) return launch_status(op, e);
    }
    if (serial) return ok();
    e = hipEventRecord(p->ev_done, p->aux);
    if (e == hipSuccess) e = hipStreamWaitEvent(s_main, p->ev_done, 0);
    return launch_status(op, e);
}

gq_status gq_sum_f32(const void *const *x, int32_t W, gq_dtype dt, float in_mul, int64_t n,
                     int32_t mean, float *r_out, gq_stream stream) {
    const char *op = "gq_sum_f32";
    GQ_TRY(check_ranks(op, W));
    if (dt != GQ_F32 && dt != GQ_F16) return fail(GQ_ERR_INVALID, op, "unknown dtype %d", (int)dt);
    if (!std::isfinite(in_mul) || !(in_mul > 0.0f))
        return fail(GQ_ERR_INVALID, op, "in_mul = %g must be finite and > 0", (double)in_mul);
    if (n < 1 || n > (int64_t{1} << 40))
        return fail(GQ_ERR_INVALID, op, "n = %lld outside [1, 2^40]", (long long)n);
    GQ_TRY(check_ptr_array(op, "x", x, W, 16));
    GQ_TRY(check_ptr(op, "r_out", r_out, 16));
    gq::SArgs a;
    std::memset(&a, 0, sizeof a);
    for (int32_t w = 0; w < W; ++w) a.x[w] = x[w];
    a.r = r_out;
    a.n = n;
    a.in_mul = in_mul;
    a.W = W;
    a.mean = mean ? 1 : 0;
    return launch_status(op, gq::launch_sum_f32(a, dt, static_cast<hipStream_t>(stream)));
}

gq_status gq_error_report(const int8_t *q, const float *scale, const float *ref,
                          const gq_units *u, double *stats_out, gq_stream stream) {
    const char *op = "gq_error_report";
    GQ_TRY(check_ptr(op, "q", q, 16));
    GQ_TRY(check_ptr(op, "scale", scale, 4));
    GQ_TRY(check_ptr(op, "ref", ref, 16));
    GQ_TRY(check_ptr(op, "stats_out", stats_out, 8));
    GQ_TRY(check_units(op, u));
    const gq::Table &t = u->tab[gq::TAB_R];
    if (!gq::table_ready(t, u->n_units))
        return fail(GQ_ERR_INVALID, op, "unit table is incomplete");
    gq::EArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = q;
    a.scale = scale;
    a.ref = ref;
    a.stats = stats_out;
    a.tiles = t.d_tiles;
    a.unit_first = t.d_unit_first;
    a.partial = reinterpret_cast<uint64_t *>(t.d_partial);
    a.n = u->n;
    a.n_tiles = t.n_tiles;
    a.n_units = u->n_units;
    return launch_status(op, gq::launch_error_report(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
