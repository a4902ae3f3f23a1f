// gq_internal.h -- types shared by the C-ABI layer (gq_abi.cpp) and the
// gfx950 kernels (gq_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gq.h"

namespace gq {

// One work item of a kernel launch: a contiguous element range of one unit.
// A unit that fits in one work group is one tile ("single"); a larger unit
// is split into `count` tiles at slot-aligned positions, and its scale needs
// a max over all of them.
struct Tile {
    int64_t begin;   // first element (index into the rank's flat buffer)
    int64_t end;     // one past the last element
    int32_t unit;    // unit index
    int32_t first;   // index of the unit's first tile in the table
    int32_t count;   // number of tiles of the unit
    int32_t slot;    // dense index of a multi-tile unit (-1 for a single tile)
};
static_assert(sizeof(Tile) == 32, "Tile layout");

// Slot geometry of a tile table.  A slot is V consecutive elements aligned
// to V in the flat buffer (one 16-byte load); a work group of `block`
// threads holds up to block * slots slots of a tile in registers.
enum TableId { TAB_Q32 = 0, TAB_Q16 = 1, TAB_R = 2, TAB_COUNT = 3 };

// Schedules of the persistent quantize kernel, chosen per unit table:
//  SCHED_LAYER  units spanning many tiles (per-tensor or per-layer scales):
//               512-thread tiles; a work group holds two published tiles
//               (one parked in LDS), so a tile's unit max is first asked for
//               two tiles after its own max was published, and the older
//               tile is coded while the next tile's loads are in flight.
//  SCHED_CHUNK  units of about one tile (per-chunk scales, small tensors):
//               1024-thread tiles of 144 KiB, which hold a whole chunk of
//               the chunk plan for every tensor of 1 MiB or more (those
//               chunks are below 128 KiB * 9/8), or of 128 KiB where that
//               adds no tile to any unit; the next tile's loads are in
//               flight while the current tile's codes are written.
enum Sched { SCHED_LAYER = 0, SCHED_CHUNK = 1 };

constexpr int Q_SLOTS_LAYER = 8;     // 8 x 16 bytes per thread
constexpr int Q_SLOTS_CHUNK = 9;     // 9 x 16 bytes per thread
// Chunk tiles of 8 rows (128 KiB) where no unit needs more tiles of that
// size than of 9 rows, e.g. tables of whole 128 KiB fp32 chunks, whose
// ninth row would stay empty in every tile: the same tiles, one row of
// loads and checks fewer per lane.
constexpr int Q_SLOTS_CHUNK_SHORT = 8;
constexpr int Q_BLOCK_LAYER = 512;   // fp32: 16384 elements per tile (64 KiB)
constexpr int Q_BLOCK_CHUNK = 1024;  // fp32: 36864 elements per tile (144 KiB)
constexpr int R_BLOCK = 512;
// Reduce tiles hold 16 codes (16 sums) per thread and slot.  Wide tiles (two
// slots, 16384 elements) halve the tiles and unit exchanges where most
// elements sit in units wider than a narrow tile; narrow tiles (one slot,
// 8192 elements) serve tables of short units, which would otherwise leave
// most of a wide tile's lanes idle.
constexpr int R_SLOTS_NARROW = 1;
constexpr int R_SLOTS_WIDE = 2;
// Chunk-wide reduce tiles: two slots on 1024 threads (32768 elements, one
// whole 128 KiB fp32 chunk of the chunk plan), for tables whose non-small
// elements sit mostly in units of that size: each such unit is one tile,
// summed and requantized with no exchange between work groups.
constexpr int R_BLOCK_CHUNK = 1024;

// Units whose 16-byte slots span at most 64 * SMALL_SLOTS[table] slots are
// "small": one wave handles a whole unit, in a phase of its own of the
// persistent kernel, with no tile exchange and no ticket.  Reduce tables
// with narrow tiles double that span: their waves sum a unit in two halves.
constexpr int SMALL_SLOTS_Q = 16;    // fp32: 4096 elements, fp16: 8192 elements
constexpr int SMALL_SLOTS_R = 2;     // 2048 elements (4096 in two halves, narrow tables)
// The short-table quantize kernel's waves hold one slot more per lane: a
// unit of 64 * SMALL_SLOTS_Q * V elements then fits at any offset.
constexpr int SHORT_SLOTS_Q = SMALL_SLOTS_Q + 1;

constexpr int kSlotElems[TAB_COUNT] = {4, 8, 16};  // V of each table

// Short reduce tables (see short_table) cut every unit of at most
// PIECE_WAVES * PIECE_SLOTS slots into pieces of PIECE_SLOTS slots (one
// slot per lane of a wave), and pack the pieces into work groups of
// PIECE_WAVES waves so that no unit straddles two groups (a group's unused
// waves get empty pieces).  The waves of one unit combine their maxima in
// LDS.
constexpr int PIECE_WAVES = 8;
constexpr int PIECE_SLOTS = 64;

// Short tables pack units of at most 32 slots several to a wave: a pack
// holds up to 64 / lanes units of at most `lanes` slots (lanes = 4, 8, 16 or
// 32), each taken by its own group of `lanes` lanes, one slot per lane,
// which combine their maxima by shuffles within the group.  (One unit per
// wave would leave most of its lanes idle and pay a wave's whole chain of
// memory round trips for a few elements.)  In a quantize table, a pack
// with lanes = 64 holds one larger unit, taken by the whole wave.
struct Pack {
    int32_t first;   // index of the pack's first unit in the table's pack unit list
    int32_t count;   // units in the pack
    int32_t lanes;   // lanes per unit (a power of two, 4 .. 64)
    int32_t pad;
};
static_assert(sizeof(Pack) == 16, "Pack layout");
constexpr int PACK_MIN_LANES = 4;
// A wave of a short reduce table's piece list that takes a pack: its
// entry's slot field holds PACK_WAVE and its first field the pack's index.
constexpr int32_t PACK_WAVE = -2;

// Cross-work-group state of the persistent kernels: one published-max word
// per tile and rank and one result word per multi-tile unit and rank (high
// half: the launch's tag, low half: a max), one arrival counter per
// multi-tile unit and rank (never reset: a multiple of the unit's tile
// count between launches), and a control block {launch epoch, exited work
// groups}.

struct Table {
    int sched = SCHED_LAYER;
    int block = 0;                  // threads per work group
    int slots = 0;                  // slots per thread
    int64_t n_tiles = 0;
    int64_t n_multi = 0;            // tiles of multi-tile units
    int64_t n_multi_units = 0;      // multi-tile units
    int32_t max_count = 1;          // largest tile count of one unit
    Tile *d_tiles = nullptr;        // [n_tiles], every unit, unit order
    int64_t n_small = 0;            // small units
    Tile *d_small = nullptr;        // [n_small] one entry per small unit
    int64_t n_big = 0;              // tiles of the other units
    Tile *d_big = nullptr;          // [n_big], unit order (first: index into d_big)
    int32_t big_max_count = 1;      // largest tile count of a unit in d_big
    bool small_dominant = false;    // small units hold most elements
    // short tables only: the per-wave work and the tiles of the units it
    // leaves out (first: index into d_rest).  Quantize tables: packs (one
    // item per rank and pack) of the units of at most 64 * SHORT_SLOTS_Q
    // slots.  Reduce table: the pieces of the units of more than 32 and at
    // most PIECE_WAVES * PIECE_SLOTS slots, and the packs of the smaller
    // units, PIECE_WAVES waves per work group (a piece: the unit's elements
    // in its slot range; first = the wave of the group that holds the
    // unit's first piece, count = the unit's pieces; a pack's wave: slot =
    // PACK_WAVE, first = the pack's index; an unused wave's entry has count
    // 0 and slot -1; n_short is a multiple of PIECE_WAVES).
    int64_t n_short = 0;
    Tile *d_short = nullptr;        // quantize: the packs' units; reduce: the waves
    int64_t n_packs = 0;
    Pack *d_packs = nullptr;
    int64_t n_pack_units = 0;       // reduce: the packs' units
    Tile *d_pack_units = nullptr;
    int64_t n_rest = 0;
    Tile *d_rest = nullptr;
    int32_t *d_multi = nullptr;     // [n_multi] indices of multi tiles
    uint32_t *d_partial = nullptr;  // [GQ_MAX_RANKS][n_tiles] per-tile maxima
    int32_t *d_unit_first = nullptr;  // [n_units+1] first tile of each unit
    uint64_t *d_pub = nullptr;      // [GQ_MAX_RANKS][n_big] published tile maxima
    uint64_t *d_res = nullptr;      // [GQ_MAX_RANKS][n_multi_units] published unit maxima
    uint64_t *d_cnt = nullptr;      // [GQ_MAX_RANKS][n_multi_units] arrivals
    uint32_t *d_ctl = nullptr;      // [4]: launch epoch, exited work groups, next ticket
};

// Tables of short units: every unit fits one tile and the small units (one
// wave each) hold most elements.  Their fused stages need no exchange of
// maxima and run as wait-free launches instead of a persistent kernel.
inline bool short_table(const Table &t) { return t.big_max_count == 1 && t.small_dominant; }

// Every array a launcher may hand to a kernel is present and sized for the
// table (launchers check this before launching anything).
inline bool table_ready(const Table &t, int64_t n_units) {
    if (t.n_tiles < n_units || !t.d_tiles || !t.d_unit_first || !t.d_partial || !t.d_ctl)
        return false;
    if (t.n_multi > 0 && !t.d_multi) return false;
    if (t.n_small + t.n_big < 1 || (t.n_small > 0 && !t.d_small) || (t.n_big > 0 && !t.d_big))
        return false;
    if (t.n_multi_units > 0 && (!t.d_pub || !t.d_res || !t.d_cnt)) return false;
    if (short_table(t) && (t.n_short + t.n_rest < 1 || (t.n_short > 0 && !t.d_short) ||
                           (t.n_rest > 0 && !t.d_rest) || (t.n_packs > 0 && !t.d_packs) ||
                           (t.n_pack_units > 0 && !t.d_pack_units)))
        return false;
    return t.block > 0 && t.slots > 0;
}

}  // namespace gq

struct gq_units {
    int device = -1;
    int64_t n = 0;
    int64_t n_units = 0;
    gq::Table tab[gq::TAB_COUNT];
    uint32_t *d_faults = nullptr;   // bounded waits that gave up (never expected)
};

namespace gq {

// Kernel argument blocks (passed by value; W device pointers each).
struct QArgs {
    const void *x[GQ_MAX_RANKS];
    float *scale[GQ_MAX_RANKS];
    int8_t *q[GQ_MAX_RANKS];
    const Tile *tiles;
    const int32_t *list;        // NULL: blockIdx.x is the tile index
    const Tile *small;          // small units (one wave each); short tables: the packs' units
    int64_t n_small;
    const Pack *packs;          // short tables
    int64_t n_packs;
    uint32_t *partial;          // [W][n_tiles]
    const uint32_t *amax;       // [W][n_units] or NULL
    const int32_t *unit_first;  // for the finalize step
    uint32_t *amax_out;         // [W][n_units] (gq_absmax)
    uint64_t *pub;              // [W][n_tiles of the tile list in use]
    uint64_t *res;              // [W][n_multi_units]
    uint64_t *cnt;              // [W][n_multi_units]
    uint32_t *ctl;              // [4]
    uint32_t *faults;
    int64_t n;                  // elements per rank (buffer length)
    int64_t n_tiles;
    int64_t n_units;
    int64_t n_multi_units;
    float in_mul;
    int32_t W;
};

struct RArgs {
    const int8_t *q[GQ_MAX_RANKS];
    const float *scale[GQ_MAX_RANKS];
    const Tile *tiles;
    const int32_t *list;
    const Tile *small;          // small units (one wave each); short tables: the waves
    int64_t n_small;
    const Pack *packs;          // short tables
    const Tile *pack_units;     // short tables: the packs' units
    uint32_t *partial;          // [n_tiles]
    float *r;                   // NULL or [n]
    float *scale_out;           // [n_units]
    int8_t *q_out;              // [n]
    uint64_t *pub;              // [n_tiles]
    uint64_t *res;              // [n_multi_units]
    uint64_t *cnt;              // [n_multi_units]
    uint32_t *ctl;              // [4]
    uint32_t *faults;
    int64_t n;                  // elements per rank (buffer length)
    int64_t n_tiles;
    int32_t W;
};

// Arguments of the unquantized reference sum (gq_check.hip).
struct SArgs {
    const void *x[GQ_MAX_RANKS];
    float *r;                   // [n]
    int64_t n;
    float in_mul;
    int32_t W;
    int32_t mean;
};

// Arguments of the error report (gq_check.hip).  The per-tile partial
// statistics live in the reduce table's scratch (d_partial), which holds
// GQ_MAX_RANKS * 4 bytes per tile; a tile needs kReportWords * 8.
constexpr int kReportWords = 8;
static_assert(kReportWords * 8 <= GQ_MAX_RANKS * 4, "report partials fit the tile scratch");
struct EArgs {
    const int8_t *q;            // [n]
    const float *scale;         // [n_units]
    const float *ref;           // [n]
    double *stats;              // [n_units][GQ_STATS]
    const Tile *tiles;          // reduce table tiles, unit order
    const int32_t *unit_first;  // [n_units + 1]
    uint64_t *partial;          // [n_tiles][kReportWords]
    int64_t n;
    int64_t n_tiles;
    int64_t n_units;
};

// Launchers (gq_kernels.hip, gq_check.hip).  Each returns the first launch
// error.
hipError_t launch_absmax(const QArgs &a, gq_dtype dt, const Table &t, hipStream_t s);
// cap > 0 limits the persistent kernel's grid to cap work groups (the
// one-launch form then runs only if no unit spans more tiles than that).
hipError_t launch_quantize(const QArgs &a, gq_dtype dt, const Table &t, hipStream_t s,
                           int64_t cap = 0);
// wait_free: never use the persistent kernel (whose work groups wait on
// each other); used where another kernel may hold the device's compute
// units at the same time.
hipError_t launch_reduce(const RArgs &a, const Table &t, bool requantize, bool wait_free,
                         hipStream_t s, int64_t cap = 0);
hipError_t launch_sum_f32(const SArgs &a, gq_dtype dt, hipStream_t s);
hipError_t launch_copy_word(const uint32_t *src, uint32_t *dst, hipStream_t s);

// The no-allocation quantize (gq_noalloc.hip).  Its maxima live in a
// fixed-size device array of that file; noalloc_scratch returns that
// array's address on the current device (looked up once per device, with
// the device current), or nullptr if the lookup failed.
constexpr int GQ_NOALLOC_MAX_DEVICES = 64;
struct NoallocArgs {
    const void *const *x;
    float *const *scale;
    int8_t *const *q;
    const int64_t *d_off;   // [n_units + 1] device copy of the unit offsets
    int64_t n_units;
    int64_t n;              // off[n_units]
    int64_t first;          // off[0]
    float in_mul;
    gq_dtype dt;
    int32_t W;
};
void *noalloc_scratch(int device);
hipError_t launch_quantize_noalloc(const NoallocArgs &a, void *scratch_dev, hipStream_t s);
// Resident work groups of the persistent kernels a table's fused calls use
// on the current device (0 if the occupancy query failed): the grid of their
// one-launch form, which runs when no unit spans more tiles than this.
int64_t quantize_resident(gq_dtype dt, bool mul, const Table &t);
int64_t reduce_resident(const Table &t);
// The current device's compute units (0 if the query failed).
int64_t device_cus();
// Whether the fused stage of a table, launched with grid cap `cap` (0: none),
// runs a kernel whose work groups wait on each other (the one-launch
// persistent form on a table with a unit of several tiles).
bool quantize_waits(gq_dtype dt, bool mul, const Table &t, int64_t cap);
bool reduce_waits(const Table &t, int64_t cap);
hipError_t launch_error_report(const EArgs &a, hipStream_t s);

}  // namespace gq
