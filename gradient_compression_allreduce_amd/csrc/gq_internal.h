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

struct TableGeom {
    int V;       // elements per slot
    int block;   // threads per work group
    int slots;   // slots per thread
};

constexpr int Q_BLOCK = 512;
constexpr int Q_SLOTS = 8;      // fp32: 8 x 4 = 32 elements per thread (16384 per tile)
constexpr int R_BLOCK = 512;
constexpr int R_SLOTS = 1;      // 16 codes = 16 sums per thread (8192 per tile)

constexpr TableGeom kGeom[TAB_COUNT] = {
    {4, Q_BLOCK, Q_SLOTS},   // fp32 quantize / requantize
    {8, Q_BLOCK, Q_SLOTS},   // fp16 quantize: 32768 elements per tile
    {16, R_BLOCK, R_SLOTS},  // reduce
};

// Cross-work-group state of the persistent kernels: one published-max word
// per tile and rank and one result word per multi-tile unit and rank (high
// half: the launch's tag, low half: a max), one arrival counter per
// multi-tile unit and rank (never reset: a multiple of the unit's tile
// count between launches), and a control block {launch epoch, exited work
// groups}.

struct Table {
    int64_t n_tiles = 0;
    int64_t n_multi = 0;            // tiles of multi-tile units
    int64_t n_multi_units = 0;      // multi-tile units
    int32_t max_count = 1;          // largest tile count of one unit
    Tile *d_tiles = nullptr;        // [n_tiles], unit order
    int32_t *d_multi = nullptr;     // [n_multi] indices of multi tiles
    uint32_t *d_partial = nullptr;  // [GQ_MAX_RANKS][n_tiles] per-tile maxima
    int32_t *d_unit_first = nullptr;  // [n_units+1] first tile of each unit
    uint64_t *d_pub = nullptr;      // [GQ_MAX_RANKS][n_tiles] published tile maxima
    uint64_t *d_res = nullptr;      // [GQ_MAX_RANKS][n_multi_units] published unit maxima
    uint64_t *d_cnt = nullptr;      // [GQ_MAX_RANKS][n_multi_units] arrivals
    uint32_t *d_ctl = nullptr;      // [4]: launch epoch, exited work groups, next ticket
};

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
    uint32_t *partial;          // [W][n_tiles]
    const uint32_t *amax;       // [W][n_units] or NULL
    const int32_t *unit_first;  // for the finalize step
    uint32_t *amax_out;         // [W][n_units] (gq_absmax)
    uint64_t *pub;              // [W][n_tiles]
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

// Launchers (gq_kernels.hip).  Each returns the first launch error.
hipError_t launch_absmax(const QArgs &a, gq_dtype dt, const Table &t, hipStream_t s);
hipError_t launch_quantize(const QArgs &a, gq_dtype dt, const Table &t, hipStream_t s);
hipError_t launch_reduce(const RArgs &a, const Table &t, bool requantize, hipStream_t s);

}  // namespace gq
