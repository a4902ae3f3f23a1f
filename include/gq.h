/*
 * gq.h -- C ABI of libgq.so: the per-device compute of an INT8-compressed
 * gradient AllReduce on AMD Instinct MI355X (gfx950).
 *
 * The method comes from the pipelined HCCL AllReduce article
 * (bjdmk.com.cn/news/6235379):
 *   §2.1   each gradient is cut into chunks by dynamic_chunk: a chunk count
 *          of max(1, nbytes // (128 KiB rounded down to a 64-byte multiple))
 *          and the pieces of torch.chunk;
 *   §2.2.1 quantize_gradient: scale = max|g| / 127 and int8 codes
 *          clamp(round(g / scale), -128, 127); the codes and the scale are
 *          what an INT8 AllReduce exchanges;
 *   §6.1   a loss-scaled fp16 gradient is unscaled before quantizing.
 * The article does not define the INT8 AllReduce's arithmetic.  This library
 * implements its reduction step on one device as: dequantize every rank's
 * codes with that rank's scale, add the W contributions in fp32 in rank
 * order 0..W-1 (a rounded multiply, then a rounded add; never a fused
 * multiply-add), and quantize the sum again with a fresh absmax scale.  A
 * unit whose maximum is 0 (or whose scale rounds to 0) gets scale 0 and all
 * codes 0; a NaN quotient (a unit holding inf or NaN) gives code 0.
 *
 * "Units" are the element ranges that share one scale: a whole tensor, one
 * layer tensor of a flattened bucket, or one chunk of a chunk plan.  W ranks
 * of a data-parallel job are W separate buffers in this device's memory,
 * all sharing one unit table (the same model on every rank).
 *
 * Conventions for every function below:
 *   - Returns GQ_OK (0) or an error code; gq_last_error() then describes the
 *     failure (operation, argument, reason) for the calling thread.
 *   - Arguments are checked before anything is enqueued: an error return
 *     means no work was launched and no output was touched.
 *   - Device pointers must point to memory of the device that was current
 *     when the unit table was created, and that device must be current at
 *     the call.  Element buffers (inputs, codes, sums) must be 16-byte
 *     aligned; scale and max buffers 4-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously: outputs are valid once the stream has reached
 *     that point.  The compute calls never synchronize; creating and
 *     destroying tables and plans, and the fault queries and resets, do
 *     (each says so).
 *   - Buffers are owned by the caller and only borrowed while the enqueued
 *     work runs.  The library never allocates in the compute calls.
 *   - A unit table holds scratch memory: calls that use the same table must
 *     be ordered (same stream, or ordered by events); calls on different
 *     tables may be enqueued on different streams.
 *   - gq_quantize (fused form), gq_reduce_requantize and gq_pipe_step run
 *     persistent kernels, whose work groups wait for each other.  Such a
 *     call must not run at the same time as another one of them on the same
 *     device (nor beside any other kernel whose work groups wait on each
 *     other): enqueue them on one stream, or order the streams with events.
 *     Two of them side by side could each hold compute units the other
 *     needs; their waits then give up after about a second, the tables'
 *     fault counters (gq_units_faults) record it, and those calls' outputs
 *     are invalid.  gq_pipe_step's own two streams are safe: the kernels it
 *     runs side by side either are both wholly resident at once (grids
 *     capped at the compute unit count, two work groups per compute unit)
 *     or include one that never waits, and otherwise its reduce takes a
 *     form that never waits.
 *   - Non-finite inputs follow IEEE arithmetic (see above); there is no
 *     error for them.
 */
#ifndef GQ_H
#define GQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQ_OK = 0,
    GQ_ERR_INVALID = 1,  /* null pointer, bad size, bad unit table, W out of range */
    GQ_ERR_ALIGN = 2,    /* a pointer is not aligned as required */
    GQ_ERR_CAPACITY = 3, /* an output array is too small (plan query) */
    GQ_ERR_HIP = 4,      /* the HIP runtime reported an error (launch, alloc) */
    GQ_ERR_DEVICE = 5    /* wrong current device for this unit table */
} gq_status;

typedef enum {
    GQ_F32 = 0, /* IEEE binary32 gradient elements */
    GQ_F16 = 1  /* IEEE binary16 gradient elements (loss-scaled, see in_mul) */
} gq_dtype;

/* Largest number of simulated ranks a call accepts. */
#define GQ_MAX_RANKS 64

/* Bound (exclusive) on the work tiles of a unit table in any of its slot
 * geometries (a unit takes at least one tile; long units several).  It
 * keeps every launch's grid below 2^32 work-items and the tickets a launch
 * hands out (ranks x tiles + resident work groups) below 2^32. */
#define GQ_MAX_TILES (1 << 22)

/* A hipStream_t, passed as an opaque pointer. */
typedef void *gq_stream;

/* Opaque unit table (host copy + device-resident work tables and scratch). */
typedef struct gq_units gq_units;

/* Description of the last error on the calling thread ("" if none). */
const char *gq_last_error(void);

/* Library version string. */
const char *gq_version(void);

/*
 * gq_plan_chunks -- §2.1 dynamic_chunk, host only (no GPU needed).
 *   k = max(1, numel*elem_bytes // (chunk_bytes - chunk_bytes % align_bytes))
 *   pieces = torch.chunk(tensor, k): ceil(numel/k) elements each, the last
 *   one shorter; count = ceil(numel / ceil(numel/k)) (equal to k unless
 *   k*(k-1) >= numel).
 * off_out  host array receiving count+1 element offsets (off[0] = 0,
 *          off[count] = numel); may be NULL when cap = 0 (size query).
 * cap      capacity of off_out in elements.
 * count_out receives the number of pieces (also on GQ_ERR_CAPACITY).
 * The article's constants are chunk_bytes = 131072 and align_bytes = 64.
 * Errors: GQ_ERR_INVALID (numel < 1, elem_bytes < 1, chunk or alignment
 * < 1, chunk_bytes rounded down to the alignment is 0, count_out NULL);
 * GQ_ERR_CAPACITY (cap < count + 1; nothing written to off_out).
 */
gq_status gq_plan_chunks(int64_t numel, int32_t elem_bytes, int64_t chunk_bytes,
                         int32_t align_bytes, int64_t *off_out, int64_t cap,
                         int64_t *count_out);

/*
 * gq_units_create -- build a unit table on the current device.
 * n_units  1 .. GQ_MAX_TILES - 1.
 * h_off    host array of n_units+1 element offsets: h_off[0] >= 0, strictly
 *          increasing; n = h_off[n_units] elements per rank (1 .. 2^40).
 *          Unit u is [h_off[u], h_off[u+1]).  Units may start at any
 *          element offset; elements before h_off[0] belong to no unit and
 *          are neither read into a result nor written.  Per-tensor units
 *          are the tensors' boundaries in the flat buffer; per-chunk units
 *          concatenate each tensor's gq_plan_chunks offsets.
 * out      receives the table.
 * Allocates device memory (work tables + scratch, about 1 KiB per 32K
 * elements) and synchronizes the device.  Errors: GQ_ERR_INVALID (also
 * for a table that would need GQ_MAX_TILES work tiles or more in one of
 * its slot geometries, from about 3.4e10 elements per rank), GQ_ERR_HIP
 * (allocation or copy failed).
 */
gq_status gq_units_create(const int64_t *h_off, int64_t n_units, gq_units **out);

/* Free a unit table.  The work that uses it must have completed.  NULL is
 * accepted.  Errors: GQ_ERR_HIP. */
gq_status gq_units_destroy(gq_units *u);

/* Elements per rank and number of units of a table. */
gq_status gq_units_info(const gq_units *u, int64_t *n, int64_t *n_units);

/*
 * gq_units_schedule -- which schedule the fused quantize of a table uses for
 * elements of type dt.  GQ_SCHED_CHUNK (144 KiB tiles, which hold a 128 KiB
 * chunk of every tensor of 1 MiB or more; 128 KiB tiles where that adds no
 * tile to any unit, see gq_units_quantize_tile) when most elements of the
 * non-small units sit in units that fit one such tile but not one 64 KiB
 * tile (per-chunk scales), or when small units (one wave's share) hold most
 * elements; GQ_SCHED_LAYER (64 KiB tiles) otherwise: per-tensor or
 * per-layer scales, and units too short to fill a 144 KiB tile.  Chosen
 * when the table is created; results do not depend on it.
 */
#define GQ_SCHED_LAYER 0
#define GQ_SCHED_CHUNK 1
gq_status gq_units_schedule(const gq_units *u, gq_dtype dt, int32_t *sched);

/*
 * gq_units_quantize_tile -- elements of type dt per work-group tile of a
 * table's fused quantize: 64 KiB of input under GQ_SCHED_LAYER; under
 * GQ_SCHED_CHUNK 144 KiB, or 128 KiB where no unit needs more tiles of that
 * size (e.g. whole 128 KiB fp32 chunks: 32768 fp32 elements).  Chosen when
 * the table is created; results do not depend on it.  elems: host pointer
 * receiving the number.
 */
gq_status gq_units_quantize_tile(const gq_units *u, gq_dtype dt, int64_t *elems);

/*
 * gq_units_reduce_tile -- elements per work-group tile of a table's reduce:
 * 32768 (chunk-wide tiles, when most elements sit in units of 16385 to
 * 32768 elements, e.g. 128 KiB fp32 chunks: each such unit one tile),
 * 16384 (wide tiles, when most elements sit in units wider than 8192
 * elements: per-layer scales, fp16 chunks) or 8192 (narrow tiles, for
 * tables of short units).  Chosen when the table is created; results do
 * not depend on it.  elems: host pointer receiving the number.
 */
gq_status gq_units_reduce_tile(const gq_units *u, int64_t *elems);

/*
 * gq_units_launch_plan -- informational: how the fused calls (gq_quantize
 * with computed maxima for elements of type dt and multiplier in_mul, and
 * gq_reduce_requantize) run on this table on the current device.
 * q_groups, r_groups  resident work groups of the persistent quantize and
 *                     reduce kernels (the grid of their one-launch form);
 * q_form, r_form      the form each stage takes:
 *   GQ_FORM_PERSISTENT   one persistent launch whose work groups combine a
 *                        long unit's tile maxima (no unit spans more tiles
 *                        than the resident groups); every input read once;
 *   GQ_FORM_TWO_PASS     per-tile maxima, then a pass that reads the tiles
 *                        of the long units again (a unit spans more tiles
 *                        than the resident groups);
 *   GQ_FORM_SHORT_UNITS  tables of short units (every unit fits one tile,
 *                        and units of one wave's share hold most elements):
 *                        wait-free launches, one wave per (rank, unit) and
 *                        one work group per other unit; every input read
 *                        once.
 * Any output pointer may be NULL.  Results do not depend on the form.
 * Errors: GQ_ERR_INVALID (dt, in_mul, NULL table), GQ_ERR_DEVICE,
 * GQ_ERR_HIP (the occupancy query failed, e.g. no device).
 */
#define GQ_FORM_PERSISTENT 0
#define GQ_FORM_TWO_PASS 1
#define GQ_FORM_SHORT_UNITS 2
gq_status gq_units_launch_plan(const gq_units *u, gq_dtype dt, float in_mul, int64_t *q_groups,
                               int32_t *q_form, int64_t *r_groups, int32_t *r_form);

/*
 * gq_units_faults -- number of bounded waits that gave up on the table
 * since it was created or its count was last cleared.  The persistent
 * kernels size their grid to what the device keeps resident; a wait can
 * only give up (after about a second) if the device did not run the whole
 * grid, e.g. while other long-running work held its compute units.  The
 * results of such a launch are invalid.  While the count is nonzero, every
 * wait on the table gives up at its first unsatisfied look (so a launch in
 * that state still ends soon, and its outputs may be invalid too): fix the
 * cause, then clear the count (gq_units_clear_faults) or create a new
 * table.  Synchronizes the device.  count: host pointer receiving the
 * number.
 */
gq_status gq_units_faults(const gq_units *u, uint64_t *count);

/*
 * gq_units_faults_async -- the same count, without synchronizing: a copy of
 * the table's fault count is enqueued on `stream` into count_out (device
 * memory, one uint32, 4-byte aligned), after the work enqueued before it on
 * that stream.  Read it once the stream has reached that point (the
 * caller's usual synchronization).  A nonzero value means that the outputs
 * of every call on the table since the count was last cleared (or the table
 * created) are invalid.  Errors: GQ_ERR_INVALID (NULL table or count_out),
 * GQ_ERR_ALIGN, GQ_ERR_DEVICE, GQ_ERR_HIP.
 */
gq_status gq_units_faults_async(const gq_units *u, uint32_t *count_out, gq_stream stream);

/*
 * gq_units_clear_faults -- sets the table's fault count to zero, so that
 * its waits wait normally again.  The table's other state needs no repair:
 * every launch that has ended leaves it consistent, whether or not its
 * waits gave up.  Synchronizes the device.  Errors: GQ_ERR_INVALID (NULL
 * table), GQ_ERR_DEVICE (table on another device), GQ_ERR_HIP.
 */
gq_status gq_units_clear_faults(gq_units *u);

/*
 * gq_units_force_timeout -- testing aid for the time-out path: makes the
 * fault count nonzero (1 if it was 0), so that the persistent launches on
 * the table (gq_quantize in its fused form, gq_reduce_requantize) take
 * every wait that is not satisfied at its first look as timed out, count
 * it, and go on, until the count is cleared.  Their outputs may then be
 * invalid.  Synchronizes the device.  Errors as gq_units_clear_faults.
 */
gq_status gq_units_force_timeout(gq_units *u);

/*
 * gq_absmax -- §2.2.1 max|g| per unit and rank, with g = float(x) * in_mul
 * (§6.1 unscale; in_mul = 1 for fp32, 1/S for a loss-scaled fp16 gradient).
 * x          host array of W device pointers; x[w] holds n elements of dt.
 * W          1 .. GQ_MAX_RANKS.
 * in_mul     finite, > 0.
 * amax_bits  device array [W][n_units] (rank-major), overwritten with the
 *            bit pattern of max|g| (sign cleared; unsigned order, so a NaN
 *            in the unit wins over inf, inf over every finite value).
 */
gq_status gq_absmax(const void *const *x, int32_t W, gq_dtype dt, float in_mul,
                    const gq_units *u, uint32_t *amax_bits, gq_stream stream);

/*
 * gq_quantize -- §2.2.1 quantize_gradient for W ranks, one scale per unit.
 * scale = fl32(max|g| / 127); code = clamp(round_half_even(fl32(g / scale)),
 * -128, 127); scale 0 gives codes 0; a NaN quotient gives code 0.
 * x          host array of W device pointers (n elements of dt each).
 * amax_bits  NULL: the maxima are computed here, fused with the code pass
 *            (every input read once) for units of up to as many work-group
 *            tiles as the device keeps resident (16K-37K elements per tile:
 *            hundreds of millions of elements); larger units take a second
 *            pass.  Otherwise a device
 *            array [W][n_units] from gq_absmax (or any caller-provided
 *            maxima as bit patterns of non-negative floats).
 * scale_out  host array of W device pointers, each receiving n_units fp32.
 * q_out      host array of W device pointers, each receiving n int8 codes.
 */
gq_status gq_quantize(const void *const *x, int32_t W, gq_dtype dt, float in_mul,
                      const gq_units *u, const uint32_t *amax_bits,
                      float *const *scale_out, int8_t *const *q_out,
                      gq_stream stream);

/*
 * gq_quantize_noalloc -- gq_quantize with the maxima computed (amax_bits =
 * NULL), for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * needs no unit table and allocates nothing: the per-(rank, unit) maxima
 * live in a fixed array of GQ_NOALLOC_MAX_MAXIMA words (4 MiB) in the
 * library's device memory, one per device, which every call on that device
 * shares and which keeps the last call's maxima (each call clears what it
 * uses first).  Calls on one device therefore must not overlap: enqueue
 * them on one stream or order them with events; two overlapping calls race
 * and their outputs are invalid.  Outputs equal gq_quantize's bit for bit.
 * Its three launches never wait on each other's work groups, and the
 * inputs are read twice (once for the maxima, once for the codes).
 * x          host array of W device pointers, n elements of dt each.
 * h_off      host array of n_units+1 unit offsets, as for gq_units_create
 *            (h_off[0] >= 0, strictly increasing, n = h_off[n_units] <=
 *            2^40), checked here.
 * d_off      a device copy of the same n_units+1 int64 offsets (8-byte
 *            aligned), read by the kernels while the call runs.  If it
 *            differs from h_off the outputs are undefined, but every access
 *            stays inside the buffers h_off describes.
 * n_units    1 .. GQ_NOALLOC_MAX_MAXIMA / W.
 * scale_out  host array of W device pointers, each receiving n_units fp32.
 * q_out      host array of W device pointers, each receiving n int8 codes.
 * Errors: GQ_ERR_INVALID (W, dt, in_mul, offsets, NULL pointers, or W *
 * n_units above GQ_NOALLOC_MAX_MAXIMA), GQ_ERR_ALIGN, GQ_ERR_HIP (the
 * array's address could not be looked up, or a launch failed).
 */
#define GQ_NOALLOC_MAX_MAXIMA (1 << 20)
gq_status gq_quantize_noalloc(const void *const *x, int32_t W, gq_dtype dt, float in_mul,
                              const int64_t *h_off, const int64_t *d_off, int64_t n_units,
                              float *const *scale_out, int8_t *const *q_out, gq_stream stream);

/*
 * gq_reduce_dequant -- the INT8 AllReduce reduction of §2.2.1 on one device:
 *   r[i] = (((+0 + q_0[i]*s_0[u]) + q_1[i]*s_1[u]) + ...) + q_{W-1}[i]*s_{W-1}[u]
 * in binary32, each product and each sum rounded (no fused multiply-add),
 * ranks in order, u the unit of element i.
 * q          host array of W device pointers (n int8 codes each).
 * scale      host array of W device pointers (n_units fp32 each).
 * r_out      device array of n fp32.
 */
gq_status gq_reduce_dequant(const int8_t *const *q, const float *const *scale,
                            int32_t W, const gq_units *u, float *r_out,
                            gq_stream stream);

/*
 * gq_requantize -- quantize a reduced fp32 sum again with fresh per-unit
 * scales (gq_quantize of r with W = 1, in_mul = 1).
 * r          device array of n fp32.
 * scale_out  device array of n_units fp32.  q_out: device array of n int8.
 */
gq_status gq_requantize(const float *r, const gq_units *u, float *scale_out,
                        int8_t *q_out, gq_stream stream);

/*
 * gq_reduce_requantize -- gq_reduce_dequant followed by gq_requantize,
 * fused: the sum stays on chip for units of up to as many reduce tiles
 * (gq_units_reduce_tile elements each) as the device keeps resident work
 * groups (it is recomputed from the codes in a second pass for larger
 * units).
 * Results are bit-identical to the two separate calls.
 * r_out      NULL, or a device array of n fp32 that also receives the sum.
 */
gq_status gq_reduce_requantize(const int8_t *const *q, const float *const *scale,
                               int32_t W, const gq_units *u, float *r_out,
                               float *scale_out, int8_t *q_out, gq_stream stream);

/* ---- Two-stream bucket pipeline ------------------------------------------
 * The article's three-stage pipeline (§2.1, pipeline scheduling) overlaps
 * the stages of successive gradient blocks with double buffering, and its
 * tuning parameters (§4.2) set the pipeline depth to 2.  Here the blocks
 * are buckets (consecutive groups of whole units, such as a data-parallel
 * job's 25 MiB gradient buckets), and two slots of codes stand in for the
 * whole model's codes.  Bucket b uses code slot b % 2.  Where every kernel
 * of the plan that waits on its own work groups fits two of them per
 * compute unit, buckets alternate between the caller's stream and a second
 * stream (even buckets on the caller's), each bucket's quantize then its
 * reduce + requantize on its own stream, so that a bucket's stages overlap
 * the other stream's bucket with no event inside the step; the waiting
 * kernels' grids are then capped at the compute unit count (two of them
 * side by side are both wholly resident).  Otherwise every quantize runs
 * on the caller's stream and every reduce on the second stream after an
 * event, bucket b's reduce overlapping bucket b+1's quantize, and bucket
 * b+2's quantize waits until bucket b's reduce has released the slot. */

typedef struct gq_pipe gq_pipe;

/*
 * gq_pipe_create -- plan the pipelined step on the current device.
 * h_off         n_units+1 unit offsets as for gq_units_create, h_off[0] = 0.
 * bucket_units  n_buckets+1 unit indices: bucket b is the units
 *               [bucket_units[b], bucket_units[b+1]); bucket_units[0] = 0,
 *               strictly increasing, bucket_units[n_buckets] = n_units.
 * mode          GQ_PIPE_OVERLAP: the two streams above.  GQ_PIPE_SERIAL:
 *               every stage on the caller's stream, bucket after bucket
 *               (no overlap; every stage in its full form, each bucket's
 *               codes read soon after they were written).
 * out           receives the plan.
 * Builds one unit table per bucket, a second stream (default priority) and
 * the events that order the two; allocates and synchronizes.  Errors:
 * GQ_ERR_INVALID, GQ_ERR_HIP.
 */
#define GQ_PIPE_OVERLAP 0
#define GQ_PIPE_SERIAL 1
gq_status gq_pipe_create(const int64_t *h_off, int64_t n_units, const int64_t *bucket_units,
                         int64_t n_buckets, int32_t mode, gq_pipe **out);

/* Free a plan (its work must have completed; NULL is accepted). */
gq_status gq_pipe_destroy(gq_pipe *p);

/*
 * gq_pipe_slots -- sizes of one slot: slot_elems int8 codes and slot_units
 * fp32 scales per rank (a bucket's elements from a 16-element boundary at
 * or before its first unit, and its unit count, for the largest bucket).
 */
gq_status gq_pipe_slots(const gq_pipe *p, int64_t *slot_elems, int64_t *slot_units);

/*
 * gq_pipe_schedule -- which schedule gq_pipe_step runs for this plan with
 * gradients of type dt and multiplier in_mul on the current device
 * (informational; see the pipeline comment above): GQ_PIPE_SCHED_ALTERNATE
 * (buckets alternate between the two streams, waiting kernels' grids
 * capped at the compute unit count), GQ_PIPE_SCHED_EVENTS (quantizes on the
 * caller's stream, reduces on the second stream after events) or
 * GQ_PIPE_SCHED_SERIAL (a GQ_PIPE_SERIAL plan).  Errors: GQ_ERR_INVALID,
 * GQ_ERR_DEVICE, GQ_ERR_HIP.
 */
#define GQ_PIPE_SCHED_ALTERNATE 0
#define GQ_PIPE_SCHED_EVENTS 1
#define GQ_PIPE_SCHED_SERIAL 2
gq_status gq_pipe_schedule(const gq_pipe *p, gq_dtype dt, float in_mul, int32_t *schedule);

/*
 * gq_pipe_faults -- bounded waits that gave up in the plan's persistent
 * launches (see gq_units_faults; the plan's tables keep their counts until
 * gq_pipe_clear_faults).  Synchronizes the device.
 */
gq_status gq_pipe_faults(const gq_pipe *p, uint64_t *count);

/*
 * gq_pipe_clear_faults -- gq_units_clear_faults on each of the plan's
 * tables.  Synchronizes the device.  Errors: GQ_ERR_INVALID (NULL plan),
 * GQ_ERR_DEVICE, GQ_ERR_HIP.
 */
gq_status gq_pipe_clear_faults(gq_pipe *p);

/*
 * gq_pipe_step -- the whole per-device step (the codes and scales of every
 * rank, their rank-order reduction and its requantization), bucket by
 * bucket with the two-slot pipeline above.  scale_out and q_out equal
 * those of gq_quantize followed by gq_reduce_requantize bit for bit.
 * x           host array of W device pointers, n elements of dt each,
 *             16-byte aligned.
 * q_slot      host array of 2*W device pointers: slot s of rank w is
 *             q_slot[s*W + w], slot_elems int8, 16-byte aligned.  After the
 *             call a slot holds the codes of the last bucket that used it,
 *             from that bucket's 16-element boundary on.
 * scale_slot  host array of 2*W device pointers, slot_units fp32 each,
 *             4-byte aligned; likewise the last bucket's scales.
 * scale_out   device array of n_units fp32.  q_out: device array of n int8.
 * `stream` waits for all of the step's work before anything later on it
 * runs.  A launch error after the first bucket leaves earlier buckets'
 * work enqueued.  Calls sharing a plan must be ordered.
 */
gq_status gq_pipe_step(gq_pipe *p, const void *const *x, int32_t W, gq_dtype dt, float in_mul,
                       int8_t *const *q_slot, float *const *scale_slot, float *scale_out,
                       int8_t *q_out, gq_stream stream);

/* ---- Adaptive chunk size -------------------------------------------------
 * The article's adaptive chunking (§6.2) keeps the last 100 (chunk size,
 * latency) observations and predicts the best chunk size from them with an
 * exponentially weighted moving average; the prediction step is not
 * printed.  Reading taken here: an observation's cost is its latency per
 * byte of chunk; for every chunk size in the history, the costs of that
 * size are averaged in arrival order as e = alpha*x + (1-alpha)*e, starting
 * from the first such cost (binary64, one rounding per operation); the size
 * with the lowest average is predicted, ties going to the larger size; an
 * empty history predicts the default.  A different chunk size gives
 * different chunks and, with per-chunk scales, different codes: callers opt
 * in by planning with gq_chunker_plan.  Host only; calls on one chunker
 * must not overlap. */

typedef struct gq_chunker gq_chunker;

/* capacity: history length (the article: 100), 1 .. 2^20.  alpha: weight
 * of the newest cost, in (0, 1].  default_bytes: prediction of an empty
 * history (the article's 128 KiB), >= 1.  Errors: GQ_ERR_INVALID. */
gq_status gq_chunker_create(int32_t capacity, double alpha, int64_t default_bytes,
                            gq_chunker **out);

/* Free a chunker (NULL is accepted). */
gq_status gq_chunker_destroy(gq_chunker *c);

/* Record one observation: a chunk of chunk_bytes (>= 1) took latency
 * seconds (finite, >= 0).  The oldest observation leaves a full history.
 * Errors: GQ_ERR_INVALID. */
gq_status gq_chunker_update(gq_chunker *c, int64_t chunk_bytes, double latency);

/* The predicted chunk size in bytes (host pointer). */
gq_status gq_chunker_predict(const gq_chunker *c, int64_t *chunk_bytes);

/* gq_plan_chunks with the predicted chunk size and the article's 64-byte
 * alignment term (same outputs and errors). */
gq_status gq_chunker_plan(const gq_chunker *c, int64_t numel, int32_t elem_bytes,
                          int64_t *off_out, int64_t cap, int64_t *count_out);

/* ---- Precision check with quantization switched off ----------------------
 * The article's troubleshooting section (§5.2, gradient anomalies) checks
 * whether a problem is one of precision by switching gradient quantization
 * off.  These two calls give that fp32 reference and measure an INT8 result
 * against it, unit by unit. */

/*
 * gq_sum_f32 -- the fp32 AllReduce reduction of the unquantized gradients
 * on one device:
 *   r[i] = (((+0 + g_0[i]) + g_1[i]) + ...) + g_{W-1}[i],  g_w = float(x_w) * in_mul
 * each sum rounded to binary32, ranks in order (the same order as the INT8
 * reduction).  mean != 0 then divides every sum by W (one rounded binary32
 * division): the averaged gradient of data-parallel training, as in the
 * torchtitan-npu article's mixed-precision listing, which divides
 * all-reduced fp32 gradients by the group size.
 * x      host array of W device pointers, each n elements of dt, 16-byte
 *        aligned.
 * n      elements per rank, 1 .. 2^40.  No unit table is needed.
 * r_out  device array of n fp32, 16-byte aligned, not overlapping x.
 * Errors: GQ_ERR_INVALID (W, dt, n, in_mul as for gq_absmax; NULL
 * pointers), GQ_ERR_ALIGN, GQ_ERR_HIP.
 */
gq_status gq_sum_f32(const void *const *x, int32_t W, gq_dtype dt, float in_mul, int64_t n,
                     int32_t mean, float *r_out, gq_stream stream);

/*
 * gq_error_report -- per-unit statistics, in binary64, of an INT8 result
 * against an fp32 reference: d[i] = fl32(float(q[i]) * scale[u]) (the value
 * the codes stand for, one binary32 rounding) and ref[i], over the elements
 * i of unit u.  GQ_STATS doubles per unit, in the order of GQ_STAT_*:
 *   MAX_ABS_ERR   max |d - ref|   (the binary64 difference, rounded once)
 *   MAX_ABS_REF   max |ref|
 *   MAX_REL_ERR   MAX_ABS_ERR / MAX_ABS_REF
 *   SUM_ABS_ERR   sum |d - ref|
 *   SUM_ABS_REF   sum |ref|
 *   MEAN_REL_ERR  SUM_ABS_ERR / SUM_ABS_REF
 *   SUM_DD, SUM_RR, SUM_DR   sum d^2, sum ref^2, sum d*ref
 *   COS           SUM_DR / sqrt(SUM_DD * SUM_RR)   (cosine similarity)
 * A 0/0 ratio is 0 (a unit with nothing in it has no error); COS is 1 when
 * d and ref are both zero and 0 when exactly one is.  Maxima compare |x| as
 * bit patterns, so a NaN anywhere in the unit gives a NaN maximum; NaN and
 * inf enter the sums by IEEE rules.  The maxima are exact.  The sums are
 * taken in a fixed order (repeatable bit for bit), not element order: each
 * lies within 2 (m-1) 2^-53 / (1 - (m-1) 2^-53) of the sum of its terms'
 * magnitudes from the element-order sum, m the unit's length.
 * q          device array of n int8 codes, 16-byte aligned.
 * scale      device array of n_units fp32.
 * ref        device array of n fp32, 16-byte aligned.
 * stats_out  device array of n_units * GQ_STATS doubles, 8-byte aligned.
 * Uses the table's scratch (ordered with other calls on the table).
 * Errors: GQ_ERR_INVALID, GQ_ERR_ALIGN, GQ_ERR_DEVICE, GQ_ERR_HIP.
 */
#define GQ_STAT_MAX_ABS_ERR 0
#define GQ_STAT_MAX_ABS_REF 1
#define GQ_STAT_MAX_REL_ERR 2
#define GQ_STAT_SUM_ABS_ERR 3
#define GQ_STAT_SUM_ABS_REF 4
#define GQ_STAT_MEAN_REL_ERR 5
#define GQ_STAT_SUM_DD 6
#define GQ_STAT_SUM_RR 7
#define GQ_STAT_SUM_DR 8
#define GQ_STAT_COS 9
#define GQ_STATS 10
gq_status gq_error_report(const int8_t *q, const float *scale, const float *ref,
                          const gq_units *u, double *stats_out, gq_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* GQ_H */
