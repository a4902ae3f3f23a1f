// gq_chunker.cpp -- adaptive chunk size (pipelined HCCL AllReduce article,
// bjdmk.com.cn/news/6235379, §6.2 adaptive chunking): a history of the last
// `capacity` (chunk size, latency) observations and an exponentially
// weighted moving average that predicts the best chunk size.  The article
// prints the history and the update but not the prediction; this follows
// the reading stated in include/gq.h: per chunk size, the average of
// latency per byte over that size's observations in arrival order; the
// lowest average wins, ties to the larger size.  Host code only.
#include <cmath>
#include <cstdint>
#include <map>
#include <new>
#include <vector>

#include "../../include/gq.h"

struct gq_chunker {
    int32_t capacity = 100;
    double alpha = 0.25;
    int64_t default_bytes = 131072;
    std::vector<int64_t> size;   // ring of observations
    std::vector<double> latency;
    int64_t head = 0;            // index of the oldest entry once the ring is full
    int64_t count = 0;           // observations held (<= capacity)
};

// Error reporting shared with gq_abi.cpp (GQ_OK clears the text).
extern "C" __attribute__((visibility("hidden"))) gq_status
gq_set_error_internal(gq_status code, const char *op, const char *what);

namespace {

gq_status chunker_fail(gq_status code, const char *what) {
    return gq_set_error_internal(code, "gq_chunker", what);
}

}  // namespace

extern "C" {

gq_status gq_chunker_create(int32_t capacity, double alpha, int64_t default_bytes,
                            gq_chunker **out) {
    if (!out) return chunker_fail(GQ_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (capacity < 1 || capacity > (1 << 20))
        return chunker_fail(GQ_ERR_INVALID, "capacity outside [1, 2^20]");
    if (!(alpha > 0.0 && alpha <= 1.0)) return chunker_fail(GQ_ERR_INVALID, "alpha outside (0, 1]");
    if (default_bytes < 1) return chunker_fail(GQ_ERR_INVALID, "default_bytes < 1");
    gq_chunker *c = new (std::nothrow) gq_chunker;
    if (!c) return chunker_fail(GQ_ERR_INVALID, "out of host memory");
    c->capacity = capacity;
    c->alpha = alpha;
    c->default_bytes = default_bytes;
    c->size.assign(static_cast<size_t>(capacity), 0);
    c->latency.assign(static_cast<size_t>(capacity), 0.0);
    *out = c;
    return gq_set_error_internal(GQ_OK, "", "");
}

gq_status gq_chunker_destroy(gq_chunker *c) {
    delete c;
    return gq_set_error_internal(GQ_OK, "", "");
}

gq_status gq_chunker_update(gq_chunker *c, int64_t chunk_bytes, double latency) {
    if (!c) return chunker_fail(GQ_ERR_INVALID, "chunker is NULL");
    if (chunk_bytes < 1) return chunker_fail(GQ_ERR_INVALID, "chunk_bytes < 1");
    if (!std::isfinite(latency) || latency < 0.0)
        return chunker_fail(GQ_ERR_INVALID, "latency must be finite and >= 0");
    const int64_t cap = c->capacity;
    int64_t slot;
    if (c->count < cap) {
        slot = (c->head + c->count) % cap;
        ++c->count;
    } else {
        slot = c->head;               // overwrite the oldest
        c->head = (c->head + 1) % cap;
    }
    c->size[static_cast<size_t>(slot)] = chunk_bytes;
    c->latency[static_cast<size_t>(slot)] = latency;
    return gq_set_error_internal(GQ_OK, "", "");
}

gq_status gq_chunker_predict(const gq_chunker *c, int64_t *chunk_bytes) {
    if (!c || !chunk_bytes) return chunker_fail(GQ_ERR_INVALID, "chunker or chunk_bytes is NULL");
    struct Avg {
        double e = 0.0;
        bool started = false;
    };
    std::map<int64_t, Avg> avg;
    const double a = c->alpha, keep = 1.0 - c->alpha;
    for (int64_t k = 0; k < c->count; ++k) {  // oldest first
        const size_t i = static_cast<size_t>((c->head + k) % c->capacity);
        const int64_t s = c->size[i];
        const double x = c->latency[i] / static_cast<double>(s);
        Avg &v = avg[s];
        if (v.started) {
            v.e = a * x + keep * v.e;
        } else {
            v.e = x;
            v.started = true;
        }
    }
    int64_t best = c->default_bytes;
    bool have = false;
    double best_e = 0.0;
    for (auto it = avg.rbegin(); it != avg.rend(); ++it) {  // larger sizes first: ties stay
        if (!have || it->second.e < best_e) {
            best = it->first;
            best_e = it->second.e;
            have = true;
        }
    }
    *chunk_bytes = best;
    return gq_set_error_internal(GQ_OK, "", "");
}

gq_status gq_chunker_plan(const gq_chunker *c, int64_t numel, int32_t elem_bytes,
                          int64_t *off_out, int64_t cap, int64_t *count_out) {
    int64_t chunk = 0;
    const gq_status st = gq_chunker_predict(c, &chunk);
    if (st != GQ_OK) return st;
    return gq_plan_chunks(numel, elem_bytes, chunk, 64, off_out, cap, count_out);
}

}  // extern "C"
