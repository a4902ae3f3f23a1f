// abi_step.cpp -- drives libgq.so through its C ABI alone (no Python tensor
// library): device buffers from hipMalloc, a hipStream_t of its own, the
// chunk planner, a unit table, the fused quantize of W ranks and the fused
// reduce + requantize, results copied back to host arrays.  Built into a
// small shared library that the GPU tests load and call; the comparison
// with the oracle happens in the test.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/gq.h"

namespace {

int report(const char *what, gq_status st) {
    std::fprintf(stderr, "abi_step: %s failed (%d): %s\n", what, static_cast<int>(st),
                 gq_last_error());
    return 10 + static_cast<int>(st);
}

}  // namespace

extern "C" {

// Chunk plan of one tensor of numel elements of elem_bytes, through the C
// ABI's size query then fill.  Returns the number of chunks, or -1.
int64_t abi_plan(int64_t numel, int32_t elem_bytes, int64_t *off_out, int64_t cap) {
    int64_t count = 0;
    gq_status st = gq_plan_chunks(numel, elem_bytes, 131072, 64, nullptr, 0, &count);
    if (st != GQ_ERR_CAPACITY || count < 1) return -1;
    if (cap < count + 1) return -1;
    st = gq_plan_chunks(numel, elem_bytes, 131072, 64, off_out, cap, &count);
    return st == GQ_OK ? count : -1;
}

// One step for W fp32 ranks of n elements (x: host, rank-major [W][n]) and
// the units off[0..n_units].  Outputs (host): scales [W][n_units], codes
// [W][n], scale_out [n_units], q_out [n].  Returns 0 on success.
int abi_step(const float *x, int32_t W, int64_t n, const int64_t *off, int64_t n_units,
             float *scales, int8_t *codes, float *scale_out, int8_t *q_out) {
    gq_units *u = nullptr;
    gq_status st = gq_units_create(off, n_units, &u);
    if (st != GQ_OK) return report("gq_units_create", st);
    hipStream_t s = nullptr;
    if (hipStreamCreate(&s) != hipSuccess) return 2;
    std::vector<void *> dx(W), dq(W), ds(W);
    void *d_sout = nullptr, *d_qout = nullptr;
    int rc = 0;
    for (int32_t w = 0; w < W && rc == 0; ++w) {
        if (hipMalloc(&dx[w], n * sizeof(float)) != hipSuccess ||
            hipMalloc(&dq[w], n) != hipSuccess ||
            hipMalloc(&ds[w], n_units * sizeof(float)) != hipSuccess ||
            hipMemcpy(dx[w], x + static_cast<int64_t>(w) * n, n * sizeof(float),
                      hipMemcpyHostToDevice) != hipSuccess)
            rc = 3;
    }
    if (rc == 0 && (hipMalloc(&d_sout, n_units * sizeof(float)) != hipSuccess ||
                    hipMalloc(&d_qout, n) != hipSuccess))
        rc = 3;
    if (rc == 0) {
        std::vector<const void *> px(dx.begin(), dx.end());
        std::vector<float *> ps(W);
        std::vector<int8_t *> pq(W);
        std::vector<const int8_t *> cq(W);
        std::vector<const float *> cs(W);
        for (int32_t w = 0; w < W; ++w) {
            ps[w] = static_cast<float *>(ds[w]);
            pq[w] = static_cast<int8_t *>(dq[w]);
            cq[w] = pq[w];
            cs[w] = ps[w];
        }
        st = gq_quantize(px.data(), W, GQ_F32, 1.0f, u, nullptr, ps.data(), pq.data(), s);
        if (st != GQ_OK) rc = report("gq_quantize", st);
        if (rc == 0) {
            st = gq_reduce_requantize(cq.data(), cs.data(), W, u, nullptr,
                                      static_cast<float *>(d_sout), static_cast<int8_t *>(d_qout), s);
            if (st != GQ_OK) rc = report("gq_reduce_requantize", st);
        }
        // an argument error leaves the stream untouched and is reported
        if (rc == 0 && gq_quantize(px.data(), 0, GQ_F32, 1.0f, u, nullptr, ps.data(), pq.data(),
                                   s) != GQ_ERR_INVALID)
            rc = 4;
        if (rc == 0 && hipStreamSynchronize(s) != hipSuccess) rc = 5;
        uint64_t faults = 1;
        if (rc == 0 && (gq_units_faults(u, &faults) != GQ_OK || faults != 0)) rc = 6;
        for (int32_t w = 0; w < W && rc == 0; ++w) {
            if (hipMemcpy(scales + static_cast<int64_t>(w) * n_units, ds[w], n_units * sizeof(float),
                          hipMemcpyDeviceToHost) != hipSuccess ||
                hipMemcpy(codes + static_cast<int64_t>(w) * n, dq[w], n, hipMemcpyDeviceToHost) !=
                    hipSuccess)
                rc = 7;
        }
        if (rc == 0 && (hipMemcpy(scale_out, d_sout, n_units * sizeof(float),
                                  hipMemcpyDeviceToHost) != hipSuccess ||
                        hipMemcpy(q_out, d_qout, n, hipMemcpyDeviceToHost) != hipSuccess))
            rc = 7;
    }
    for (int32_t w = 0; w < W; ++w) {
        if (dx[w]) (void)hipFree(dx[w]);
        if (dq[w]) (void)hipFree(dq[w]);
        if (ds[w]) (void)hipFree(ds[w]);
    }
    if (d_sout) (void)hipFree(d_sout);
    if (d_qout) (void)hipFree(d_qout);
    (void)hipStreamDestroy(s);
    if (gq_units_destroy(u) != GQ_OK && rc == 0) rc = 8;
    return rc;
}

}  // extern "C"
