// bench_host.hip -- host-side timing of librattn's C ABI for the benchmark.
// Built into librattn_bench.so; NOT part of the product ABI (include/rattn.h).
//
// The quantity the pages put first is the per-call dispatch floor: host call
// to completion at ViT sizes, where launch overhead exceeds the compute (paper
// abstract; radpulse.milrad-way.com write-up, sections on FlashAttention-2's
// 62 us ceiling and the 40 us Triton kernel).  These loops time it from C++
// with std::chrono::steady_clock, so that no interpreter sits in the loop:
//   * empty-kernel launch + hipStreamSynchronize: the platform's floor;
//   * rattn_forward + sync, the whole pack -> forward -> unpack step + sync, and
//     the one-launch rattn_fused + sync;
//   * the same step replayed from a captured hipGraph + sync, and the graph
//     launch's own enqueue cost;
//   * enqueue-only cost of the calls (no sync inside the timed span);
//   * a stack of attention layers on one keep mask: packed once, attended per
//     layer, unpacked once (section on the integrated packing pipeline: the
//     packed buffer is kept across blocks), against the one-launch form
//     repeated per layer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <utility>
#include <chrono>
#include <vector>

#include "rattn.h"

extern "C" {

typedef struct bench_stats {
    double median_us, p5_us, p95_us, mean_us, min_us;
} bench_stats;

typedef struct bench_step {
    const void *src[3];   // padded q, k, v [B, N, H, 64]
    void *packed[3];      // flat q, k, v [>= T, H, 64]
    void *o;              // flat attention output
    void *out_padded;     // [B, N, H, 64] (nullable)
    void *cls;            // [B, H, 64] (nullable)
    const uint8_t *keep;  // [B, N]
    int32_t *cu;          // [B+1]
    int32_t *max_dev;     // nullable
    int32_t *total_dev;   // nullable
    int B, N, H, max_seqlen, dtype;
    float scale;
    void *stream;
    int layers;           // attention layers of the stacked steps (what = 3, 4)
    void *out_padded2;    // second padded [B, N, H, 64] buffer for the stacked one-launch form
    const uint8_t *keep2; // [>= T] second keep flag per flat row (what = 5)
    int32_t *cu2;         // [B+1] cu_seqlens after the re-pack
    void *repacked[3];    // flat q, k, v after the re-pack [>= T2, H, 64]
} bench_step;

}  // extern "C"

namespace {

__global__ void empty_kernel() {}

using clk = std::chrono::steady_clock;

void summarize(std::vector<double> &v, bench_stats *s) {
    std::sort(v.begin(), v.end());
    const size_t n = v.size();
    auto at = [&](double f) { return v[std::min(n - 1, (size_t)(f * (n - 1) + 0.5))]; };
    double sum = 0;
    for (double x : v) sum += x;
    s->median_us = at(0.5);
    s->p5_us = at(0.05);
    s->p95_us = at(0.95);
    s->mean_us = sum / n;
    s->min_us = v[0];
}

rattn_status do_forward(const bench_step *a) {
    return rattn_forward(a->packed[0], a->packed[1], a->packed[2], a->o, a->cu, a->B,
                         a->max_seqlen, a->H, RATTN_HEAD_DIM, a->scale, (rattn_dtype)a->dtype,
                         a->stream);
}

rattn_status do_step(const bench_step *a) {
    rattn_status s = rattn_pack(a->src, a->packed, 3, a->keep, a->B, a->N, a->H * RATTN_HEAD_DIM,
                                (rattn_dtype)a->dtype, a->cu, a->max_dev, a->total_dev, a->stream);
    if (s != RATTN_OK) return s;
    s = do_forward(a);
    if (s != RATTN_OK) return s;
    return rattn_unpack(a->o, a->out_padded, a->cls, a->keep, a->cu, a->B, a->N,
                        a->H * RATTN_HEAD_DIM, (rattn_dtype)a->dtype, a->stream);
}

rattn_status do_fused(const bench_step *a) {
    return rattn_fused(a->src[0], a->src[1], a->src[2], a->keep, a->out_padded, a->cls, a->B, a->N,
                       a->H, RATTN_HEAD_DIM, a->max_seqlen, a->scale, (rattn_dtype)a->dtype,
                       a->stream);
}

// `layers` attention layers on one mask, each layer's output the next layer's
// query (k and v stay those of the first layer: the work per layer is the same
// as with fresh k, v): rattn_pack once, rattn_forward per layer on the flat
// buffers (ping-pong between the flat q and o), rattn_unpack of the last
// output once.
rattn_status do_layers_packed(const bench_step *a) {
    const int row = a->H * RATTN_HEAD_DIM;
    const rattn_dtype dt = (rattn_dtype)a->dtype;
    rattn_status s = rattn_pack(a->src, a->packed, 3, a->keep, a->B, a->N, row, dt, a->cu,
                                a->max_dev, a->total_dev, a->stream);
    void *qb = a->packed[0], *ob = a->o;
    for (int l = 0; s == RATTN_OK && l < a->layers; ++l) {
        s = rattn_forward(qb, a->packed[1], a->packed[2], ob, a->cu, a->B, a->max_seqlen, a->H,
                          RATTN_HEAD_DIM, a->scale, dt, a->stream);
        std::swap(qb, ob);
    }
    if (s != RATTN_OK) return s;
    return rattn_unpack(qb, a->out_padded, a->cls, a->keep, a->cu, a->B, a->N, row, dt, a->stream);
}

// The same stack with the one-launch form per layer: every layer gathers from
// and scatters to the padded layout (ping-pong between out_padded and
// out_padded2); the CLS rows are written by the last layer.
rattn_status do_layers_fused(const bench_step *a) {
    const void *qb = a->src[0];
    void *ob = a->out_padded, *other = a->out_padded2;
    rattn_status s = RATTN_OK;
    for (int l = 0; s == RATTN_OK && l < a->layers; ++l) {
        s = rattn_fused(qb, a->src[1], a->src[2], a->keep, ob, l == a->layers - 1 ? a->cls : nullptr,
                        a->B, a->N, a->H, RATTN_HEAD_DIM, a->max_seqlen, a->scale,
                        (rattn_dtype)a->dtype, a->stream);
        qb = ob;
        std::swap(ob, other);
    }
    return s;
}

// A later pruning stage on the packed q, k, v (which a preceding what = 1 or 3
// step has written): rattn_repack under keep2.
rattn_status do_repack(const bench_step *a) {
    return rattn_repack(a->packed, a->repacked, 3, a->keep2, a->cu, a->B, a->H * RATTN_HEAD_DIM,
                        (rattn_dtype)a->dtype, a->cu2, nullptr, a->stream);
}

// what = 0: rattn_forward; 1: rattn_pack + rattn_forward + rattn_unpack;
// 2: rattn_fused (the same pack -> attend -> unpack in one launch);
// 3: `layers` layers packed once (do_layers_packed); 4: the same layers with
// rattn_fused per layer (do_layers_fused); 5: rattn_repack (do_repack).
rattn_status run(const bench_step *a, int what) {
    switch (what) {
        case 0: return do_forward(a);
        case 1: return do_step(a);
        case 2: return do_fused(a);
        case 3: return do_layers_packed(a);
        case 4: return do_layers_fused(a);
        case 5: return do_repack(a);
        default: return RATTN_ERR_INVALID_ARG;
    }
}

}  // namespace

extern "C" {

// Empty kernel launch + stream sync, `iters` times after `warmup`.
int bench_empty_floor(int iters, int warmup, void *stream, bench_stats *out) {
    hipStream_t s = (hipStream_t)stream;
    std::vector<double> t;
    t.reserve(iters);
    for (int i = 0; i < warmup + iters; ++i) {
        auto t0 = clk::now();
        hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
        if (hipStreamSynchronize(s) != hipSuccess) return -1;
        auto t1 = clk::now();
        if (i >= warmup) t.push_back(std::chrono::duration<double, std::micro>(t1 - t0).count());
    }
    summarize(t, out);
    return 0;
}

// Each iteration: host call(s) + hipStreamSynchronize, timed on the host.
int bench_call_floor(const bench_step *a, int what, int iters, int warmup, bench_stats *out) {
    hipStream_t s = (hipStream_t)a->stream;
    std::vector<double> t;
    t.reserve(iters);
    for (int i = 0; i < warmup + iters; ++i) {
        auto t0 = clk::now();
        if (run(a, what) != RATTN_OK) return -2;
        if (hipStreamSynchronize(s) != hipSuccess) return -1;
        auto t1 = clk::now();
        if (i >= warmup) t.push_back(std::chrono::duration<double, std::micro>(t1 - t0).count());
    }
    summarize(t, out);
    return 0;
}

// Host time of the call(s) alone (enqueue, no sync inside the span); the
// stream is drained every 64 iterations outside the timed spans.
int bench_enqueue_cost(const bench_step *a, int what, int iters, bench_stats *out) {
    hipStream_t s = (hipStream_t)a->stream;
    std::vector<double> t;
    t.reserve(iters);
    for (int i = 0; i < iters; ++i) {
        auto t0 = clk::now();
        if (run(a, what) != RATTN_OK) return -2;
        auto t1 = clk::now();
        t.push_back(std::chrono::duration<double, std::micro>(t1 - t0).count());
        if ((i & 63) == 63 && hipStreamSynchronize(s) != hipSuccess) return -1;
    }
    if (hipStreamSynchronize(s) != hipSuccess) return -1;
    summarize(t, out);
    return 0;
}

// Enqueue `steps` calls back to back with no synchronisation (the caller
// brackets it with its own synchronisation and clock).
int bench_loop(const bench_step *a, int what, int steps) {
    for (int i = 0; i < steps; ++i)
        if (run(a, what) != RATTN_OK) return -2;
    return 0;
}

// The same call(s) captured once into a hipGraph and replayed: launch + sync
// per iteration.  The capture stream must not be the legacy default stream.
int bench_graph_floor(const bench_step *a, int what, int iters, int warmup, bench_stats *out) {
    hipStream_t s = (hipStream_t)a->stream;
    if (!s) return -3;
    hipGraph_t g = nullptr;
    hipGraphExec_t ge = nullptr;
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) return -1;
    rattn_status st = run(a, what);
    if (hipStreamEndCapture(s, &g) != hipSuccess || st != RATTN_OK) return -2;
    if (hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) != hipSuccess) return -1;
    std::vector<double> t;
    t.reserve(iters);
    int rc = 0;
    for (int i = 0; i < warmup + iters; ++i) {
        auto t0 = clk::now();
        if (hipGraphLaunch(ge, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess) {
            rc = -1;
            break;
        }
        auto t1 = clk::now();
        if (i >= warmup) t.push_back(std::chrono::duration<double, std::micro>(t1 - t0).count());
    }
    (void)hipGraphExecDestroy(ge);
    (void)hipGraphDestroy(g);
    if (rc == 0) summarize(t, out);
    return rc;
}

// Host time of hipGraphLaunch alone for the same captured call(s), no sync
// inside the timed span (the stream is drained every 64 launches outside it):
// the graph's own enqueue cost, next to bench_enqueue_cost's direct calls.
int bench_graph_enqueue_cost(const bench_step *a, int what, int iters, bench_stats *out) {
    hipStream_t s = (hipStream_t)a->stream;
    if (!s) return -3;
    hipGraph_t g = nullptr;
    hipGraphExec_t ge = nullptr;
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) return -1;
    rattn_status st = run(a, what);
    if (hipStreamEndCapture(s, &g) != hipSuccess || st != RATTN_OK) return -2;
    if (hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) != hipSuccess) return -1;
    std::vector<double> t;
    t.reserve(iters);
    int rc = 0;
    for (int i = 0; i < iters; ++i) {
        auto t0 = clk::now();
        if (hipGraphLaunch(ge, s) != hipSuccess) {
            rc = -1;
            break;
        }
        auto t1 = clk::now();
        t.push_back(std::chrono::duration<double, std::micro>(t1 - t0).count());
        if ((i & 63) == 63 && hipStreamSynchronize(s) != hipSuccess) {
            rc = -1;
            break;
        }
    }
    if (hipStreamSynchronize(s) != hipSuccess) rc = -1;
    (void)hipGraphExecDestroy(ge);
    (void)hipGraphDestroy(g);
    if (rc == 0) summarize(t, out);
    return rc;
}

}  // extern "C"
