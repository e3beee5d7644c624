// ep_loop.cpp -- a native serving loop over the C ABI, the way a C++ serving
// process would drive the library, in two forms:
//   - direct: ep_layout_dispatch + ep_combine enqueued back to back on one
//     stream, no synchronisation inside the loop;
//   - graph1: the same two calls recorded once into a HIP graph
//     (ep_graph_begin / ep_graph_end) and the graph replayed once per step.
// For each it reports the host time per step (what the enqueue costs), the
// wall time per step (whichever of host and GPU paces the loop) and, for the
// graph, the device time per step between two events around all replays.  At
// a few tokens the sources found the host pacing the GPU (MoRI PR #614,
// view-cache paragraph); this measures that quantity for this library without
// an interpreter in between.
//
//   ep_loop T H K E P [payload fp8|bf16] [steps]
//
// Inputs are synthetic: token t's K experts are distinct (a fixed stride
// through the experts), hidden values and expert outputs a fixed pattern,
// weights 1/K.  Prints one JSON line.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ep.h"

#define CK(x)                                                                         \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_),  \
                         __LINE__);                                                   \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

int main(int argc, char** argv)
{
    if (argc < 6) {
        std::fprintf(stderr, "usage: %s T H K E P [fp8|bf16] [steps]\n", argv[0]);
        return 2;
    }
    const int T = std::atoi(argv[1]), H = std::atoi(argv[2]), K = std::atoi(argv[3]);
    const int E = std::atoi(argv[4]), P = std::atoi(argv[5]);
    const int payload = (argc > 6 && std::strcmp(argv[6], "bf16") == 0) ? EP_PAYLOAD_BF16
                                                                        : EP_PAYLOAD_FP8_E4M3FN;
    const int steps = argc > 7 ? std::atoi(argv[7]) : 5000;
    if (T < 1 || K < 1 || K > E || steps < 1) {
        std::fprintf(stderr, "bad arguments\n");
        return 2;
    }
    const size_t n = (size_t)T * K;
    std::vector<int32_t> idx(n);
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) idx[(size_t)t * K + k] = (int32_t)((t * 7 + k * (E / K)) % E);
    std::vector<float> w(n, 1.0f / K);
    const size_t xb = (size_t)T * H * 2, rowb = payload == EP_PAYLOAD_BF16 ? (size_t)H * 2 : (size_t)H;

    int32_t *d_idx, *cnt, *off, *pc, *po, *rop, *src;
    uint32_t* st;
    uint16_t *x, *y, *out;
    void* rx;
    float *rs, *d_w;
    CK(hipMalloc(&d_idx, n * 4));
    CK(hipMalloc(&cnt, (size_t)E * 4));
    CK(hipMalloc(&off, (size_t)(E + 1) * 4));
    CK(hipMalloc(&pc, (size_t)P * 4));
    CK(hipMalloc(&po, (size_t)(P + 1) * 4));
    CK(hipMalloc(&rop, n * 4));
    CK(hipMalloc(&src, n * 4));
    CK(hipMalloc(&st, 4));
    CK(hipMalloc(&x, xb));
    CK(hipMalloc(&y, n * H * 2));
    CK(hipMalloc(&out, xb));
    CK(hipMalloc(&rx, n * rowb));
    CK(hipMalloc(&rs, n * (H / 128 > 0 ? H / 128 : 1) * 4));
    CK(hipMalloc(&d_w, n * 4));
    const size_t wsb = ep_layout_workspace_bytes(T, K, E);
    void* ws = nullptr;
    if (wsb) CK(hipMalloc(&ws, wsb));
    CK(hipMemcpy(d_idx, idx.data(), n * 4, hipMemcpyHostToDevice));
    CK(hipMemcpy(d_w, w.data(), n * 4, hipMemcpyHostToDevice));
    CK(hipMemset(x, 0x3c, xb));
    CK(hipMemset(y, 0x3c, n * H * 2));
    hipStream_t s;
    CK(hipStreamCreate(&s));

    auto step = [&]() {
        int rc = ep_layout_dispatch(d_idx, x, T, H, K, E, P, payload, cnt, off, pc, po, rop, src,
                                    st, ws, wsb, rx, rs, s);
        if (rc == EP_OK) rc = ep_combine(y, rop, d_w, T, H, K, out, s);
        return rc;
    };
    for (int i = 0; i < 200; ++i)
        if (int rc = step()) {
            std::fprintf(stderr, "step failed: %s\n", ep_strerror(rc));
            return 1;
        }
    CK(hipStreamSynchronize(s));
    using clk = std::chrono::steady_clock;
    auto us = [](clk::time_point a, clk::time_point b, int n) {
        return std::chrono::duration<double, std::micro>(b - a).count() / n;
    };
    // direct launches
    const auto t0 = clk::now();
    for (int i = 0; i < steps; ++i) step();
    const auto t1 = clk::now();
    CK(hipStreamSynchronize(s));
    const auto t2 = clk::now();
    // one-step graph, replayed once per step
    void* g = nullptr;
    if (int rc = ep_graph_begin(s)) {
        std::fprintf(stderr, "ep_graph_begin: %s\n", ep_strerror(rc));
        return 1;
    }
    const int rc_step = step();
    if (int rc = ep_graph_end(s, &g)) {
        std::fprintf(stderr, "ep_graph_end: %s\n", ep_strerror(rc));
        return 1;
    }
    if (rc_step) {
        std::fprintf(stderr, "captured step failed: %s\n", ep_strerror(rc_step));
        return 1;
    }
    for (int i = 0; i < 200; ++i) ep_graph_launch(g, s);
    CK(hipStreamSynchronize(s));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    const auto g0 = clk::now();
    CK(hipEventRecord(e0, s));
    for (int i = 0; i < steps; ++i) ep_graph_launch(g, s);
    CK(hipEventRecord(e1, s));
    const auto g1 = clk::now();
    CK(hipStreamSynchronize(s));
    const auto g2 = clk::now();
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, e0, e1));
    ep_graph_destroy(g);
    std::printf("{\"T\": %d, \"H\": %d, \"K\": %d, \"E\": %d, \"P\": %d, \"steps\": %d, "
                "\"host_us_per_step\": %.3f, \"wall_us_per_step\": %.3f, "
                "\"graph1_host_us_per_step\": %.3f, \"graph1_wall_us_per_step\": %.3f, "
                "\"graph1_events_us_per_step\": %.3f}\n",
                T, H, K, E, P, steps, us(t0, t1, steps), us(t0, t2, steps), us(g0, g1, steps),
                us(g0, g2, steps), ms * 1000.0 / steps);
    CK(hipEventDestroy(e0));
    CK(hipEventDestroy(e1));
    CK(hipStreamDestroy(s));
    return 0;
}
