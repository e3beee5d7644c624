// ep_loop.cpp -- a native serving loop over the C ABI: ep_layout_dispatch +
// ep_combine enqueued back to back on one stream, no synchronisation inside
// the loop, the way a C++ serving process would drive the library.  Reports
// the host time per step (what the enqueue costs) and the wall time per step
// (whichever of host and GPU paces the loop).  At a few tokens the sources
// found the host pacing the GPU (MoRI PR #614, view-cache paragraph); this
// measures that quantity for this library without an interpreter in between.
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
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < steps; ++i) step();
    const auto t1 = std::chrono::steady_clock::now();
    CK(hipStreamSynchronize(s));
    const auto t2 = std::chrono::steady_clock::now();
    const double host = std::chrono::duration<double, std::micro>(t1 - t0).count() / steps;
    const double wall = std::chrono::duration<double, std::micro>(t2 - t0).count() / steps;
    std::printf("{\"T\": %d, \"H\": %d, \"K\": %d, \"E\": %d, \"P\": %d, \"steps\": %d, "
                "\"host_us_per_step\": %.3f, \"wall_us_per_step\": %.3f}\n",
                T, H, K, E, P, steps, host, wall);
    CK(hipStreamDestroy(s));
    return 0;
}
