// ep_ceilings.cpp -- plain HBM read, write and copy rates of the GPU it runs
// on, from hand-written streaming kernels: the ceilings the dispatch and
// combine kernels are compared with.  Built with the library (hipcc -x hip),
// not part of it; no library call is made.
//
//   ep_ceilings [MiB per buffer = 1024] [launches per sample = 20] [samples = 7]
//
// Every kernel moves 16 bytes per lane per access (one dwordx4 per lane: a
// 1 KB contiguous piece per wave access), four independent accesses in flight
// per lane; the buffers are far larger than the 256 MB memory-side cache, so
// every byte comes from or goes to HBM.  Two work splits: grid-strided (timed
// at several grid sizes) and tiled (one workgroup per contiguous 16 KB tile,
// one pass, as the dispatch and combine kernels run one wave per item).  HIP
// events around back-to-back launches on one stream, after a warm-up launch;
// the JSON line gives, per kernel, the median over samples of the best form
// and the rate of every form.
//   read       sum of 16-byte loads (one word per thread written only if a
//              checksum hits an impossible value, so the loads stay)
//   read_nt    the same with nontemporal loads
//   write      16-byte stores of a pattern
//   write_nt   the same, nontemporal
//   copy       load + store (bytes counted: read + written)
//   copy_nt    load + nontemporal store
//   gather, gather_nt  the combine's access pattern at 4096 tokens x hidden
//              7168 x top-8: one wave per (token, 512-column step) loads its
//              16 bytes per lane from 8 rows of 14336 bytes spread over the
//              32768 rows (a fixed odd-multiplier permutation) and stores 16
//              bytes of the token's output row; bytes counted: 8 rows read +
//              1 row written per token, as the combine's algorithmic bytes.
//              Timed with 1, 2 and 4 waves per workgroup (cached or
//              nontemporal loads; the store is nontemporal).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#define CK(x)                                                                              \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                       \
        }                                                                                  \
    } while (0)

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;


template <bool kNt>
__device__ __forceinline__ uint4 ld(const uint4* p)
{
    if constexpr (kNt) {
        uint4 v;
        v.x = __builtin_nontemporal_load(&p->x);
        v.y = __builtin_nontemporal_load(&p->y);
        v.z = __builtin_nontemporal_load(&p->z);
        v.w = __builtin_nontemporal_load(&p->w);
        return v;
    } else {
        return *p;
    }
}

template <bool kNt>
__device__ __forceinline__ void st(uint4* p, uint4 v)
{
    if constexpr (kNt) {
        __builtin_nontemporal_store(v.x, &p->x);
        __builtin_nontemporal_store(v.y, &p->y);
        __builtin_nontemporal_store(v.z, &p->z);
        __builtin_nontemporal_store(v.w, &p->w);
    } else {
        *p = v;
    }
}

// n16 is a multiple of kUnroll * the grid's threads (the host sizes it so)
template <bool kNt>
__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                        uint32_t* __restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += kUnroll * stride) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = ld<kNt>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <bool kNt>
__global__ __launch_bounds__(kThreads) void write_kernel(uint4* __restrict__ dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += kUnroll * stride) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t k = (uint32_t)(i + u * stride);
            st<kNt>(dst + i + u * stride, make_uint4(k, k + 1u, k + 2u, k + 3u));
        }
    }
}

template <bool kNt>
__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += kUnroll * stride) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = ld<false>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) st<kNt>(dst + i + u * stride, v[u]);
    }
}

// tiled: workgroup b of kT threads moves tile b, kT * kU 16-byte pieces
// (grid = n16 / (kT * kU))
template <int kT, int kU, bool kNt>
__global__ __launch_bounds__(kT) void read_tiles(const uint4* __restrict__ src,
                                                 uint32_t* __restrict__ sink)
{
    const int64_t base = (int64_t)blockIdx.x * kT * kU + threadIdx.x;
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = ld<kNt>(src + base + u * kT);
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

template <int kT, int kU, bool kNt>
__global__ __launch_bounds__(kT) void write_tiles(uint4* __restrict__ dst)
{
    const int64_t base = (int64_t)blockIdx.x * kT * kU + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const uint32_t k = (uint32_t)(base + u * kT);
        st<kNt>(dst + base + u * kT, make_uint4(k, k + 1u, k + 2u, k + 3u));
    }
}

template <int kT, int kU, bool kNt>
__global__ __launch_bounds__(kT) void copy_tiles(const uint4* __restrict__ src,
                                                 uint4* __restrict__ dst)
{
    const int64_t base = (int64_t)blockIdx.x * kT * kU + threadIdx.x;
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = ld<false>(src + base + u * kT);
#pragma unroll
    for (int u = 0; u < kU; ++u) st<kNt>(dst + base + u * kT, v[u]);
}

// tile shapes (threads, pieces per thread), selected by negative "grid" codes
constexpr int kShapes = 5;
constexpr int kShapeT[kShapes] = {256, 256, 128, 64, 512};
constexpr int kShapeU[kShapes] = {4, 1, 1, 1, 1};

template <int kI>
struct Shape {
    static constexpr int kT = kShapeT[kI], kU = kShapeU[kI];
};

// one launcher per (operation, nontemporal) over the shapes
template <int kI, bool kNt>
void launch_tiles(int op, hipStream_t s, uint4* a, uint4* b, uint32_t* k, int64_t n)
{
    constexpr int kT = Shape<kI>::kT, kU = Shape<kI>::kU;
    const unsigned grid = (unsigned)(n / (kT * kU));
    if (op == 0) hipLaunchKernelGGL((read_tiles<kT, kU, kNt>), dim3(grid), dim3(kT), 0, s, a, k);
    if (op == 1) hipLaunchKernelGGL((write_tiles<kT, kU, kNt>), dim3(grid), dim3(kT), 0, s, b);
    if (op == 2) hipLaunchKernelGGL((copy_tiles<kT, kU, kNt>), dim3(grid), dim3(kT), 0, s, a, b);
}

template <bool kNt>
void tiles_by_shape(int shape, int op, hipStream_t s, uint4* a, uint4* b, uint32_t* k, int64_t n)
{
    switch (shape) {
    case 0: launch_tiles<0, kNt>(op, s, a, b, k, n); break;
    case 1: launch_tiles<1, kNt>(op, s, a, b, k, n); break;
    case 2: launch_tiles<2, kNt>(op, s, a, b, k, n); break;
    case 3: launch_tiles<3, kNt>(op, s, a, b, k, n); break;
    default: launch_tiles<4, kNt>(op, s, a, b, k, n); break;
    }
}

// The combine-shaped gather (see the header): rows of kRow16 16-byte pieces,
// kGatherK source rows per token, one wave per (token, 64-piece step).
constexpr int kRow16 = 7168 * 2 / 16;      // 896 pieces per row
constexpr int kGatherK = 8;
constexpr int kGatherT = 4096;
constexpr int kSteps = kRow16 / 64;        // 14
constexpr uint32_t kGatherRows = (uint32_t)kGatherT * kGatherK;   // 32768, a power of two

template <bool kNt>
__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst)
{
    const int lane = threadIdx.x % 64;
    const int item = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;   // grid covers items exactly
    const int t = item / kSteps;
    const int step = item - t * kSteps;
    uint4 v[kGatherK];
#pragma unroll
    for (int k = 0; k < kGatherK; ++k) {
        // an odd multiplier permutes [0, 2^15): every row is read exactly once
        const uint32_t row = ((uint32_t)(t * kGatherK + k) * 2654435761u) & (kGatherRows - 1u);
        v[k] = ld<kNt>(src + (int64_t)row * kRow16 + step * 64 + lane);
    }
    uint4 acc = v[0];
#pragma unroll
    for (int k = 1; k < kGatherK; ++k) {
        acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
    }
    st<true>(dst + (int64_t)t * kRow16 + step * 64 + lane, acc);
}

}  // namespace

int main(int argc, char** argv)
{
    const int64_t mib = argc > 1 ? atoll(argv[1]) : 1024;
    const int reps = argc > 2 ? atoi(argv[2]) : 20;
    const int samples = argc > 3 ? atoi(argv[3]) : 7;
    // grid-strided grid sizes, then tile shapes as -1 - shape index
    const std::vector<int> grids = {1024, 2048, 4096, 8192, 16384, -1, -2, -3, -4, -5};
    // a multiple of every grid's threads times the unroll: every access in bounds
    const int64_t quantum = (int64_t)16384 * kThreads * kUnroll;
    // (and of every tile: at most 1024 pieces)
    int64_t n16 = (mib << 20) / 16;
    n16 = n16 / quantum * quantum;
    if (n16 <= 0 || reps < 1 || samples < 1) {
        fprintf(stderr, "usage: ep_ceilings [MiB >= 256] [launches >= 1] [samples >= 1]\n");
        return 2;
    }
    const size_t bytes = (size_t)n16 * 16;
    if ((int64_t)kGatherRows * kRow16 > n16) {
        fprintf(stderr, "ep_ceilings: the gather needs buffers of at least %lld MiB\n",
                (long long)(((int64_t)kGatherRows * kRow16 * 16) >> 20) + 1);
        return 2;
    }
    uint4 *a = nullptr, *b = nullptr;
    uint32_t* sink = nullptr;
    CK(hipMalloc(&a, bytes));
    CK(hipMalloc(&b, bytes));
    CK(hipMalloc(&sink, (size_t)16384 * kThreads * 4));
    CK(hipMemset(a, 1, bytes));
    CK(hipMemset(b, 2, bytes));
    hipStream_t s;
    CK(hipStreamCreate(&s));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    CK(hipDeviceSynchronize());

    struct Kernel {
        const char* name;
        double bytes_per_launch;
        void (*launch)(int grid, hipStream_t s, uint4* a, uint4* b, uint32_t* sink, int64_t n16);
    };
    const Kernel kernels[] = {
        {"read", (double)bytes,
         [](int g, hipStream_t s, uint4* a, uint4* b, uint32_t* k, int64_t n) {
             if (g < 0) tiles_by_shape<false>(-1 - g, 0, s, a, b, k, n);
             else hipLaunchKernelGGL(read_kernel<false>, dim3(g), dim3(kThreads), 0, s, a, n, k);
         }},
        {"read_nt", (double)bytes,
         [](int g, hipStream_t s, uint4* a, uint4* b, uint32_t* k, int64_t n) {
             if (g < 0) tiles_by_shape<true>(-1 - g, 0, s, a, b, k, n);
             else hipLaunchKernelGGL(read_kernel<true>, dim3(g), dim3(kThreads), 0, s, a, n, k);
         }},
        {"write", (double)bytes,
         [](int g, hipStream_t s, uint4* a, uint4* b, uint32_t* k, int64_t n) {
             if (g < 0) tiles_by_shape<false>(-1 - g, 1, s, a, b, k, n);
             else hipLaunchKernelGGL(write_kernel<false>, dim3(g), dim3(kThreads), 0, s, b, n);
         }},
        {"write_nt", (double)bytes,
         [](int g, hipStream_t s, uint4* a, uint4* b, uint32_t* k, int64_t n) {
             if (g < 0) tiles_by_shape<true>(-1 - g, 1, s, a, b, k, n);
             else hipLaunchKernelGGL(write_kernel<true>, dim3(g), dim3(kThreads), 0, s, b, n);
         }},
        {"copy", 2.0 * (double)bytes,
         [](int g, hipStream_t s, uint4* a, uint4* b, uint32_t* k, int64_t n) {
             if (g < 0) tiles_by_shape<false>(-1 - g, 2, s, a, b, k, n);
             else hipLaunchKernelGGL(copy_kernel<false>, dim3(g), dim3(kThreads), 0, s, a, b, n);
         }},
        {"copy_nt", 2.0 * (double)bytes,
         [](int g, hipStream_t s, uint4* a, uint4* b, uint32_t* k, int64_t n) {
             if (g < 0) tiles_by_shape<true>(-1 - g, 2, s, a, b, k, n);
             else hipLaunchKernelGGL(copy_kernel<true>, dim3(g), dim3(kThreads), 0, s, a, b, n);
         }},
    };

    std::string out = "{\"ceilings_native\": {";
    bool first = true;
    for (const Kernel& k : kernels) {
        double best_med = 0.0;
        int best_grid = 0;
        std::string per_grid;
        for (int g : grids) {
            k.launch(g, s, a, b, sink, n16);   // warm-up
            CK(hipGetLastError());
            std::vector<double> gbps;
            for (int i = 0; i < samples; ++i) {
                CK(hipEventRecord(e0, s));
                for (int r = 0; r < reps; ++r) k.launch(g, s, a, b, sink, n16);
                CK(hipEventRecord(e1, s));
                CK(hipEventSynchronize(e1));
                float ms = 0.0f;
                CK(hipEventElapsedTime(&ms, e0, e1));
                gbps.push_back(k.bytes_per_launch * reps / (ms * 1e-3) / 1e9);
            }
            std::sort(gbps.begin(), gbps.end());
            const double med = gbps[gbps.size() / 2];
            char buf[96];
            if (g < 0)
                snprintf(buf, sizeof buf, "%s\"tiles %dx%d\": %.1f", per_grid.empty() ? "" : ", ",
                         kShapeT[-1 - g], kShapeU[-1 - g], med);
            else
                snprintf(buf, sizeof buf, "%s\"%d\": %.1f", per_grid.empty() ? "" : ", ", g, med);
            per_grid += buf;
            if (med > best_med) { best_med = med; best_grid = g; }
        }
        char buf[256];
        if (best_grid < 0)
            snprintf(buf, sizeof buf, "%s\"%s\": {\"GBps\": %.1f, \"form\": \"tiles %dx%d\", \"by_form\": {",
                     first ? "" : ", ", k.name, best_med, kShapeT[-1 - best_grid], kShapeU[-1 - best_grid]);
        else
            snprintf(buf, sizeof buf, "%s\"%s\": {\"GBps\": %.1f, \"form\": \"grid %d\", \"by_form\": {",
                     first ? "" : ", ", k.name, best_med, best_grid);
        out += buf;
        out += per_grid + "}}";
        first = false;
        fprintf(stderr, "%s done\n", k.name);
    }
    // the combine-shaped gather: 1, 2 and 4 waves per workgroup
    const int items = kGatherT * kSteps;
    const double gather_bytes = (double)(kGatherRows + kGatherT) * kRow16 * 16;
    for (int nt = 0; nt < 2; ++nt) {
        double best_med = 0.0;
        int best_w = 0;
        std::string per_form;
        for (int w : {1, 2, 4}) {
            auto launch = [&]() {
                if (nt) hipLaunchKernelGGL(gather_kernel<true>, dim3(items / w), dim3(64 * w), 0, s, a, b);
                else hipLaunchKernelGGL(gather_kernel<false>, dim3(items / w), dim3(64 * w), 0, s, a, b);
            };
            launch();   // warm-up
            CK(hipGetLastError());
            std::vector<double> gbps;
            for (int i = 0; i < samples; ++i) {
                CK(hipEventRecord(e0, s));
                for (int r = 0; r < reps; ++r) launch();
                CK(hipEventRecord(e1, s));
                CK(hipEventSynchronize(e1));
                float ms = 0.0f;
                CK(hipEventElapsedTime(&ms, e0, e1));
                gbps.push_back(gather_bytes * reps / (ms * 1e-3) / 1e9);
            }
            std::sort(gbps.begin(), gbps.end());
            const double med = gbps[gbps.size() / 2];
            char buf[96];
            snprintf(buf, sizeof buf, "%s\"%d waves\": %.1f", per_form.empty() ? "" : ", ", w, med);
            per_form += buf;
            if (med > best_med) { best_med = med; best_w = w; }
        }
        char buf[256];
        snprintf(buf, sizeof buf, ", \"%s\": {\"GBps\": %.1f, \"form\": \"%d waves\", \"by_form\": {",
                 nt ? "gather_nt" : "gather", best_med, best_w);
        out += buf;
        out += per_form + "}}";
        fprintf(stderr, "%s done\n", nt ? "gather_nt" : "gather");
    }
    char tail[160];
    snprintf(tail, sizeof tail,
             "}, \"buffer_MiB\": %lld, \"launches_per_sample\": %d, \"samples\": %d, \"threads\": %d}",
             (long long)(bytes >> 20), reps, samples, kThreads);
    out += tail;
    printf("%s\n", out.c_str());
    CK(hipFree(a));
    CK(hipFree(b));
    CK(hipFree(sink));
    return 0;
}
