// dispatch.hip -- scatter-quantise each token's hidden vector into the
// receive rows of its top-k experts (gfx950).
//
// fp8 payload: per token and 128-column block, amax = max |x|,
// scale = amax / 448 (fp32), byte = e4m3fn(x / scale); the same bytes and
// scale go to every valid row of the token.  A dispatched token carries its
// hidden data and its scale factors (DeepEP PR #693 "Pipeline direct NVLink
// dispatch with triple-buffered prefetch", Summary); fp8 dispatch with bf16
// combine is the serving configuration of MoRI PR #614 "perf(ep):
// InterNodeV1LL low-token latency on MI300X + CX7" (tuned-rules paragraph).
// bf16 payload: the row is copied unchanged.
//
// Work split.  A work item is (token, 512-column step): one wave, 64 lanes,
// 16 bytes (8 bf16) per lane.  Items are strided flatly over every wave of
// the grid, so a handful of tokens still spreads over many CUs (MoRI PR #614,
// DispatchIntraNode paragraph: splitting per block over tokens starved most
// blocks at 4 tokens; MultiWarpIter paragraph: keep at least 512 elements per
// warp).  Per lane:
//   - one 16-byte load of x (global_load_dwordx4, fully coalesced);
//   - the 128-column block of a scale is one 16-lane DPP row, so amax is a
//     per-lane max over 8 values and 4 DPP max steps (quad_perm xor 1,
//     quad_perm xor 2, row_half_mirror, row_mirror), with no LDS traffic;
//   - x / scale is the IEEE-correct fp32 division; v_cvt_pk_fp8_f32 packs
//     two values per instruction (round to nearest even; a NaN-preserving
//     clamp to +-448 in front gives the saturating behaviour);
//   - K stores of 8 bytes (512 contiguous bytes per wave per row, whole
//     128-byte lines) and one 4-byte scale per 16-lane row.
// The next item's x vector and row indices are loaded before the current
// item's quantise-and-store work, so each wave keeps one load in flight
// while its stores drain (the prefetch idea of DeepEP PR #693, with a
// register double buffer instead of shared-memory TMA staging).
#include "ep_device.h"
#include "ep_launch.h"
#include "ep_numerics.h"

namespace ep {
namespace {

template <int kPayload>
__global__ __launch_bounds__(kMoveThreads) void dispatch_kernel(
    const uint16_t* __restrict__ x, int H, int K, const int32_t* __restrict__ row_of_pair,
    uint8_t* __restrict__ recv_x, float* __restrict__ recv_scales,
    int steps_per_token, int n_items, int n_rows)
{
    const int lane = threadIdx.x % kWave;
    const int stride = gridDim.x * kMoveWaves;
    const int nb = H / kScaleBlock;
    int item = blockIdx.x * kMoveWaves + wave_uniform(threadIdx.x / kWave);
    if (item >= n_items) return;

    // load stage of one item: row ids (lanes < K) and this lane's 16 bytes of x
    auto load_item = [&](int it, int& myrow, uint4& v, int& col0) {
        const int t = it / steps_per_token;
        col0 = (it - t * steps_per_token) * kStepCols + lane * kColsPerLane;
        myrow = (lane < K) ? row_of_pair[(int64_t)t * K + lane] : -1;
        v = (col0 < H) ? *reinterpret_cast<const uint4*>(x + (int64_t)t * H + col0)
                       : make_uint4(0, 0, 0, 0);
    };

    int myrow, col0;
    uint4 v;
    load_item(item, myrow, v, col0);

    while (true) {
        const int next = item + stride;      // n_items + stride < 2^31 (checked by the launcher)
        int nrow = -1, ncol0 = 0;
        uint4 nv = make_uint4(0, 0, 0, 0);
        if (next < n_items) load_item(next, nrow, nv, ncol0);

        const bool active = col0 < H;
        if constexpr (kPayload == 0) {
            float scale;
            const uint2 q = quantise_e4m3fn_block8(v, scale);
            for (int k = 0; k < K; ++k) {
                const int r = read_lane(myrow, k);
                if (r < 0 || r >= n_rows) continue;     // masked (or not a receive row)
                if (active) {
                    *reinterpret_cast<uint2*>(recv_x + (int64_t)r * H + col0) = q;
                    if ((lane % kLanesPerScaleBlock) == 0)
                        recv_scales[(int64_t)r * nb + col0 / kScaleBlock] = scale;
                }
            }
        } else {
            uint16_t* dst = reinterpret_cast<uint16_t*>(recv_x);
            for (int k = 0; k < K; ++k) {
                const int r = read_lane(myrow, k);
                if (r < 0 || r >= n_rows) continue;
                if (active) *reinterpret_cast<uint4*>(dst + (int64_t)r * H + col0) = v;
            }
        }

        if (next >= n_items) break;
        item = next;
        myrow = nrow;
        v = nv;
        col0 = ncol0;
    }
}

__global__ __launch_bounds__(256) void e4m3fn_encode_kernel(const float* __restrict__ in, int64_t n,
                                                            uint8_t* __restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = i; j < n; j += stride) out[j] = encode_e4m3fn_one(in[j]);
}

constexpr int64_t kMaxGridBlocks = 1 << 20;

}  // namespace

hipError_t launch_dispatch(const uint16_t* x, int T, int H, int K, const int32_t* row_of_pair,
                           int payload, void* recv_x, float* recv_scales, hipStream_t stream)
{
    const int steps = (H + kStepCols - 1) / kStepCols;
    const int64_t items = (int64_t)T * steps;
    if (items == 0) return hipSuccess;
    if (items + kMaxGridBlocks * kMoveWaves >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    int64_t blocks = (items + kMoveWaves - 1) / kMoveWaves;
    if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
    if (payload == 0)
        hipLaunchKernelGGL(dispatch_kernel<0>, dim3((unsigned)blocks), dim3(kMoveThreads), 0, stream,
                           x, H, K, row_of_pair, (uint8_t*)recv_x, recv_scales, steps, (int)items, T * K);
    else
        hipLaunchKernelGGL(dispatch_kernel<1>, dim3((unsigned)blocks), dim3(kMoveThreads), 0, stream,
                           x, H, K, row_of_pair, (uint8_t*)recv_x, nullptr, steps, (int)items, T * K);
    return hipGetLastError();
}

hipError_t launch_e4m3fn_encode(const float* in, int64_t n, uint8_t* out, hipStream_t stream)
{
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(e4m3fn_encode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, n, out);
    return hipGetLastError();
}

}  // namespace ep
