// api.hip -- the C entry points declared in include/ep.h: argument checks,
// launches, error reporting and HIP graph capture helpers.
//
// Every check runs on the host before anything is enqueued, so a rejected
// call leaves the stream untouched (configuration errors are refused early
// and loudly, as the tuning CLI of MoRI PR #614 "perf(ep): InterNodeV1LL
// low-token latency on MI300X + CX7" does for its environment knobs).
#include <mutex>

#include "ep.h"
#include "ep_device.h"
#include "ep_launch.h"

static_assert(ep::kFusedTiny == EP_PLAN_FUSED_TINY && ep::kFusedCount == EP_PLAN_FUSED_COUNT &&
                  ep::kFusedGeneral == EP_PLAN_FUSED_GENERAL,
              "the plan codes of the header are the launcher's kernel kinds");

namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool ptr_ok(const void* p, uintptr_t a) { return p != nullptr && aligned(p, a); }

int from_hip(hipError_t e)
{
    if (e == hipSuccess) return EP_OK;
    g_last_hip_error = (int)e;
    return EP_EHIP;
}

bool routing_ok(int T, int K)
{
    return T >= 0 && K >= 1 && K <= EP_MAX_TOPK && (int64_t)T * K < ((int64_t)1 << 31);
}

bool dedup_ok(int T, int P)
{
    return T >= 0 && P >= 1 && P <= EP_MAX_DEDUP_PARTITIONS && (int64_t)T * P < ((int64_t)1 << 31);
}

}  // namespace

extern "C" {

size_t ep_layout_workspace_bytes(int T, int K, int E)
{
    if (!routing_ok(T, K) || E < 1 || E > EP_MAX_EXPERTS) return 0;
    return ep::layout_workspace_bytes(T, K, E);
}

int ep_layout(const int32_t* topk_idx, int T, int K, int E, int P,
              int32_t* expert_count, int32_t* expert_offset, int32_t* part_count,
              int32_t* part_offset, int32_t* row_of_pair, int32_t* src_pair, uint32_t* status,
              void* ws, size_t ws_bytes, void* stream)
{
    if (!routing_ok(T, K) || E < 1 || E > EP_MAX_EXPERTS || P < 1 || E % P != 0) return EP_EINVAL;
    if (!ptr_ok(expert_count, 4) || !ptr_ok(expert_offset, 4) || !ptr_ok(part_count, 4) ||
        !ptr_ok(part_offset, 4) || !ptr_ok(status, 4))
        return EP_EINVAL;
    if (T > 0 && (!ptr_ok(topk_idx, 4) || !ptr_ok(row_of_pair, 4) || !ptr_ok(src_pair, 4)))
        return EP_EINVAL;
    const size_t need = ep::layout_workspace_bytes(T, K, E);
    if (need > 0 && (ws_bytes < need || !ptr_ok(ws, 16))) return EP_EINVAL;
    return from_hip(ep::launch_layout(topk_idx, T, K, E, P, expert_count, expert_offset, part_count,
                                      part_offset, row_of_pair, src_pair, status, ws,
                                      (hipStream_t)stream));
}

int ep_dispatch(const uint16_t* x, int T, int H, int K, const int32_t* row_of_pair, int payload,
                void* recv_x, float* recv_scales, void* stream)
{
    if (payload != EP_PAYLOAD_FP8_E4M3FN && payload != EP_PAYLOAD_BF16) return EP_ENOTSUP;
    if (!routing_ok(T, K) || H <= 0) return EP_EINVAL;
    if (payload == EP_PAYLOAD_FP8_E4M3FN && H % ep::kScaleBlock != 0) return EP_EINVAL;
    if (payload == EP_PAYLOAD_BF16 && H % ep::kColsPerLane != 0) return EP_EINVAL;
    if (T == 0) return EP_OK;
    if (!ptr_ok(x, 16) || !ptr_ok(row_of_pair, 4) || !ptr_ok(recv_x, 16)) return EP_EINVAL;
    if (payload == EP_PAYLOAD_FP8_E4M3FN && !ptr_ok(recv_scales, 4)) return EP_EINVAL;
    if (!ep::dispatch_launch_ok(T, H, ep::kDefaultGeometry)) return EP_EINVAL;
    return from_hip(ep::launch_dispatch(x, T, H, K, row_of_pair, payload, recv_x, recv_scales,
                                        (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Launch geometry from the API's (waves_per_block, max_blocks, slice_cols);
// 0 means the default for each.  False for values the kernels do not take.
bool move_geometry(int waves_per_block, int max_blocks, int slice_cols, ep::MoveGeometry* g)
{
    if (waves_per_block == 0) waves_per_block = ep::kDefaultGeometry.waves;
    if (slice_cols == 0) slice_cols = ep::kStepCols;
    if (waves_per_block != 1 && waves_per_block != 2 && waves_per_block != 4 &&
        waves_per_block != 8)
        return false;
    if (max_blocks < 0) return false;
    if (slice_cols != ep::kStepCols && slice_cols != ep::kMaxSliceSteps * ep::kStepCols) return false;
    *g = ep::MoveGeometry{waves_per_block, max_blocks, slice_cols / ep::kStepCols};
    return true;
}

// How ep_layout_dispatch(_geom) runs a batch: fused (one launch, plan) or
// the layout then the dispatch kernel with geometry g.  False when the
// geometry is not accepted for this batch.
bool layout_dispatch_route(int T, int H, int K, int waves_per_block, int max_blocks,
                           int slice_cols, bool* fused, ep::FusedPlan* plan, ep::MoveGeometry* g)
{
    *fused = T > 0 && ep::fused_layout_dispatch_fits(T, H, K);
    if (*fused) {
        // the fused kernels take only a workgroup size
        if (max_blocks != 0 || (slice_cols != 0 && slice_cols != ep::kStepCols)) return false;
        return ep::plan_layout_dispatch(T, H, K, waves_per_block, plan);
    }
    if (!move_geometry(waves_per_block, max_blocks, slice_cols, g)) return false;
    return T == 0 || ep::dispatch_launch_ok(T, H, *g);
}

// The launches of ep_layout_dispatch(_geom), for a workspace ws of ws_bytes
// (the caller's, or the library's scratch buffer); every check is made
// before the first launch.
int layout_dispatch_checked(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K, int E,
                            int P, int payload, int32_t* expert_count, int32_t* expert_offset,
                            int32_t* part_count, int32_t* part_offset, int32_t* row_of_pair,
                            int32_t* src_pair, uint32_t* status, void* ws, size_t ws_bytes,
                            void* recv_x, float* recv_scales, int waves_per_block, int max_blocks,
                            int slice_cols, void* stream)
{
    const size_t need = ep::layout_workspace_bytes(T, K, E);
    if (need > 0 && (ws_bytes < need || !ptr_ok(ws, 16))) return EP_EINVAL;
    bool fused = false;
    ep::FusedPlan plan{};
    ep::MoveGeometry g = ep::kDefaultGeometry;
    if (!layout_dispatch_route(T, H, K, waves_per_block, max_blocks, slice_cols, &fused, &plan, &g))
        return EP_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (fused)
        return from_hip(ep::launch_layout_dispatch(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                                   expert_offset, part_count, part_offset,
                                                   row_of_pair, src_pair, status, recv_x,
                                                   recv_scales, s, plan.waves));
    int rc = from_hip(ep::launch_layout(topk_idx, T, K, E, P, expert_count, expert_offset,
                                        part_count, part_offset, row_of_pair, src_pair, status,
                                        ws, s));
    if (rc != EP_OK || T == 0) return rc;
    return from_hip(ep::launch_dispatch(x, T, H, K, row_of_pair, payload, recv_x, recv_scales, s, g));
}

// Argument checks of ep_layout_dispatch that do not involve the workspace.
int layout_dispatch_args(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K, int E,
                         int P, int payload, int32_t* expert_count, int32_t* expert_offset,
                         int32_t* part_count, int32_t* part_offset, int32_t* row_of_pair,
                         int32_t* src_pair, uint32_t* status, void* recv_x, float* recv_scales)
{
    if (payload != EP_PAYLOAD_FP8_E4M3FN && payload != EP_PAYLOAD_BF16) return EP_ENOTSUP;
    if (!routing_ok(T, K) || E < 1 || E > EP_MAX_EXPERTS || P < 1 || E % P != 0 || H <= 0)
        return EP_EINVAL;
    if (payload == EP_PAYLOAD_FP8_E4M3FN && H % ep::kScaleBlock != 0) return EP_EINVAL;
    if (payload == EP_PAYLOAD_BF16 && H % ep::kColsPerLane != 0) return EP_EINVAL;
    if (!ptr_ok(expert_count, 4) || !ptr_ok(expert_offset, 4) || !ptr_ok(part_count, 4) ||
        !ptr_ok(part_offset, 4) || !ptr_ok(status, 4))
        return EP_EINVAL;
    if (T > 0) {
        if (!ptr_ok(topk_idx, 4) || !ptr_ok(row_of_pair, 4) || !ptr_ok(src_pair, 4) ||
            !ptr_ok(x, 16) || !ptr_ok(recv_x, 16))
            return EP_EINVAL;
        if (payload == EP_PAYLOAD_FP8_E4M3FN && !ptr_ok(recv_scales, 4)) return EP_EINVAL;
    }
    return EP_OK;
}

}  // namespace

// ---- the no-allocation variant's scratch buffer ----------------------------
// The layout workspace of ep_layout_dispatch_noalloc: a device array of the
// library's own, one copy per device (each at its own address), held until
// the process ends.  Host code never uses the name `scratch` as an address
// (on the host it is only a stand-in for the symbol): the device address is
// looked up once per device with hipGetSymbolAddress and kept in
// g_scratch_addr, and only that address reaches a kernel.
static __device__ __align__(256) unsigned char scratch[EP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices];       // null: not looked up on that device yet

// Device address of `scratch` on the current device, which must be the
// stream's device; looked up on the first call for that device.
int scratch_address(void* stream, void** addr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e);
    if (dev < 0 || dev >= kMaxDevices) return EP_EINVAL;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess) return from_hip(e);
        if (sdev != dev) return EP_EINVAL;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return from_hip(e);
        if (p == nullptr) return EP_EINVAL;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return EP_OK;
}

}  // namespace

extern "C" {

int ep_layout_dispatch(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K, int E,
                       int P, int payload, int32_t* expert_count, int32_t* expert_offset,
                       int32_t* part_count, int32_t* part_offset, int32_t* row_of_pair,
                       int32_t* src_pair, uint32_t* status, void* ws, size_t ws_bytes,
                       void* recv_x, float* recv_scales, void* stream)
{
    const int rc = layout_dispatch_args(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                        expert_offset, part_count, part_offset, row_of_pair,
                                        src_pair, status, recv_x, recv_scales);
    if (rc != EP_OK) return rc;
    return layout_dispatch_checked(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                   expert_offset, part_count, part_offset, row_of_pair, src_pair,
                                   status, ws, ws_bytes, recv_x, recv_scales, 0, 0, 0, stream);
}

int ep_layout_dispatch_geom(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K, int E,
                            int P, int payload, int32_t* expert_count, int32_t* expert_offset,
                            int32_t* part_count, int32_t* part_offset, int32_t* row_of_pair,
                            int32_t* src_pair, uint32_t* status, void* ws, size_t ws_bytes,
                            void* recv_x, float* recv_scales, int waves_per_block, int max_blocks,
                            int slice_cols, void* stream)
{
    const int rc = layout_dispatch_args(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                        expert_offset, part_count, part_offset, row_of_pair,
                                        src_pair, status, recv_x, recv_scales);
    if (rc != EP_OK) return rc;
    return layout_dispatch_checked(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                   expert_offset, part_count, part_offset, row_of_pair, src_pair,
                                   status, ws, ws_bytes, recv_x, recv_scales, waves_per_block,
                                   max_blocks, slice_cols, stream);
}

int ep_layout_dispatch_plan(int T, int H, int K, int E, int P, int payload, int waves_per_block,
                            int max_blocks, int slice_cols, int32_t* plan)
{
    if (plan == nullptr) return EP_EINVAL;
    if (payload != EP_PAYLOAD_FP8_E4M3FN && payload != EP_PAYLOAD_BF16) return EP_ENOTSUP;
    if (!routing_ok(T, K) || E < 1 || E > EP_MAX_EXPERTS || P < 1 || E % P != 0 || H <= 0)
        return EP_EINVAL;
    if (payload == EP_PAYLOAD_FP8_E4M3FN && H % ep::kScaleBlock != 0) return EP_EINVAL;
    if (payload == EP_PAYLOAD_BF16 && H % ep::kColsPerLane != 0) return EP_EINVAL;
    bool fused = false;
    ep::FusedPlan fp{};
    ep::MoveGeometry g = ep::kDefaultGeometry;
    if (!layout_dispatch_route(T, H, K, waves_per_block, max_blocks, slice_cols, &fused, &fp, &g))
        return EP_EINVAL;
    if (fused) {
        plan[0] = fp.kind;
        plan[1] = fp.waves;
        plan[2] = (int32_t)fp.blocks;
        plan[3] = ep::kStepCols;
    } else {
        plan[0] = EP_PLAN_LAYOUT_THEN_DISPATCH;
        plan[1] = g.waves;
        plan[2] = g.max_blocks;
        plan[3] = g.slice_steps * ep::kStepCols;
    }
    return EP_OK;
}

int ep_layout_dispatch_noalloc(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K,
                               int E, int P, int payload, int32_t* expert_count,
                               int32_t* expert_offset, int32_t* part_count, int32_t* part_offset,
                               int32_t* row_of_pair, int32_t* src_pair, uint32_t* status,
                               void* recv_x, float* recv_scales, void* stream)
{
    int rc = layout_dispatch_args(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                  expert_offset, part_count, part_offset, row_of_pair, src_pair,
                                  status, recv_x, recv_scales);
    if (rc != EP_OK) return rc;
    const size_t need = ep::layout_workspace_bytes(T, K, E);
    if (need > EP_NOALLOC_SCRATCH_BYTES) return EP_ESCRATCH;     // before any HIP call
    void* ws = nullptr;
    if (need > 0) {
        rc = scratch_address(stream, &ws);
        if (rc != EP_OK) return rc;
    }
    return layout_dispatch_checked(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                   expert_offset, part_count, part_offset, row_of_pair, src_pair,
                                   status, ws, need > 0 ? (size_t)EP_NOALLOC_SCRATCH_BYTES : 0,
                                   recv_x, recv_scales, 0, 0, 0, stream);
}

int ep_dispatch_geom(const uint16_t* x, int T, int H, int K, const int32_t* row_of_pair,
                     int payload, void* recv_x, float* recv_scales, int waves_per_block,
                     int max_blocks, int slice_cols, void* stream)
{
    ep::MoveGeometry g;
    if (waves_per_block == 0 || !move_geometry(waves_per_block, max_blocks, slice_cols, &g))
        return EP_EINVAL;
    if (payload != EP_PAYLOAD_FP8_E4M3FN && payload != EP_PAYLOAD_BF16) return EP_ENOTSUP;
    if (!routing_ok(T, K) || H <= 0) return EP_EINVAL;
    if (payload == EP_PAYLOAD_FP8_E4M3FN && H % ep::kScaleBlock != 0) return EP_EINVAL;
    if (payload == EP_PAYLOAD_BF16 && H % ep::kColsPerLane != 0) return EP_EINVAL;
    if (T == 0) return EP_OK;
    if (!ptr_ok(x, 16) || !ptr_ok(row_of_pair, 4) || !ptr_ok(recv_x, 16)) return EP_EINVAL;
    if (payload == EP_PAYLOAD_FP8_E4M3FN && !ptr_ok(recv_scales, 4)) return EP_EINVAL;
    if (!ep::dispatch_launch_ok(T, H, g)) return EP_EINVAL;
    return from_hip(ep::launch_dispatch(x, T, H, K, row_of_pair, payload, recv_x, recv_scales,
                                        (hipStream_t)stream, g));
}

int ep_combine_geom(const uint16_t* expert_out, const int32_t* row_of_pair, const float* topk_w,
                    int T, int H, int K, uint16_t* out, int waves_per_block, int max_blocks,
                    int slice_cols, void* stream)
{
    ep::MoveGeometry g;
    if (waves_per_block == 0 || !move_geometry(waves_per_block, max_blocks, slice_cols, &g))
        return EP_EINVAL;
    if (!routing_ok(T, K) || H <= 0 || H % ep::kColsPerLane != 0) return EP_EINVAL;
    if (T == 0) return EP_OK;
    if (!ptr_ok(expert_out, 16) || !ptr_ok(row_of_pair, 4) || !ptr_ok(topk_w, 4) || !ptr_ok(out, 16))
        return EP_EINVAL;
    if (!ep::combine_launch_ok(T, H, g)) return EP_EINVAL;
    return from_hip(ep::launch_combine(expert_out, row_of_pair, topk_w, T, H, K, out,
                                       (hipStream_t)stream, g));
}

int ep_combine(const uint16_t* expert_out, const int32_t* row_of_pair, const float* topk_w, int T,
               int H, int K, uint16_t* out, void* stream)
{
    if (!routing_ok(T, K) || H <= 0 || H % ep::kColsPerLane != 0) return EP_EINVAL;
    if (T == 0) return EP_OK;
    if (!ptr_ok(expert_out, 16) || !ptr_ok(row_of_pair, 4) || !ptr_ok(topk_w, 4) || !ptr_ok(out, 16))
        return EP_EINVAL;
    const ep::MoveGeometry g = ep::combine_default_geometry(T, H, K);
    if (!ep::combine_launch_ok(T, H, g)) return EP_EINVAL;
    return from_hip(ep::launch_combine(expert_out, row_of_pair, topk_w, T, H, K, out,
                                       (hipStream_t)stream, g));
}

int ep_combine_plan(int T, int H, int K, int waves_per_block, int max_blocks, int slice_cols,
                    int32_t* plan)
{
    if (plan == nullptr) return EP_EINVAL;
    if (!routing_ok(T, K) || H <= 0 || H % ep::kColsPerLane != 0) return EP_EINVAL;
    ep::MoveGeometry g = ep::combine_default_geometry(T, H, K);
    if (waves_per_block != 0) {
        if (!move_geometry(waves_per_block, max_blocks, slice_cols, &g)) return EP_EINVAL;
    } else if (max_blocks != 0 || slice_cols != 0) {
        return EP_EINVAL;
    }
    if (T > 0 && !ep::combine_launch_ok(T, H, g)) return EP_EINVAL;
    plan[0] = g.waves;
    plan[1] = g.max_blocks;
    plan[2] = g.slice_steps * ep::kStepCols;
    plan[3] = ep::combine_streaming(T, H, K) ? 1 : 0;
    return EP_OK;
}

size_t ep_dedup_layout_workspace_bytes(int T, int K, int E, int P)
{
    if (!routing_ok(T, K) || !dedup_ok(T, P) || E < 1 || E > EP_MAX_EXPERTS || E % P != 0) return 0;
    return ep::dedup_layout_workspace_bytes(T, P);
}

int ep_dedup_layout(const int32_t* topk_idx, int T, int K, int E, int P, int32_t* tp_row,
                    int32_t* part_tokens, int32_t* part_token_offset, int32_t* tp_src,
                    uint32_t* kmask, uint32_t* status, void* ws, size_t ws_bytes, void* stream)
{
    if (!routing_ok(T, K) || !dedup_ok(T, P) || E < 1 || E > EP_MAX_EXPERTS || E % P != 0)
        return EP_EINVAL;
    if (!ptr_ok(part_tokens, 4) || !ptr_ok(part_token_offset, 4) || !ptr_ok(status, 4))
        return EP_EINVAL;
    if (T > 0 && (!ptr_ok(topk_idx, 4) || !ptr_ok(tp_row, 4) || !ptr_ok(tp_src, 4) ||
                  !ptr_ok(kmask, 4)))
        return EP_EINVAL;
    const size_t need = ep::dedup_layout_workspace_bytes(T, P);
    if (need > 0 && (ws_bytes < need || !ptr_ok(ws, 16))) return EP_EINVAL;
    return from_hip(ep::launch_dedup_layout(topk_idx, T, K, E, P, tp_row, part_tokens,
                                            part_token_offset, tp_src, kmask, status, ws,
                                            (hipStream_t)stream));
}

size_t ep_dedup_layout_dispatch_workspace_bytes(int T, int K, int E, int P)
{
    if (!routing_ok(T, K) || !dedup_ok(T, P) || E < 1 || E > EP_MAX_EXPERTS || E % P != 0) return 0;
    const size_t a = ep::layout_workspace_bytes(T, K, E);
    const size_t b = ep::dedup_layout_workspace_bytes(T, P);
    return a > b ? a : b;
}

namespace {

// Argument checks of ep_dedup_layout_dispatch(_geom) that involve neither the
// workspace nor the geometry.
int dedup_layout_dispatch_args(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K,
                               int E, int P, int payload, int32_t* expert_count,
                               int32_t* expert_offset, int32_t* part_count, int32_t* part_offset,
                               int32_t* row_of_pair, int32_t* src_pair, int32_t* tp_row,
                               int32_t* part_tokens, int32_t* part_token_offset, int32_t* tp_src,
                               uint32_t* kmask, uint32_t* status, void* recv_x, float* recv_scales)
{
    if (payload != EP_PAYLOAD_FP8_E4M3FN && payload != EP_PAYLOAD_BF16) return EP_ENOTSUP;
    if (!routing_ok(T, K) || !dedup_ok(T, P) || E < 1 || E > EP_MAX_EXPERTS || E % P != 0 || H <= 0)
        return EP_EINVAL;
    if (payload == EP_PAYLOAD_FP8_E4M3FN && H % ep::kScaleBlock != 0) return EP_EINVAL;
    if (payload == EP_PAYLOAD_BF16 && H % ep::kColsPerLane != 0) return EP_EINVAL;
    if (!ptr_ok(expert_count, 4) || !ptr_ok(expert_offset, 4) || !ptr_ok(part_count, 4) ||
        !ptr_ok(part_offset, 4) || !ptr_ok(part_tokens, 4) || !ptr_ok(part_token_offset, 4) ||
        !ptr_ok(status, 4))
        return EP_EINVAL;
    if (T > 0) {
        if (!ptr_ok(topk_idx, 4) || !ptr_ok(row_of_pair, 4) || !ptr_ok(src_pair, 4) ||
            !ptr_ok(tp_row, 4) || !ptr_ok(tp_src, 4) || !ptr_ok(kmask, 4) || !ptr_ok(x, 16) ||
            !ptr_ok(recv_x, 16))
            return EP_EINVAL;
        if (payload == EP_PAYLOAD_FP8_E4M3FN && !ptr_ok(recv_scales, 4)) return EP_EINVAL;
    }
    return EP_OK;
}

// Which path a dedup batch takes and its geometry: the fused kernels (a
// workgroup size only) or the two layouts then the dispatch to the couple
// rows (K = P entries per token over tp_row) with the dispatch geometry.
bool dedup_layout_dispatch_route(int T, int H, int K, int P, int waves_per_block, int max_blocks,
                                 int slice_cols, bool* fused, ep::FusedPlan* plan,
                                 ep::MoveGeometry* g)
{
    *fused = T > 0 && ep::fused_layout_dispatch_fits(T, H, K);
    if (*fused) {
        if (max_blocks != 0 || (slice_cols != 0 && slice_cols != ep::kStepCols)) return false;
        return ep::plan_dedup_layout_dispatch(T, H, K, P, waves_per_block, plan);
    }
    if (!move_geometry(waves_per_block, max_blocks, slice_cols, g)) return false;
    return T == 0 || ep::dispatch_launch_ok(T, H, *g);
}

int dedup_layout_dispatch_checked(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K,
                                  int E, int P, int payload, int32_t* expert_count,
                                  int32_t* expert_offset, int32_t* part_count,
                                  int32_t* part_offset, int32_t* row_of_pair, int32_t* src_pair,
                                  int32_t* tp_row, int32_t* part_tokens,
                                  int32_t* part_token_offset, int32_t* tp_src, uint32_t* kmask,
                                  uint32_t* status, void* ws, size_t ws_bytes, void* recv_x,
                                  float* recv_scales, int waves_per_block, int max_blocks,
                                  int slice_cols, void* stream)
{
    const size_t need = ep_dedup_layout_dispatch_workspace_bytes(T, K, E, P);
    if (need > 0 && (ws_bytes < need || !ptr_ok(ws, 16))) return EP_EINVAL;
    bool fused = false;
    ep::FusedPlan plan{};
    ep::MoveGeometry g = ep::kDefaultGeometry;
    if (!dedup_layout_dispatch_route(T, H, K, P, waves_per_block, max_blocks, slice_cols, &fused,
                                     &plan, &g))
        return EP_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (fused)
        return from_hip(ep::launch_dedup_layout_dispatch(
            topk_idx, x, T, H, K, E, P, payload, expert_count, expert_offset, part_count,
            part_offset, row_of_pair, src_pair, tp_row, part_tokens, part_token_offset, tp_src,
            kmask, status, recv_x, recv_scales, s, plan.waves));
    // larger batches: the two layouts one after the other on the stream (they
    // share the workspace), then the dispatch to the dedup rows
    int rc = from_hip(ep::launch_layout(topk_idx, T, K, E, P, expert_count, expert_offset,
                                        part_count, part_offset, row_of_pair, src_pair, status,
                                        ws, s));
    if (rc != EP_OK) return rc;
    rc = from_hip(ep::launch_dedup_layout(topk_idx, T, K, E, P, tp_row, part_tokens,
                                          part_token_offset, tp_src, kmask, status, ws, s));
    if (rc != EP_OK || T == 0) return rc;
    return from_hip(ep::launch_dispatch(x, T, H, P, tp_row, payload, recv_x, recv_scales, s, g));
}

}  // namespace

int ep_dedup_layout_dispatch(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K, int E,
                             int P, int payload, int32_t* expert_count, int32_t* expert_offset,
                             int32_t* part_count, int32_t* part_offset, int32_t* row_of_pair,
                             int32_t* src_pair, int32_t* tp_row, int32_t* part_tokens,
                             int32_t* part_token_offset, int32_t* tp_src, uint32_t* kmask,
                             uint32_t* status, void* ws, size_t ws_bytes, void* recv_x,
                             float* recv_scales, void* stream)
{
    const int rc = dedup_layout_dispatch_args(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                              expert_offset, part_count, part_offset, row_of_pair,
                                              src_pair, tp_row, part_tokens, part_token_offset,
                                              tp_src, kmask, status, recv_x, recv_scales);
    if (rc != EP_OK) return rc;
    return dedup_layout_dispatch_checked(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                         expert_offset, part_count, part_offset, row_of_pair,
                                         src_pair, tp_row, part_tokens, part_token_offset, tp_src,
                                         kmask, status, ws, ws_bytes, recv_x, recv_scales, 0, 0, 0,
                                         stream);
}

int ep_dedup_layout_dispatch_geom(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K,
                                  int E, int P, int payload, int32_t* expert_count,
                                  int32_t* expert_offset, int32_t* part_count,
                                  int32_t* part_offset, int32_t* row_of_pair, int32_t* src_pair,
                                  int32_t* tp_row, int32_t* part_tokens,
                                  int32_t* part_token_offset, int32_t* tp_src, uint32_t* kmask,
                                  uint32_t* status, void* ws, size_t ws_bytes, void* recv_x,
                                  float* recv_scales, int waves_per_block, int max_blocks,
                                  int slice_cols, void* stream)
{
    const int rc = dedup_layout_dispatch_args(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                              expert_offset, part_count, part_offset, row_of_pair,
                                              src_pair, tp_row, part_tokens, part_token_offset,
                                              tp_src, kmask, status, recv_x, recv_scales);
    if (rc != EP_OK) return rc;
    return dedup_layout_dispatch_checked(topk_idx, x, T, H, K, E, P, payload, expert_count,
                                         expert_offset, part_count, part_offset, row_of_pair,
                                         src_pair, tp_row, part_tokens, part_token_offset, tp_src,
                                         kmask, status, ws, ws_bytes, recv_x, recv_scales,
                                         waves_per_block, max_blocks, slice_cols, stream);
}

int ep_dedup_layout_dispatch_plan(int T, int H, int K, int E, int P, int payload,
                                  int waves_per_block, int max_blocks, int slice_cols,
                                  int32_t* plan)
{
    if (plan == nullptr) return EP_EINVAL;
    if (payload != EP_PAYLOAD_FP8_E4M3FN && payload != EP_PAYLOAD_BF16) return EP_ENOTSUP;
    if (!routing_ok(T, K) || !dedup_ok(T, P) || E < 1 || E > EP_MAX_EXPERTS || E % P != 0 || H <= 0)
        return EP_EINVAL;
    if (payload == EP_PAYLOAD_FP8_E4M3FN && H % ep::kScaleBlock != 0) return EP_EINVAL;
    if (payload == EP_PAYLOAD_BF16 && H % ep::kColsPerLane != 0) return EP_EINVAL;
    bool fused = false;
    ep::FusedPlan fp{};
    ep::MoveGeometry g = ep::kDefaultGeometry;
    if (!dedup_layout_dispatch_route(T, H, K, P, waves_per_block, max_blocks, slice_cols, &fused,
                                     &fp, &g))
        return EP_EINVAL;
    if (fused) {
        plan[0] = fp.kind;
        plan[1] = fp.waves;
        plan[2] = (int32_t)fp.blocks;
        plan[3] = ep::kStepCols;
    } else {
        plan[0] = EP_PLAN_LAYOUT_THEN_DISPATCH;
        plan[1] = g.waves;
        plan[2] = g.max_blocks;
        plan[3] = g.slice_steps * ep::kStepCols;
    }
    return EP_OK;
}

int ep_combine_partial(const uint16_t* expert_out, const int32_t* row_of_pair,
                       const float* topk_w, const int32_t* tp_row, const uint32_t* kmask, int T,
                       int H, int K, int P, uint16_t* partial, void* stream)
{
    if (!routing_ok(T, K) || !dedup_ok(T, P) || H <= 0 || H % ep::kColsPerLane != 0)
        return EP_EINVAL;
    if (T == 0) return EP_OK;
    if (!ptr_ok(expert_out, 16) || !ptr_ok(row_of_pair, 4) || !ptr_ok(topk_w, 4) ||
        !ptr_ok(tp_row, 4) || !ptr_ok(kmask, 4) || !ptr_ok(partial, 16))
        return EP_EINVAL;
    if (!ep::combine_launch_ok(T, H, ep::kDefaultGeometry)) return EP_EINVAL;
    return from_hip(ep::launch_combine_partial(expert_out, row_of_pair, topk_w, tp_row, kmask, T, H,
                                               K, P, partial, (hipStream_t)stream));
}

int ep_combine_reduce(const uint16_t* partial, const int32_t* tp_row, int T, int H, int P,
                      uint16_t* out, void* stream)
{
    if (!dedup_ok(T, P) || H <= 0 || H % ep::kColsPerLane != 0) return EP_EINVAL;
    if (T == 0) return EP_OK;
    if (!ptr_ok(partial, 16) || !ptr_ok(tp_row, 4) || !ptr_ok(out, 16)) return EP_EINVAL;
    if (!ep::combine_launch_ok(T, H, ep::kDefaultGeometry)) return EP_EINVAL;
    return from_hip(ep::launch_combine_reduce(partial, tp_row, T, H, P, out, (hipStream_t)stream));
}

int ep_e4m3fn_encode(const float* in, int64_t n, uint8_t* out, void* stream)
{
    if (n < 0) return EP_EINVAL;
    if (n == 0) return EP_OK;
    if (!ptr_ok(in, 4) || out == nullptr) return EP_EINVAL;
    return from_hip(ep::launch_e4m3fn_encode(in, n, out, (hipStream_t)stream));
}

int ep_topk_idx_narrow(const int64_t* topk_idx64, int64_t n, int32_t* topk_idx32, void* stream)
{
    if (n < 0) return EP_EINVAL;
    if (n == 0) return EP_OK;
    if (!ptr_ok(topk_idx64, 8) || !ptr_ok(topk_idx32, 4)) return EP_EINVAL;
    return from_hip(ep::launch_idx_narrow(topk_idx64, n, topk_idx32, (hipStream_t)stream));
}

int ep_graph_begin(void* stream)
{
    if (stream == nullptr) return EP_EINVAL;
    return from_hip(hipStreamBeginCapture((hipStream_t)stream, hipStreamCaptureModeThreadLocal));
}

int ep_graph_end(void* stream, void** graph)
{
    if (stream == nullptr || graph == nullptr) return EP_EINVAL;
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture((hipStream_t)stream, &g);
    if (e != hipSuccess) return from_hip(e);
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e != hipSuccess) return from_hip(e);
    *graph = (void*)exec;
    return EP_OK;
}

int ep_graph_launch(void* graph, void* stream)
{
    if (graph == nullptr) return EP_EINVAL;
    return from_hip(hipGraphLaunch((hipGraphExec_t)graph, (hipStream_t)stream));
}

int ep_graph_destroy(void* graph)
{
    if (graph == nullptr) return EP_EINVAL;
    return from_hip(hipGraphExecDestroy((hipGraphExec_t)graph));
}

const char* ep_strerror(int code)
{
    switch (code) {
    case EP_OK: return "ok";
    case EP_EINVAL: return "invalid argument (size, divisibility, null or misaligned pointer, workspace)";
    case EP_ENOTSUP: return "unsupported payload";
    case EP_EHIP: return "HIP launch failed (see ep_last_hip_error)";
    case EP_ESCRATCH:
        return "batch needs a larger layout workspace than the library's no-allocation scratch "
               "buffer (EP_NOALLOC_SCRATCH_BYTES); use ep_layout_dispatch with a workspace";
    default: return "unknown ep error code";
    }
}

int ep_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
