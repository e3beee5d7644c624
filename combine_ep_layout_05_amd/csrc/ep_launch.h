// ep_launch.h -- host-side launchers of the kernels (one per .hip file).
// Arguments are validated by the C entry points before these are called;
// each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep_device.h"

namespace ep {

size_t layout_workspace_bytes(int T, int K, int E);

hipError_t launch_layout(const int32_t* topk_idx, int T, int K, int E, int P,
                         int32_t* expert_count, int32_t* expert_offset,
                         int32_t* part_count, int32_t* part_offset,
                         int32_t* row_of_pair, int32_t* src_pair, uint32_t* status,
                         void* ws, hipStream_t stream);

// Whether launch_dispatch / launch_combine accept a geometry for T tokens
// (units) of hidden size H: the checks the launchers make, for the API to
// make before it enqueues anything.
bool dispatch_launch_ok(int T, int H, MoveGeometry g);
bool combine_launch_ok(int n_units, int H, MoveGeometry g);

hipError_t launch_dispatch(const uint16_t* x, int T, int H, int K,
                           const int32_t* row_of_pair, int payload,
                           void* recv_x, float* recv_scales, hipStream_t stream,
                           MoveGeometry g = kDefaultGeometry);

bool fused_layout_dispatch_fits(int T, int H, int K);

// Which fused layout+dispatch kernel a batch runs and how it is launched.
enum FusedKind { kFusedTiny = 0, kFusedCount = 1, kFusedGeneral = 2 };
struct FusedPlan {
    int kind;          // FusedKind
    int waves;         // waves per workgroup
    bool own8;         // counting kernel: at most 8 own entries per workgroup
    unsigned blocks;   // workgroups launched
};
// The plan for T >= 1 tokens with T*K <= kFusedMaxPairs and `waves` waves
// per workgroup (0: the default for the batch); false when the batch does
// not fit the fused kernels or that workgroup size is not one they take.
bool plan_layout_dispatch(int T, int H, int K, int waves, FusedPlan* plan);

hipError_t launch_layout_dispatch(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K,
                                  int E, int P, int payload, int32_t* expert_count,
                                  int32_t* expert_offset, int32_t* part_count,
                                  int32_t* part_offset, int32_t* row_of_pair, int32_t* src_pair,
                                  uint32_t* status, void* recv_x, float* recv_scales,
                                  hipStream_t stream, int waves = 0);

// Whether the combine of T tokens x top-k K at hidden size H streams (its
// gathered rows reach kStreamMinBytes: nontemporal accesses, launch-order
// blocks), and the geometry ep_combine launches it with: 2 waves per
// workgroup when it streams, else kDefaultGeometry; uncapped, 512 columns.
bool combine_streaming(int T, int H, int K);
MoveGeometry combine_default_geometry(int T, int H, int K);

hipError_t launch_combine(const uint16_t* y, const int32_t* row_of_pair,
                          const float* topk_w, int T, int H, int K,
                          uint16_t* out, hipStream_t stream,
                          MoveGeometry g = kDefaultGeometry);

size_t dedup_layout_workspace_bytes(int T, int P);

hipError_t launch_dedup_layout(const int32_t* topk_idx, int T, int K, int E, int P,
                               int32_t* tp_row, int32_t* part_tokens, int32_t* part_token_offset,
                               int32_t* tp_src, uint32_t* kmask, uint32_t* status, void* ws,
                               hipStream_t stream);

hipError_t launch_combine_partial(const uint16_t* y, const int32_t* row_of_pair,
                                  const float* topk_w, const int32_t* tp_row,
                                  const uint32_t* kmask, int T, int H, int K, int P,
                                  uint16_t* partial, hipStream_t stream);

hipError_t launch_combine_reduce(const uint16_t* partial, const int32_t* tp_row, int T, int H,
                                 int P, uint16_t* out, hipStream_t stream);

// The same for the per-destination (dedup) fused kernels: the counting one
// (K a power of two, T*K <= 1024, 8, 7 or 6 waves dividing the 512-column
// steps per token, so that every workgroup lies inside one token) or the
// general one (4 or 8 waves); P <= kMaxTopK.
bool plan_dedup_layout_dispatch(int T, int H, int K, int P, int waves, FusedPlan* plan);

hipError_t launch_dedup_layout_dispatch(const int32_t* topk_idx, const uint16_t* x, int T, int H,
                                        int K, int E, int P, int payload, int32_t* expert_count,
                                        int32_t* expert_offset, int32_t* part_count,
                                        int32_t* part_offset, int32_t* row_of_pair,
                                        int32_t* src_pair, int32_t* tp_row, int32_t* part_tokens,
                                        int32_t* part_token_offset, int32_t* tp_src,
                                        uint32_t* kmask, uint32_t* status, void* recv_x,
                                        float* recv_scales, hipStream_t stream, int waves = 0);

hipError_t launch_e4m3fn_encode(const float* in, int64_t n, uint8_t* out,
                                hipStream_t stream);

hipError_t launch_idx_narrow(const int64_t* in, int64_t n, int32_t* out, hipStream_t stream);

}  // namespace ep
