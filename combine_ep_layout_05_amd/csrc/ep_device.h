// ep_device.h -- constants and wave-level device helpers shared by the
// layout, dispatch and combine kernels (gfx950, wave64).
//
// One source of truth for every size the host launch code and the kernels
// both depend on: block shapes, the single-workgroup layout limit, the chunk
// size of the multi-workgroup layout and the column span one wave covers per
// step.  The sources show what goes wrong when a host-side buffer count and a
// device-side constant are defined apart (DeepEP PR #693, review comments on
// the staging-buffer count); here both sides include this header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;                  // gfx950 wavefront width

// ---- layout ---------------------------------------------------------------
constexpr int kLayoutThreads = 1024;       // one pair per thread per round
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kMaxExperts = 1024;          // one expert column per thread
constexpr int kSmallMaxPairs = 2048;       // single-workgroup layout up to this
constexpr int kChunkPairs = 1024;          // pairs per workgroup above it
constexpr int kMaxChunksTwoPass = 256;     // above: a separate scan launch
static_assert(kMaxExperts <= kLayoutThreads, "scan assigns one expert per thread");
static_assert(kChunkPairs % kLayoutThreads == 0, "a chunk is whole rounds");
static_assert(kLayoutWaves * kWave <= 0xFFFF, "per-wave counts fit in uint16");

// ---- dispatch / combine ---------------------------------------------------
constexpr int kMaxTopK = 16;
constexpr int kFusedMaxPairs = 4096;       // layout fused into dispatch up to this T*K
constexpr int kMoveThreads = 256;          // 4 waves per workgroup
// payload bytes of one call above which dispatch/combine use streaming
// (nontemporal) accesses; below it the working set stays cache resident
constexpr int64_t kStreamMinBytes = (int64_t)64 << 20;
constexpr int kMoveWaves = kMoveThreads / kWave;
constexpr int kColsPerLane = 8;            // 16 B of bf16 per lane per step
constexpr int kStepCols = kWave * kColsPerLane;   // 512 columns per wave step
constexpr int kScaleBlock = 128;           // columns per fp8 scale
constexpr int kLanesPerScaleBlock = kScaleBlock / kColsPerLane;   // 16 = one DPP row
static_assert(kLanesPerScaleBlock == 16, "a scale block must be one 16-lane DPP row");

// Launch geometry of the dispatch and combine kernels: waves per workgroup
// (1, 2, 4 or 8; the kernels read it from blockDim), a cap on the number of
// workgroups (0: one wave per work item; otherwise the waves stride over the
// items) and the slice of a work item in 512-column steps (1 or 2: 512 or
// 1024 columns of one token per wave).  The default is 4 waves, uncapped,
// 512 columns.
constexpr int kMaxMoveWaves = 8;
constexpr int kMaxSliceSteps = 2;
struct MoveGeometry {
    int waves;
    int max_blocks;
    int slice_steps;
};
constexpr MoveGeometry kDefaultGeometry{kMoveWaves, 0, 1};
static_assert(kMoveWaves * kMaxTopK <= kWave, "a workgroup's own entries fit in one wave");
static_assert(kMaxExperts <= 1024, "fused slot ranks compare 10 id bits");

// Bits of v strictly below this lane set in `mask` (wave64).
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// 16- and 8-byte global accesses with a cache policy.  kStream = true marks
// data touched once (nontemporal: the access does not displace reusable lines
// in L2 / the memory-side cache).  At large batches the combine streams far
// more than the caches hold, and keeping its reads and writes from evicting
// the dispatch's freshly written rows measured faster on MI355X.
typedef unsigned int ep_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int ep_u32x2 __attribute__((ext_vector_type(2)));

template <bool kStream>
__device__ __forceinline__ uint4 load16(const void* p)
{
    ep_u32x4 v;
    if constexpr (kStream) v = __builtin_nontemporal_load(reinterpret_cast<const ep_u32x4*>(p));
    else v = *reinterpret_cast<const ep_u32x4*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool kStream>
__device__ __forceinline__ void store16(void* p, uint4 u)
{
    ep_u32x4 v = {u.x, u.y, u.z, u.w};
    if constexpr (kStream) __builtin_nontemporal_store(v, reinterpret_cast<ep_u32x4*>(p));
    else *reinterpret_cast<ep_u32x4*>(p) = v;
}

template <bool kStream>
__device__ __forceinline__ void store8(void* p, uint2 u)
{
    ep_u32x2 v = {u.x, u.y};
    if constexpr (kStream) __builtin_nontemporal_store(v, reinterpret_cast<ep_u32x2*>(p));
    else *reinterpret_cast<ep_u32x2*>(p) = v;
}

// Inclusive prefix sum over the 64 lanes (DPP: row_shr 1/2/4/8 within each
// 16-lane row, then row_bcast 15 / 31 carry the row totals; lanes without a
// source add 0).
__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
    return v;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also makes every
// wave wait for its own outstanding global loads and stores (vmcnt 0) before
// the barrier; the layout kernels synchronise through LDS alone, so their
// global stores (rows, payload) keep draining across the barrier instead.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Within each aligned group of K consecutive lanes (K = 1, 2, 4, 8 or 16,
// so a group lies inside one 16-lane DPP row): the OR of v over the group's
// lanes below this one (0 for the group's first lane).  Inclusive steps
// row_shr 1, 2, 4, 8 taken only from sources inside the group, then one more
// row_shr 1 for the exclusive value.
__device__ __forceinline__ uint32_t group_excl_or(uint32_t v, int K, int lane)
{
    const int r = lane & (K - 1);            // position in the group
    int x = (int)v;
    if (K >= 2) { const int y = __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false); x |= r >= 1 ? y : 0; }
    if (K >= 4) { const int y = __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false); x |= r >= 2 ? y : 0; }
    if (K >= 8) { const int y = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false); x |= r >= 4 ? y : 0; }
    if (K >= 16) { const int y = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false); x |= r >= 8 ? y : 0; }
    const int y = __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);        // row_shr:1
    return r >= 1 ? (uint32_t)y : 0u;
}

// Orders one wave's LDS accesses across a hand-off between its lanes: every
// LDS write or atomic of this wave issued before it completes, and is visible
// to the wave's LDS reads issued after it (a wave barrier between a release
// and an acquire fence on the local address space).  For the places where the
// lanes of one wave pass values through LDS with no workgroup barrier: the
// hardware completes one wave's LDS operations in order, and this keeps the
// compiler from reordering the non-atomic accesses around the hand-off.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// MI355X runs a launch's workgroups on its 8 XCDs round robin (workgroup b
// on XCD b % 8), each XCD with its own L2.  xcd_block renumbers the grid so
// that every XCD holds one contiguous range of logical blocks: kernels that
// map logical block -> items the same way then run a token's items on the
// same XCD, and a kernel reading what the previous one wrote for that token
// (row maps, dedup masks, partial rows) finds it in that XCD's L2 instead of
// going out to the memory-side cache.
constexpr int kXcds = 8;
constexpr int kCUs = 256;                  // compute units of an MI355X

__device__ __forceinline__ int xcd_block(int b, int nblocks)
{
    const int per = nblocks / kXcds, rem = nblocks % kXcds;
    const int x = b % kXcds, slot = b / kXcds;
    return x * per + (x < rem ? x : rem) + slot;
}

__device__ __forceinline__ int wave_uniform(int v)
{
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ int read_lane(int v, int lane)
{
    return __builtin_amdgcn_readlane(v, lane);
}

}  // namespace ep
