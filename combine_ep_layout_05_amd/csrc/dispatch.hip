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
// the grid (waves per workgroup and the workgroup count are the launch
// geometry: 4 waves and one wave per item unless the caller tunes them), so a handful of tokens still spreads over many CUs (MoRI PR #614,
// DispatchIntraNode paragraph: splitting per block over tokens starved most
// blocks at 4 tokens; MultiWarpIter paragraph: keep at least 512 elements per
// warp).  Per lane:
//   - one 16-byte load of x (global_load_dwordx4, fully coalesced);
//   - the 128-column block of a scale is one 16-lane DPP row, so amax is a
//     per-lane max over 8 values and 4 DPP max steps (quad_perm xor 1,
//     quad_perm xor 2, row_half_mirror, row_mirror), with no LDS traffic;
//   - x / scale gives the byte of the IEEE fp32 quotient: a reciprocal plus
//     one remainder correction where the scale is >= 2^-90 (shown
//     byte-identical to the division over every pair of bf16 values), the
//     division itself otherwise (ep_numerics.h); v_cvt_pk_fp8_f32 packs two
//     values per instruction (round to nearest even; a NaN-preserving clamp
//     to +-448 in front gives the saturating behaviour);
//   - per receive row one 8-byte store per lane (512 contiguous bytes per
//     wave, whole 128-byte lines; the row base in scalar registers) and one
//     16-byte store of the item's 4 block scales, by the lane holding the row.
// The next item's x vector and row indices are loaded before the current
// item's quantise-and-store work, so each wave keeps one load in flight
// while its stores drain (the prefetch idea of DeepEP PR #693, with a
// register double buffer instead of shared-memory TMA staging).
#include <algorithm>
#include <numeric>
#include <type_traits>

#include "ep_device.h"
#include "ep_launch.h"
#include "ep_numerics.h"

namespace ep {
namespace {

// Write one item to the receive rows of its token's entries.  An item is
// kSub consecutive 512-column steps of one token (one wave, 8 columns per
// lane and step); step s holds the fp8 bytes q[s] and the block scales
// scale[s] (kPayload 0) or the bf16 vector v[s] unchanged (kPayload 1).
// Lanes lane0 .. lane0+K-1 of `myrow` hold the rows of the token's entries
// 0..K-1 (K <= kMaxRows); rows outside [0, n_rows) -- masked entries -- are
// skipped.  col_base is the item's first column.
//   - Payload: a loop over the entries that have a row (one ballot gives
//     them as bits, the loop takes the lowest each time).  A row's base
//     address is formed in scalar registers and this lane's byte offset
//     stays in one vector register, so a row costs one lane read, a few
//     scalar instructions and one store per step (the scalar-base store
//     form), and when the item lies inside the row the loop runs without
//     per-lane column masks.  The loop over the set bits replaced an unrolled
//     loop over all kMaxRows entries with a uniform test each: graphs of 50
//     launches on MI355X, 128 x 7168, the fused dedup launch (16 candidate
//     rows, about 6.4 present) 5.28 -> 4.98 us (E = 32, P = 8: 4.89 -> 4.71),
//     dedup step 13.86 -> 13.74 us; the plain launches within 0.3 %.
//   - fp8 scales: the item's block scales (lanes 0, 16, 32, 48 of each step)
//     go to each row as one 16-byte store per step, made by the lane that
//     holds the row, instead of four lanes storing 4 bytes into every row
//     under a lane mask.
// The payload stores are nontemporal (the receive rows are read by the expert
// computation, not by this launch again), in every dispatch kernel and at
// every batch size.  Measured on MI355X against cached stores, graphs of 50
// steps, top-8, even with everything cache resident: 128 x 7168 the fused
// launch 4.40 -> 4.30 us and the step with the combine after it 7.31 -> 6.89
// us (with 16 rotating input sets, nothing left in the caches: 11.7 -> 10.1
// us); 600 x 7168, unfused dispatch, step 32.5 -> 29.2 us.
template <int kPayload, int kMaxRows, int kSub>
__device__ __forceinline__ void store_rows(const uint4 (&v_in)[kSub], const uint2 (&q)[kSub],
                                           const float (&scale)[kSub], int myrow, int lane0,
                                           int col_base, int lane, int H, int K, int n_rows,
                                           uint8_t* __restrict__ recv_x,
                                           float* __restrict__ recv_scales)
{
    static_assert(kMaxRows <= kWave, "a token's entries sit on lanes of one wave");
    constexpr int kBytes = kPayload == 0 ? 1 : 2;
    uint4 v[kSub];
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
        v[u] = v_in[u];
        // The bf16 store data is the loaded x vector: wait for it once here.
        // A wait for a load is a wait for every earlier store too (one
        // counter on this architecture), and the compiler would otherwise
        // put one in front of every row's store, each row being a block of
        // its own.
        if constexpr (kPayload == 1)
            asm volatile("" : "+v"(v[u].x), "+v"(v[u].y), "+v"(v[u].z), "+v"(v[u].w));
    }
    const uint32_t voff = (uint32_t)(col_base + lane * kColsPerLane) * kBytes;
    auto row_loop = [&](bool full) {
        bool lane_ok[kSub];
#pragma unroll
        for (int u = 0; u < kSub; ++u)
            lane_ok[u] = full || col_base + u * kStepCols + lane * kColsPerLane < H;
        // bit k: entry k has a row (lane0 + K <= 64)
        uint64_t rows = __ballot((uint32_t)(lane - lane0) < (uint32_t)K &&
                                 (uint32_t)myrow < (uint32_t)n_rows) >> lane0;
        while (rows) {
            const int k = (int)__builtin_ctzll(rows);
            rows &= rows - 1;
            const uint32_t r = (uint32_t)read_lane(myrow, lane0 + k);
            uint8_t* rowp = recv_x + (uint64_t)r * (uint32_t)(H * kBytes);
#pragma unroll
            for (int u = 0; u < kSub; ++u) {
                const uint32_t o = voff + (uint32_t)(u * kStepCols * kBytes);
                if (lane_ok[u]) {
                    if constexpr (kPayload == 0) store8<true>(rowp + o, q[u]);
                    else store16<true>(rowp + o, v[u]);
                }
            }
        }
    };
    if (col_base + kSub * kStepCols <= H) row_loop(true);       // uniform
    else row_loop(false);
    if constexpr (kPayload == 0) {
        constexpr int kBlk = kStepCols / kScaleBlock;            // 4 scales per step
        float sc[kSub * kBlk];
#pragma unroll
        for (int u = 0; u < kSub; ++u)
#pragma unroll
            for (int b = 0; b < kBlk; ++b)
                sc[u * kBlk + b] = __builtin_bit_cast(
                    float, read_lane(__builtin_bit_cast(int, scale[u]), b * kLanesPerScaleBlock));
        const uint32_t nsc = (uint32_t)H / kScaleBlock;          // scales per row
        const uint32_t b0 = (uint32_t)col_base / kScaleBlock;    // the item's first block
        const uint32_t nblk = nsc - b0 < (uint32_t)(kSub * kBlk) ? nsc - b0 : kSub * kBlk;
        const uint32_t k = (uint32_t)(lane - lane0);
        if (k < (uint32_t)K && (uint32_t)myrow < (uint32_t)n_rows) {
            float* sp = recv_scales + (uint64_t)(uint32_t)myrow * nsc + b0;
            if (nblk == (uint32_t)(kSub * kBlk) && (nsc & 3u) == 0u) {   // 16-byte aligned
#pragma unroll
                for (int u = 0; u < kSub; ++u)
                    *reinterpret_cast<float4*>(sp + u * kBlk) =
                        make_float4(sc[u * kBlk], sc[u * kBlk + 1], sc[u * kBlk + 2],
                                    sc[u * kBlk + 3]);
            } else {
#pragma unroll
                for (int b = 0; b < kSub * kBlk; ++b)
                    if ((uint32_t)b < nblk) sp[b] = sc[b];
            }
        }
    }
}

// One 512-column step: the form the fused kernels use.
template <int kPayload, int kMaxRows>
__device__ __forceinline__ void store_rows(uint4 v, uint2 q, float scale, int myrow, int lane0,
                                           int col_base, int lane, int H, int K, int n_rows,
                                           uint8_t* __restrict__ recv_x,
                                           float* __restrict__ recv_scales)
{
    const uint4 va[1] = {v};
    const uint2 qa[1] = {q};
    const float sa[1] = {scale};
    store_rows<kPayload, kMaxRows, 1>(va, qa, sa, myrow, lane0, col_base, lane, H, K, n_rows,
                                      recv_x, recv_scales);
}

// Quantise (fp8) one item; must be called by all 64 lanes of the wave (the
// 128-column amax uses DPP row exchanges).  bf16 needs no work.
template <int kPayload>
__device__ __forceinline__ uint2 prepare_item(uint4 v, float& scale)
{
    scale = 0.0f;
    if constexpr (kPayload == 0) return quantise_e4m3fn_block8(v, scale);
    return make_uint2(0u, 0u);
}

// An item is kSub consecutive 512-column steps of one token (the slice of
// the launch geometry: 512 or 1024 columns); items_per_token = ceil(steps /
// kSub), the last item of a token possibly partial.
template <int kPayload, int kMaxK, int kSub, bool kOnce>
__global__ __launch_bounds__(kMaxMoveWaves * kWave) void dispatch_kernel(
    const uint16_t* __restrict__ x, int H, int K, const int32_t* __restrict__ row_of_pair,
    uint8_t* __restrict__ recv_x, float* __restrict__ recv_scales,
    int items_per_token, int n_items, int n_rows)
{
    const int lane = threadIdx.x % kWave;
    const int waves = blockDim.x / kWave;
    const int stride = gridDim.x * waves;
    int item = blockIdx.x * waves + wave_uniform(threadIdx.x / kWave);
    if (item >= n_items) return;

    // load stage of one item: row ids (lanes < K) and this lane's 16 bytes of
    // x per step, all loads without a branch around them (lanes past K read
    // entry 0, columns past H read column 0; the values are dropped)
    auto load_item = [&](int it, int& myrow, uint4 (&v)[kSub], int& col_base) {
        const int t = it / items_per_token;
        col_base = (it - t * items_per_token) * (kSub * kStepCols);
        myrow = row_of_pair[(int64_t)t * K + (lane < K ? lane : 0)];
#pragma unroll
        for (int u = 0; u < kSub; ++u) {
            const int c = col_base + u * kStepCols + lane * kColsPerLane;
            v[u] = *reinterpret_cast<const uint4*>(x + (int64_t)t * H + (c < H ? c : 0));
        }
    };
    auto quantise_and_store = [&](const uint4 (&v)[kSub], int myrow, int col_base) {
        float scale[kSub];
        uint2 q[kSub];
#pragma unroll
        for (int u = 0; u < kSub; ++u) q[u] = prepare_item<kPayload>(v[u], scale[u]);
        store_rows<kPayload, kMaxK, kSub>(v, q, scale, myrow, 0, col_base, lane, H, K, n_rows,
                                          recv_x, recv_scales);
    };

    int myrow, col_base;
    uint4 v[kSub];
    load_item(item, myrow, v, col_base);
    if constexpr (kOnce) {               // the grid covers every item: no prefetch loop
        // the row ids pinned where they are loaded, so the compiler does not
        // sink the load into the lanes < K (with a lazy argument load and a
        // wait of its own); x is waited for next anyway
        asm volatile("" : "+v"(myrow));
        if (lane >= K) myrow = -1;
        quantise_and_store(v, myrow, col_base);
        return;
    }

    if (lane >= K) myrow = -1;
    while (true) {
        const int next = item + stride;      // n_items + stride < 2^31 (checked by the launcher)
        int nrow = -1, ncol = 0;
        uint4 nv[kSub];
#pragma unroll
        for (int u = 0; u < kSub; ++u) nv[u] = make_uint4(0, 0, 0, 0);
        if (next < n_items) {
            load_item(next, nrow, nv, ncol);
            if (lane >= K) nrow = -1;
        }

        quantise_and_store(v, myrow, col_base);

        if (next >= n_items) break;
        item = next;
        myrow = nrow;
        for (int u = 0; u < kSub; ++u) v[u] = nv[u];
        col_base = ncol;
    }
}

// ---------------------------------------------------------------------------
// Layout fused into the dispatch, for small batches (T*K <= kFusedMaxPairs).
//
// At a few tokens the step is paced by launches and latency, not bytes (MoRI
// PR #614, view-cache paragraph: latency flat over hidden 1024..6144 and over
// 4/8/16 tokens).  Here every dispatch workgroup derives, from all T*K ids (at
// most 16 KB, read from L2), exactly the layout values it needs, so no
// separate layout launch precedes the dispatch (up to 128 ids the barrier-free
// kernel further below takes over):
//   - the per-expert totals (LDS atomics: integer sums, order-free), and per
//     expert the number of entries before this workgroup's first token;
//   - the exclusive scan of the totals (1024 / threads consecutive experts per
//     thread, DPP wave scan; each thread leaves its experts' in-wave prefixes
//     in LDS and the wave totals complete them after one barrier);
//   - the slots of its own tokens' entries: offset + entries before + rank
//     among the workgroup's own entries (ballot match-any over the <= 64 own
//     ids in one wave, while the others quantise; each wave then computes
//     the rows of its own item and stores it with no further barrier).
// Three barriers in all.  The x vectors are loaded first and quantised while
// the histogram atomics drain, and the layout outputs are written after the
// payload stores.  Workgroup 0 writes the counts, offsets, partition sums and
// status; the workgroup holding a token's first 512-column step writes that
// token's row_of_pair and src_pair entries.  Every output equals ep_layout's
// followed by ep_dispatch's.
//
// The per-destination (dedup) variant derives in the same launch the dedup
// layout as well: each token's partition set (every valid entry ors its
// partition bit into its token's LDS word; e / L and entry / K by
// multiply-shifts that are exact in these ranges), the per-partition token
// totals and the tokens before this workgroup's first token (counted by the
// entry that finds its bit still clear), and from these, after the second
// barrier, the rows and top-k masks of each wave's token's (token,
// partition) couples.  The payload goes once to each of a token's partitions
// (the dedup rows) right then, before the expert scan; the per-expert layout
// is still written out for the expert side and the combine.
struct DedupOutputs {
    int32_t* tp_row;
    int32_t* part_tokens;
    int32_t* part_token_offset;
    int32_t* tp_src;
    uint32_t* kmask;
};

constexpr int kMaxFusedWaves = 8;          // workgroups of 4 or 8 waves

struct FusedSmem {
    int32_t cnt[kMaxExperts];
    int32_t before[kMaxExperts];
    int32_t offp[kMaxExperts];                 // in-wave exclusive prefix of cnt
    int32_t off[kMaxExperts];                  // workgroup 0: full offsets, for the partition sums
    int32_t wsum[kMaxFusedWaves];
    int32_t rank[kWave];                       // own entry q: earlier own entries, same expert
    uint32_t bad;
    // dedup variant
    int32_t ptot[kMaxTopK];                    // tokens per partition
    int32_t pbef[kMaxTopK];                    // of those, before this workgroup's first token
};

template <int kMaxN>
struct FusedDedupSmem : FusedSmem {
    uint32_t tpres[kMaxN];                     // partition set (bit p) of every token
};

// kW waves per workgroup, each wave one work item; the workgroup's own
// tokens' entries (at most 64, checked by the launcher) are ranked in one wave.
// kMaxN (2048 or 4096) bounds T*K: the ids each thread holds are kMaxN /
// threads, so small batches take the smaller instance.
template <int kPayload, bool kDedup, int kW, int kMaxN>
__global__ __launch_bounds__(kW * kWave) void layout_dispatch_kernel(
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ x, int n, int H, int K, int E,
    int P, int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ part_count, int32_t* __restrict__ part_offset,
    int32_t* __restrict__ row_of_pair, int32_t* __restrict__ src_pair,
    uint32_t* __restrict__ status, uint8_t* __restrict__ recv_x, float* __restrict__ recv_scales,
    int steps_per_token, int n_items, DedupOutputs dd)
{
    constexpr int kThreads = kW * kWave;
    constexpr int kIds = kMaxN / kThreads;                 // ids per thread
    constexpr int kPer = kMaxExperts / kThreads;           // experts per thread
    constexpr int kPerWave = kPer * kWave;
    static_assert(kIds * kThreads == kMaxN && kPer * kThreads == kMaxExperts,
                  "ids and experts split evenly over the threads");
    static_assert(kMaxN <= kFusedMaxPairs, "the launcher's bound");
    static_assert(kW <= kMaxFusedWaves, "wave totals fit");
    __shared__ std::conditional_t<kDedup, FusedDedupSmem<kMaxN>, FusedSmem> s;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = wave_uniform(tid / kWave);
    const int item0 = xcd_block(blockIdx.x, gridDim.x) * kW;
    const int item = item0 + w;
    const int last = (item0 + kW - 1 < n_items) ? item0 + kW - 1 : n_items - 1;
    const int t_lo = item0 / steps_per_token;
    const int t_hi = last / steps_per_token;
    const int nown = t_hi - t_lo + 1;             // own tokens, <= kW
    const int p_lo = t_lo * K;
    const int nq = nown * K;                      // own entries, <= 64 (the launcher picks kW so)
    const int T = n / K;
    const int L = E / P;

    // every load is independent: all ids (issued back to back, addresses
    // clamped into the array instead of branching), the own entries' ids, and
    // the x vector
    int ids[kIds];
#pragma unroll
    for (int j = 0; j < kIds; ++j) {
        ids[j] = -1;
        if (j * kThreads < n) {                           // rounds with ids (uniform)
            const int p = j * kThreads + tid;
            ids[j] = idx[p < n ? p : n - 1];
        }
    }
    int me = idx[p_lo + (lane < nq ? lane : 0)];           // own entry q = lane
    int t = 0, col0 = H;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (item < n_items) {
        t = item / steps_per_token;
        col0 = (item - t * steps_per_token) * kStepCols + lane * kColsPerLane;
        if (col0 < H) v = *reinterpret_cast<const uint4*>(x + (int64_t)t * H + col0);
    }
#pragma unroll
    for (int j = 0; j < kIds; ++j)
        if (j * kThreads + tid >= n) ids[j] = -1;
    if (lane >= nq) me = -1;
    for (int e = tid; e < E; e += kThreads) { s.cnt[e] = 0; s.before[e] = 0; }
    if (tid == 0) s.bad = 0u;
    if constexpr (kDedup) {
        if (tid < P) { s.ptot[tid] = 0; s.pbef[tid] = 0; }
        for (int tt = tid; tt < T; tt += kThreads) s.tpres[tt] = 0u;
    }
    lds_barrier();                                         // (1) counters cleared

    bool bad = false;
#pragma unroll
    for (int j = 0; j < kIds; ++j) {
        if (j * kThreads >= n) break;                     // no more ids (uniform)
        const int p = j * kThreads + tid;
        const int e = ids[j];
        bad |= (e >= E);
        if (e >= 0 && e < E) {
            atomicAdd(&s.cnt[e], 1);
            if (p < p_lo) atomicAdd(&s.before[e], 1);
        }
    }
    if (bad) s.bad = 1u;
    if constexpr (kDedup) {
        // partition set of every token: each valid entry ors its partition
        // bit into its token's LDS word; the entry that finds the bit still
        // clear counts the token once for that partition, and once more in
        // the total before t_lo when the token precedes the workgroup's own
        // (order-free sums)
        // Exact division by multiply-shift: with m = floor(2^s / d) + 1 and
        // 2^s = q*d + r, a*m / 2^s = a/d + a*(d - r) / (d * 2^s), and the
        // error term stays below 1/d (so floor is unchanged) whenever
        // a*(d - r) < 2^s: for e < 1024, L <= 1024, s = 20 (1023 * 1024 <
        // 2^20), and for entries p < 4096, K <= 16, s = 16 (4095 * 16 < 2^16).
        const uint32_t magic_l = (1u << 20) / (uint32_t)L + 1u;   // e / L = (e * magic_l) >> 20
        const uint32_t magic_k = (1u << 16) / (uint32_t)K + 1u;   // p / K = (p * magic_k) >> 16
        uint32_t old[kIds], pk[kIds];
        int tk[kIds];
#pragma unroll
        for (int j = 0; j < kIds; ++j) {
            const int p = j * kThreads + tid;
            const int e = j * kThreads < n ? ids[j] : -1;
            tk[j] = -1;
            old[j] = 0u;
            pk[j] = 0u;
            if (e >= 0 && e < E) {
                tk[j] = (int)(((uint32_t)p * magic_k) >> 16);
                pk[j] = ((uint32_t)e * magic_l) >> 20;
                old[j] = atomicOr(&s.tpres[tk[j]], 1u << pk[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kIds; ++j) {
            if (tk[j] >= 0 && !((old[j] >> pk[j]) & 1u)) {
                atomicAdd(&s.ptot[pk[j]], 1);
                if (tk[j] < t_lo) atomicAdd(&s.pbef[pk[j]], 1);
            }
        }
    }
    // while the atomics drain: quantise this wave's item; the last wave also
    // ranks the workgroup's own entries among themselves (match-any ballots)
    float scale = 0.0f;
    uint2 q = make_uint2(0u, 0u);
    if (item < n_items) q = prepare_item<kPayload>(v, scale);
    const bool mvalid = (me >= 0) && (me < E);
    if (w == kW - 1) {
        uint64_t peers = __ballot(mvalid);
        for (int b = 0; b < 10; ++b) {            // ids < kMaxExperts = 2^10
            const bool bit = (me >> b) & 1;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        s.rank[lane] = lanes_below(peers);
    }
    lds_barrier();                                         // (2) totals complete

    if constexpr (kDedup) {
        // this wave's token: couple (t, p) in lane p < P
        const int pc = (lane < P) ? s.ptot[lane] : 0;
        const int pincl = wave_inclusive_scan(pc);          // partition offsets
        const int M = read_lane(pincl, P - 1);
        int drow = -1;
        uint32_t m = 0u;
        if (item < n_items && lane < P) {
            const uint32_t bit = 1u << lane;
            int before = 0;
#pragma unroll
            for (int j = 0; j < kW - 1; ++j)
                before += (t_lo + j < t && (s.tpres[t_lo + j] & bit)) ? 1 : 0;
            if (s.tpres[t] & bit) drow = pincl - pc + s.pbef[lane] + before;
            const uint32_t lo = (uint32_t)(lane * L);
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k)           // token t's ids: own entries (t - t_lo)*K + k
                if (k < K && (uint32_t)read_lane(me, (t - t_lo) * K + k) - lo < (uint32_t)L)
                    m |= 1u << k;
        }
        if (item < n_items) {
            store_rows<kPayload, kMaxTopK>(v, q, scale, drow, 0, col0 - lane * kColsPerLane,
                                                 lane, H, P, T * P, recv_x, recv_scales);
            if (t * steps_per_token == item && lane < P) {   // the token's first step writes its couples
                const int j = t * P + lane;
                dd.tp_row[j] = drow;
                dd.kmask[j] = m;
                if (drow >= 0) dd.tp_src[drow] = j;
            }
        }
        if (blockIdx.x == 0 && w == 0 && lane < P) {
            dd.part_tokens[lane] = pc;
            dd.part_token_offset[lane] = pincl - pc;
            if (lane == P - 1) dd.part_token_offset[P] = M;
        }
        for (int r = M + blockIdx.x * kThreads + tid; r < T * P; r += gridDim.x * kThreads)
            dd.tp_src[r] = -1;
    }

    // exclusive scan of the expert totals: 4 consecutive experts per thread;
    // in-wave prefixes go to LDS, the wave totals complete them
    int c[kPer], sum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = tid * kPer + j;
        c[j] = (e < E) ? s.cnt[e] : 0;
        sum += c[j];
    }
    const int incl = wave_inclusive_scan(sum);
    if (lane == kWave - 1) s.wsum[w] = incl;
    int run = incl - sum;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = tid * kPer + j;
        if (e < E) s.offp[e] = run;
        run += c[j];
    }
    lds_barrier();                                         // (3) prefixes complete

    int wsv[kW], N = 0;
#pragma unroll
    for (int u = 0; u < kW; ++u) {
        wsv[u] = s.wsum[u];
        N += wsv[u];
    }
    auto wave_base = [&](int ww) {
        int b = 0;
#pragma unroll
        for (int u = 0; u < kW; ++u) b += (u < ww) ? wsv[u] : 0;
        return b;
    };
    int myrow = -1;                               // row of own entry q = lane
    if (mvalid)
        myrow = s.offp[me] + wave_base(me / kPerWave) + s.before[me] + s.rank[lane];

    if constexpr (!kDedup) {
        if (item < n_items)
            store_rows<kPayload, kMaxTopK>(v, q, scale, myrow, (t - t_lo) * K,
                                                 col0 - lane * kColsPerLane, lane, H, K, n, recv_x,
                                                 recv_scales);
    }

    // layout outputs, after the payload stores
    if (w == 0 && lane < nq) {
        const int tt = t_lo + lane / K;
        if (tt * steps_per_token >= item0) {      // this workgroup holds the token's first step
            const int p = p_lo + lane;
            row_of_pair[p] = myrow;
            if (myrow >= 0 && myrow < n) src_pair[myrow] = p;
        }
    }
    if (blockIdx.x == 0) {
        const int base = wave_base(w);
        int o = base + incl - sum;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = tid * kPer + j;
            if (e < E) {
                expert_count[e] = c[j];
                expert_offset[e] = o;
                s.off[e] = o;
            }
            o += c[j];
        }
        if (tid == 0) {
            expert_offset[E] = N;
            part_offset[P] = N;
            *status = s.bad ? 1u : 0u;
        }
        lds_barrier();                                     // workgroup 0 only: full offsets
        for (int p = tid; p < P; p += kThreads) {
            const int lo = s.off[p * L];
            const int hi = (p + 1 < P) ? s.off[(p + 1) * L] : N;
            part_offset[p] = lo;
            part_count[p] = hi - lo;
        }
    }
    for (int r = N + blockIdx.x * kThreads + tid; r < n; r += gridDim.x * kThreads)
        src_pair[r] = -1;
}

// ---------------------------------------------------------------------------
// Layout fused into the dispatch for tiny batches (T*K <= kTinyPairs).
//
// With at most 128 ids every wave holds all of them (two per lane) and ranks
// its own token's entries by itself: the slot of entry (e, p) is the number
// of valid entries before it in (expert, entry) order, i.e. the count of keys
// e'*2^12 + p' below e*2^12 + p -- one ballot and popcount per own entry and
// round.  No LDS and no barrier stand between the id load and the payload
// stores, where the general fused kernel spends three barriers and the LDS
// histogram and scan.  One extra workgroup (launch block 0, dispatched first)
// builds the per-expert histogram of the same ids in LDS within one wave (its
// LDS operations complete in program order, so it needs no workgroup barrier,
// only wave_lds_sync at each hand-off)
// and writes the counts, offsets, partition sums and status.  Outputs are
// those of the general kernel.
constexpr int kTinyPairs = 2 * kWave;

template <int kPayload, int kOwn>
__global__ __launch_bounds__(kMaxMoveWaves * kWave) void layout_dispatch_tiny_kernel(
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ x, int n, int H, int K, int E,
    int P, int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ part_count, int32_t* __restrict__ part_offset,
    int32_t* __restrict__ row_of_pair, int32_t* __restrict__ src_pair,
    uint32_t* __restrict__ status, uint8_t* __restrict__ recv_x, float* __restrict__ recv_scales,
    int steps_per_token, int n_items)
{
    constexpr int kPerLane = kMaxExperts / kWave;          // experts per lane in the scan
    __shared__ int32_t cnt[kMaxExperts];
    const int lane = threadIdx.x % kWave;
    const int w = wave_uniform(threadIdx.x / kWave);
    const int p0 = lane, p1 = kWave + lane;

    if (blockIdx.x == 0) {
        if (w != 0) return;
        // counts, offsets, partition sums and status, by one wave
        const int id0 = idx[p0 < n ? p0 : n - 1];
        const int id1 = idx[p1 < n ? p1 : n - 1];
        const bool v0 = p0 < n && id0 >= 0 && id0 < E;
        const bool v1 = p1 < n && id1 >= 0 && id1 < E;
        const bool bad = (p0 < n && id0 >= E) || (p1 < n && id1 >= E);
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            if (e < E) cnt[e] = 0;
        }
        wave_lds_sync();                          // counters cleared
        if (v0) atomicAdd(&cnt[id0], 1);
        if (v1) atomicAdd(&cnt[id1], 1);
        wave_lds_sync();                          // histogram complete
        int c[kPerLane], sum = 0;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            c[j] = (e < E) ? cnt[e] : 0;
            sum += c[j];
        }
        const int incl = wave_inclusive_scan(sum);
        const int N = read_lane(incl, kWave - 1);
        int o = incl - sum;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            if (e < E) {
                expert_count[e] = c[j];
                expert_offset[e] = o;
                cnt[e] = o;                      // offsets, for the partition sums below
            }
            o += c[j];
        }
        wave_lds_sync();                          // offsets written
        const int L = E / P;
        for (int p = lane; p < P; p += kWave) {
            const int lo = cnt[p * L];
            const int hi = (p + 1 < P) ? cnt[(p + 1) * L] : N;
            part_offset[p] = lo;
            part_count[p] = hi - lo;
        }
        const bool anybad = __ballot(bad) != 0;
        if (lane == 0) {
            expert_offset[E] = N;
            part_offset[P] = N;
            *status = anybad ? 1u : 0u;
        }
        return;
    }

    const int waves = blockDim.x / kWave;
    const int item = xcd_block(blockIdx.x - 1, gridDim.x - 1) * waves + w;
    if (item >= n_items) return;
    const int t = item / steps_per_token;
    const int col0 = (item - t * steps_per_token) * kStepCols + lane * kColsPerLane;
    // all loads issued before any result is used, the ids first: every id
    // (two per lane, addresses clamped), this token's entries, then the x
    // vector -- loads complete in issue order, so the ranking runs while x is
    // in flight.  The x load is unconditional (column clamped; the values of
    // columns >= H are never stored, and with fp8 they fill whole 16-lane
    // scale blocks): a load under a branch would make the wait for the ids
    // include it.
    const int id0 = idx[p0 < n ? p0 : n - 1];
    const int id1 = idx[p1 < n ? p1 : n - 1];
    const int me = idx[t * K + (lane < K ? lane : 0)];
    const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)t * H + (col0 < H ? col0 : 0));
    const bool v0 = p0 < n && id0 >= 0 && id0 < E;
    const bool v1 = p1 < n && id1 >= 0 && id1 < E;
    const uint32_t key0 = v0 ? ((uint32_t)id0 << 12) | (uint32_t)p0 : 0xFFFFFFFFu;
    const uint32_t key1 = v1 ? ((uint32_t)id1 << 12) | (uint32_t)p1 : 0xFFFFFFFFu;
    const bool mvalid = lane < K && me >= 0 && me < E;
    const uint32_t mkey = mvalid ? ((uint32_t)me << 12) | (uint32_t)(t * K + lane) : 0u;

    int myrow = -1;
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {             // slot of entry k: valid keys below its key
        const uint32_t qk = (uint32_t)read_lane((int)mkey, k);   // lanes >= K: key 0
        const int c = __builtin_popcountll(__ballot(key0 < qk)) +
                      __builtin_popcountll(__ballot(key1 < qk));
        if (lane == k) myrow = c;
    }
    if (!mvalid) myrow = -1;
    float scale;
    const uint2 q = prepare_item<kPayload>(v, scale);
    store_rows<kPayload, kOwn>(v, q, scale, myrow, 0, col0 - lane * kColsPerLane, lane, H, K,
                                     n, recv_x, recv_scales);

    if (item == t * steps_per_token && lane < K) {   // the token's first step writes its entries
        row_of_pair[t * K + lane] = myrow;
        if (myrow >= 0) src_pair[myrow] = t * K + lane;
    }
    const int N = __builtin_popcountll(__ballot(v0)) + __builtin_popcountll(__ballot(v1));
    for (int r = N + item * kWave + lane; r < n; r += n_items * kWave) src_pair[r] = -1;
}

// ---------------------------------------------------------------------------
// Layout fused into the dispatch for medium batches (128 < T*K <= 1024) by
// counting instead of a histogram.
//
// The slot of entry (e, p) is the number of valid entries before it in
// (expert, entry) order -- keys e*2^12 + p below its own.  Each wave holds
// its share of the ids (kIds per lane) and counts, for each of the
// workgroup's own entries, the keys below that entry's with one ballot and
// popcount per round; one barrier later the waves' counts are summed in LDS.
// That replaces the general kernel's histogram atomics, scan and three
// barriers.  Workgroups of kW waves are chosen so none straddles a token when
// kW divides the 512-column steps per token (7 at hidden 7168: a workgroup
// holds half a token, its own entries are one token's K), which keeps the
// counting to K entries.  One extra workgroup (launch block 0, dispatched
// first) builds the histogram in LDS and writes the counts, offsets,
// partition sums, status and the src_pair tail.  Outputs are those of the
// general kernel.
//
// The per-destination (dedup) variant needs every workgroup to hold part of
// exactly one token and K to divide 64 (a token's entries are then K aligned
// lanes of one wave, in every round).  An entry counts its token once for its
// partition when no lower entry of the token has the same partition (a DPP
// prefix OR over the K-lane group): it adds 1 to the partition's token total
// in LDS, and to the total before this workgroup's token when its token comes
// earlier.  The counters are cleared behind one extra barrier while the loads
// are in flight, and the barrier above makes the sums visible.  The couple
// rows are the partition offsets (a wave scan of the totals) plus the tokens
// before; the payload goes once to each of them.  Block 0 also writes the
// per-partition token totals and offsets and the tp_src tail.
constexpr int kCountMaxPairs = 1024;

template <int kPayload, bool kDedup, int kW, int kOwn>
__global__ __launch_bounds__(kW * kWave) void layout_dispatch_count_kernel(
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ x, int n, int H, int K, int E,
    int P, int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ part_count, int32_t* __restrict__ part_offset,
    int32_t* __restrict__ row_of_pair, int32_t* __restrict__ src_pair,
    uint32_t* __restrict__ status, uint8_t* __restrict__ recv_x, float* __restrict__ recv_scales,
    int steps_per_token, int n_items, DedupOutputs dd)
{
    constexpr int kThreads = kW * kWave;
    constexpr int kIds = (kCountMaxPairs + kThreads - 1) / kThreads;     // rounds of ids
    constexpr int kPer = (kMaxExperts + kThreads - 1) / kThreads;        // experts per thread
    __shared__ int32_t part[kOwn][kW];       // own entry q: keys below it, per wave
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t wsum[kW];
    __shared__ uint32_t sbad;
    // dedup, per partition: tokens with an expert in it (all / before the workgroup's)
    __shared__ int32_t ptok[kDedup ? 2 : 1][kDedup ? kMaxTopK : 1];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = wave_uniform(tid / kWave);

    // dedup: partition of expert e, e / L = (e * magic) >> 20, exact for
    // e < 1024 and L <= 1024 (the multiply-shift bound worked in the general
    // kernel)
    auto partition_of = [&](int e) {
        const uint32_t magic = (1u << 20) / (uint32_t)(E / P) + 1u;
        return ((uint32_t)e * magic) >> 20;
    };
    // dedup: each valid entry that is its token's first in its partition adds
    // the token to that partition's total (and to the total before this
    // workgroup's token when its entries lie below p_lo)
    auto count_tokens = [&](const int (&ids)[kIds], int p_lo) {
#pragma unroll
        for (int j = 0; j < kIds; ++j) {
            const bool ok = ids[j] >= 0 && ids[j] < E;
            const uint32_t pp = partition_of(ids[j]);
            const uint32_t bit = ok ? 1u << pp : 0u;
            const uint32_t lower = group_excl_or(bit, K, lane);   // every lane: DPP sources
            if (ok && !(lower & bit)) {
                atomicAdd(&ptok[0][pp], 1);
                if (j * kThreads + tid < p_lo) atomicAdd(&ptok[1][pp], 1);
            }
        }
    };

    if (blockIdx.x == 0) {
        // counts, offsets, partition sums, status and the src_pair tail (the id
        // loads all issued first: addresses clamped rather than guarded)
        int ids[kIds];
        bool bad = false;
#pragma unroll
        for (int j = 0; j < kIds; ++j) {
            const int p = j * kThreads + tid;
            ids[j] = idx[p < n ? p : n - 1];
        }
#pragma unroll
        for (int j = 0; j < kIds; ++j) {
            const int p = j * kThreads + tid;
            if (p >= n) ids[j] = -1;
            bad |= ids[j] >= E;
        }
        for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
        if (tid == 0) sbad = 0u;
        if constexpr (kDedup) {
            if (tid < kMaxTopK) ptok[0][tid] = 0;
        }
        lds_barrier();
#pragma unroll
        for (int j = 0; j < kIds; ++j)
            if (ids[j] >= 0 && ids[j] < E) atomicAdd(&cnt[ids[j]], 1);
        if (bad) sbad = 1u;
        if constexpr (kDedup) count_tokens(ids, 0);
        lds_barrier();
        if constexpr (kDedup) {
            // tokens per partition and their offsets; couple rows from M on are empty
            const int dtot = lane < P ? ptok[0][lane] : 0;
            const int pincl = wave_inclusive_scan(dtot);
            const int M = read_lane(pincl, P - 1);
            if (w == 0 && lane < P) {
                dd.part_tokens[lane] = dtot;
                dd.part_token_offset[lane] = pincl - dtot;
                if (lane == P - 1) dd.part_token_offset[P] = M;
            }
            for (int r = M + tid; r < (n / K) * P; r += kThreads) dd.tp_src[r] = -1;
        }
        int c[kPer], sum = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = tid * kPer + j;
            c[j] = (e < E) ? cnt[e] : 0;
            sum += c[j];
        }
        const int incl = wave_inclusive_scan(sum);
        if (lane == kWave - 1) wsum[w] = incl;
        lds_barrier();
        int base = 0, N = 0;
#pragma unroll
        for (int u = 0; u < kW; ++u) {
            const int ws = wsum[u];
            base += (u < w) ? ws : 0;
            N += ws;
        }
        int o = base + incl - sum;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = tid * kPer + j;
            if (e < E) {
                expert_count[e] = c[j];
                expert_offset[e] = o;
                cnt[e] = o;                  // this thread read cnt[e] above: no other reader
            }
            o += c[j];
        }
        if (tid == 0) {
            expert_offset[E] = N;
            part_offset[P] = N;
            *status = sbad ? 1u : 0u;
        }
        lds_barrier();
        const int L = E / P;
        for (int p = tid; p < P; p += kThreads) {
            const int lo = cnt[p * L];
            const int hi = (p + 1 < P) ? cnt[(p + 1) * L] : N;
            part_offset[p] = lo;
            part_count[p] = hi - lo;
        }
        for (int r = N + tid; r < n; r += kThreads) src_pair[r] = -1;
        return;
    }

    // every load issued before any result is used, the ids first (they need
    // no index arithmetic): this wave's share of all ids (addresses clamped;
    // they come from L2), then the own entries' ids and the x vector.  Loads
    // complete in issue order, so the counting below runs while x is still in
    // flight; the quantise follows.  The x load is unconditional (its address
    // clamped into x, the value unused where the item or the column is out of
    // range): a load under a branch would make the wait for the ids include it.
    int id[kIds];
#pragma unroll
    for (int j = 0; j < kIds; ++j) {
        const int p = j * kThreads + tid;
        id[j] = idx[p < n ? p : n - 1];
    }
    const int item0 = xcd_block(blockIdx.x - 1, gridDim.x - 1) * kW;
    const int item = item0 + w;
    const int last = (item0 + kW - 1 < n_items) ? item0 + kW - 1 : n_items - 1;
    const int t_lo = item0 / steps_per_token;
    const int r_lo = item0 - t_lo * steps_per_token;
    // token and step of item item0 + d (d < kW): one division for the
    // workgroup, then at most kW uniform subtractions
    auto token_of = [&](int d, int& r) {
        int tt = t_lo;
        r = r_lo + d;
        while (r >= steps_per_token) { r -= steps_per_token; ++tt; }
        return tt;
    };
    int r_hi;
    const int t_hi = token_of(last - item0, r_hi);
    const int nq = (t_hi - t_lo + 1) * K;    // own entries, <= kOwn (the launcher's choice)
    const int p_lo = t_lo * K;
    const int me = idx[p_lo + (lane < nq ? lane : 0)];
    int t = 0, col0 = H;
    if (item < n_items) {
        int r;
        t = token_of(w, r);
        col0 = r * kStepCols + lane * kColsPerLane;
    }
    const uint4 v = *reinterpret_cast<const uint4*>(x + (int64_t)t * H + (col0 < H ? col0 : 0));
    if constexpr (kDedup) {                  // while the loads are in flight
        if (tid < 2 * kMaxTopK) ptok[tid / kMaxTopK][tid % kMaxTopK] = 0;
        lds_barrier();
    }
    uint32_t key[kIds];
#pragma unroll
    for (int j = 0; j < kIds; ++j) {
        const int p = j * kThreads + tid;
        if (p >= n) id[j] = -1;
        key[j] = (id[j] >= 0 && id[j] < E) ? (((uint32_t)id[j] << 12) | (uint32_t)p) : 0xFFFFFFFFu;
    }
    const bool mvalid = lane < nq && me >= 0 && me < E;
    const uint32_t mkey = mvalid ? (((uint32_t)me << 12) | (uint32_t)(p_lo + lane)) : 0u;
    int below = 0;
#pragma unroll
    for (int j = 0; j < kOwn; ++j) {         // lanes past nq hold key 0: nothing below it
        const uint32_t qk = (uint32_t)read_lane((int)mkey, j);
        int c = 0;
#pragma unroll
        for (int r = 0; r < kIds; ++r) c += __builtin_popcountll(__ballot(key[r] < qk));
        if (lane == j) below = c;
    }
    if (lane < kOwn) part[lane][w] = below;
    if constexpr (kDedup) count_tokens(id, p_lo);
    float scale = 0.0f;
    uint2 q = make_uint2(0u, 0u);
    if (item < n_items) q = prepare_item<kPayload>(v, scale);
    lds_barrier();
    int myrow = 0;
#pragma unroll
    for (int u = 0; u < kW; ++u) myrow += part[lane < kOwn ? lane : 0][u];
    if (!mvalid) myrow = -1;
    if constexpr (kDedup) {
        // couple (t, lane) for lanes < P: the workgroup holds one token, t_lo
        const int dtot = lane < P ? ptok[0][lane] : 0;
        const int dbef = lane < P ? ptok[1][lane] : 0;
        const int pincl = wave_inclusive_scan(dtot);
        const int mpart = mvalid ? (int)partition_of(me) : -1;
        uint32_t m = 0u;                     // top-k mask of the couple
#pragma unroll
        for (int k = 0; k < kOwn; ++k)
            if (read_lane(mpart, k) == lane) m |= 1u << k;
        const int drow = (lane < P && m != 0u) ? pincl - dtot + dbef : -1;
        if (item < n_items)
            store_rows<kPayload, kMaxTopK>(v, q, scale, drow, 0, col0 - lane * kColsPerLane,
                                                 lane, H, P, (n / K) * P, recv_x, recv_scales);
        if (w == 1 && lane < P && t_lo * steps_per_token == item0) {   // the token's first workgroup
            const int j = t_lo * P + lane;
            dd.tp_row[j] = drow;
            dd.kmask[j] = m;
            if (drow >= 0) dd.tp_src[drow] = j;
        }
    } else {
        if (item < n_items)
            store_rows<kPayload, kOwn>(v, q, scale, myrow, (t - t_lo) * K,
                                             col0 - lane * kColsPerLane, lane, H, K, n, recv_x,
                                             recv_scales);
    }
    if (w == 0 && lane < nq) {
        // lane / K for lane < nq <= 16: (lane + 1/2) / K lies at least 1/32
        // from an integer and the reciprocal's error is below 2^-19, so the
        // truncated product is exact (a float reciprocal instead of an
        // integer division in the wave's tail)
        const int tt = t_lo + (int)(((float)lane + 0.5f) * __builtin_amdgcn_rcpf((float)K));
        if (tt * steps_per_token >= item0) {   // this workgroup holds the token's first step
            const int p = p_lo + lane;
            row_of_pair[p] = myrow;
            if (myrow >= 0) src_pair[myrow] = p;
        }
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

bool dispatch_launch_ok(int T, int H, MoveGeometry g)
{
    if (g.waves < 1 || g.waves > kMaxMoveWaves || g.max_blocks < 0) return false;
    if (g.slice_steps != 1 && g.slice_steps != 2) return false;
    const int64_t per_token = (int64_t)(H + g.slice_steps * kStepCols - 1) / (g.slice_steps * kStepCols);
    return (int64_t)T * per_token + kMaxGridBlocks * kMaxMoveWaves < ((int64_t)1 << 31);
}

hipError_t launch_dispatch(const uint16_t* x, int T, int H, int K, const int32_t* row_of_pair,
                           int payload, void* recv_x, float* recv_scales, hipStream_t stream,
                           MoveGeometry g)
{
    if (!dispatch_launch_ok(T, H, g)) return hipErrorInvalidValue;   // checked by the API first
    const int per_token = (H + g.slice_steps * kStepCols - 1) / (g.slice_steps * kStepCols);
    const int64_t items = (int64_t)T * per_token;
    if (items == 0) return hipSuccess;
    int64_t blocks = (items + g.waves - 1) / g.waves;
    if (g.max_blocks > 0 && blocks > g.max_blocks) blocks = g.max_blocks;
    if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
    const bool once = blocks * g.waves >= items;
    using Kernel = decltype(&dispatch_kernel<0, 8, 1, true>);
    // [payload][K <= 8 ? 0 : 1][slice of 1 or 2 steps][one item per wave]
    const Kernel table[2][2][2][2] = {
        {{{dispatch_kernel<0, 8, 1, false>, dispatch_kernel<0, 8, 1, true>},
          {dispatch_kernel<0, 8, 2, false>, dispatch_kernel<0, 8, 2, true>}},
         {{dispatch_kernel<0, 16, 1, false>, dispatch_kernel<0, 16, 1, true>},
          {dispatch_kernel<0, 16, 2, false>, dispatch_kernel<0, 16, 2, true>}}},
        {{{dispatch_kernel<1, 8, 1, false>, dispatch_kernel<1, 8, 1, true>},
          {dispatch_kernel<1, 8, 2, false>, dispatch_kernel<1, 8, 2, true>}},
         {{dispatch_kernel<1, 16, 1, false>, dispatch_kernel<1, 16, 1, true>},
          {dispatch_kernel<1, 16, 2, false>, dispatch_kernel<1, 16, 2, true>}}}};
    const Kernel k =
        table[payload == 0 ? 0 : 1][K <= 8 ? 0 : 1][g.slice_steps == 2 ? 1 : 0][once ? 1 : 0];
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(g.waves * kWave), 0, stream, x, H, K,
                       row_of_pair, (uint8_t*)recv_x, payload == 0 ? recv_scales : nullptr,
                       per_token, (int)items, T * K);
    return hipGetLastError();
}

bool fused_layout_dispatch_fits(int T, int H, int K)
{
    const int64_t steps = (H + kStepCols - 1) / kStepCols;
    return (int64_t)T * K <= kFusedMaxPairs && (int64_t)T * steps <= kMaxGridBlocks;
}

namespace {

// Most tokens the items of one W-wave workgroup can touch.
int max_own_tokens(int W, int steps)
{
    const int m = (W - 1 + steps - 1) / steps + 1;
    return m < W ? m : W;
}

// The same, exactly, for workgroups of W consecutive items out of n_items
// (workgroup b holds items W*b .. W*b+W-1).
int max_own_tokens_exact(int W, int steps, int n_items)
{
    int most = 0;
    const int period = (W * steps) / std::gcd(W, steps) / W;   // item0 mod steps repeats
    const int blocks = (n_items + W - 1) / W;
    for (int b = 0; b < period && b < blocks; ++b) {
        const int first = W * b;
        const int last = std::min(first + W - 1, n_items - 1);
        most = std::max(most, last / steps - first / steps + 1);
    }
    return most;
}

// Waves per fused workgroup.  Every workgroup redoes the whole histogram, so
// once 4-wave workgroups would outnumber the 256 CUs, 8-wave ones (half as
// many) finish sooner: measured at 128 x 7168, 5.8 against 6.1 us per
// launch; 16-wave ones were slower (7.0 us: every wave repeats the own-entry
// ranking).  Below that, 4 waves (at 4 and 16 tokens, 4.6 against 4.8 us).
// The workgroup's own entries must fit one wave.
int fused_waves(int64_t items, int steps, int K)
{
    if (items > 4 * kCUs && max_own_tokens(8, steps) * K <= kWave) return 8;
    return 4;
}

template <int kPayload, bool kDedup>
hipError_t launch_fused(int W, const int32_t* topk_idx, const uint16_t* x, int n, int H, int K,
                        int E, int P, int32_t* expert_count, int32_t* expert_offset,
                        int32_t* part_count, int32_t* part_offset, int32_t* row_of_pair,
                        int32_t* src_pair, uint32_t* status, void* recv_x, float* recv_scales,
                        int steps, int items, const DedupOutputs& dd, hipStream_t stream)
{
    // n >= 1: the kernel clamps its id addresses to n - 1
    if (n < 1 || (W != 4 && W != 8)) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((items + W - 1) / W);
    const bool small = n <= kFusedMaxPairs / 2;
    auto k = W == 8 ? (small ? layout_dispatch_kernel<kPayload, kDedup, 8, kFusedMaxPairs / 2>
                             : layout_dispatch_kernel<kPayload, kDedup, 8, kFusedMaxPairs>)
                    : (small ? layout_dispatch_kernel<kPayload, kDedup, 4, kFusedMaxPairs / 2>
                             : layout_dispatch_kernel<kPayload, kDedup, 4, kFusedMaxPairs>);
    hipLaunchKernelGGL(k, dim3(blocks), dim3(W * kWave), 0, stream, topk_idx, x, n, H, K, E, P,
                       expert_count, expert_offset, part_count, part_offset, row_of_pair, src_pair,
                       status, (uint8_t*)recv_x, kPayload == 0 ? recv_scales : nullptr, steps,
                       items, dd);
    return hipGetLastError();
}

// The counting kernel's instance for a payload, workgroup size (8, 7, 6 or,
// for plain entries, 4 waves) and own-entry bound (8 or 16); one extra
// workgroup, launch block 0.  n >= 1: the kernel clamps its id addresses to
// n - 1.
template <int kPayload, bool kDedup>
auto count_kernel(int W, bool own8)
{
    using Kernel = decltype(&layout_dispatch_count_kernel<kPayload, kDedup, 8, 8>);
    const Kernel w8[2] = {layout_dispatch_count_kernel<kPayload, kDedup, 8, 8>,
                          layout_dispatch_count_kernel<kPayload, kDedup, 8, 16>};
    const Kernel w7[2] = {layout_dispatch_count_kernel<kPayload, kDedup, 7, 8>,
                          layout_dispatch_count_kernel<kPayload, kDedup, 7, 16>};
    const Kernel w6[2] = {layout_dispatch_count_kernel<kPayload, kDedup, 6, 8>,
                          layout_dispatch_count_kernel<kPayload, kDedup, 6, 16>};
    const int o = own8 ? 0 : 1;
    if (W == 8) return w8[o];
    if (W == 7) return w7[o];
    if (W == 6) return w6[o];
    if constexpr (!kDedup) {
        const Kernel w4[2] = {layout_dispatch_count_kernel<kPayload, kDedup, 4, 8>,
                              layout_dispatch_count_kernel<kPayload, kDedup, 4, 16>};
        if (W == 4) return w4[o];
    }
    return Kernel(nullptr);
}

template <bool kDedup>
hipError_t launch_count(int payload, int W, bool own8, const int32_t* topk_idx, const uint16_t* x,
                        int n, int H, int K, int E, int P, int32_t* expert_count,
                        int32_t* expert_offset, int32_t* part_count, int32_t* part_offset,
                        int32_t* row_of_pair, int32_t* src_pair, uint32_t* status, void* recv_x,
                        float* recv_scales, int steps, int items, const DedupOutputs& dd,
                        hipStream_t stream)
{
    const auto k = payload == 0 ? count_kernel<0, kDedup>(W, own8) : count_kernel<1, kDedup>(W, own8);
    if (k == nullptr || n < 1) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((items + W - 1) / W) + 1;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(W * kWave), 0, stream, topk_idx, x, n, H, K, E, P,
                       expert_count, expert_offset, part_count, part_offset, row_of_pair, src_pair,
                       status, (uint8_t*)recv_x, payload == 0 ? recv_scales : nullptr, steps,
                       items, dd);
    return hipGetLastError();
}

}  // namespace

bool plan_layout_dispatch(int T, int H, int K, int waves, FusedPlan* plan)
{
    const int steps = (H + kStepCols - 1) / kStepCols;
    const int64_t items = (int64_t)T * steps;
    const int64_t n = (int64_t)T * K;
    if (T < 1 || n > kFusedMaxPairs || items > kMaxGridBlocks || waves < 0) return false;
    FusedPlan pl{};
    if (n <= kTinyPairs) {
        // one wave per item, waves per workgroup free (1, 2, 4 or 8; 4 by default)
        pl.kind = kFusedTiny;
        pl.waves = waves ? waves : kMoveWaves;
        if (pl.waves != 1 && pl.waves != 2 && pl.waves != 4 && pl.waves != 8) return false;
        pl.blocks = (unsigned)((items + pl.waves - 1) / pl.waves) + 1;
        *plan = pl;
        return true;
    }
    if (n <= kCountMaxPairs) {
        // by default workgroups of 8, 7 or 6 waves, the largest that divides
        // the steps per token (a workgroup then holds part of one token, or
        // whole tokens), else 8; 4 on request; own entries at most 16
        int W = waves;
        if (W == 0) {
            W = 8;
            for (int c = 8; c >= 6; --c)
                if (steps % c == 0 || c % steps == 0) { W = c; break; }
        }
        if (W == 4 || W == 6 || W == 7 || W == 8) {
            const int own = max_own_tokens_exact(W, steps, (int)items) * K;
            if (own <= 16) {
                pl.kind = kFusedCount;
                pl.waves = W;
                pl.own8 = own <= 8;
                pl.blocks = (unsigned)((items + W - 1) / W) + 1;
                *plan = pl;
                return true;
            }
        }
        if (waves != 0 && waves != 4 && waves != 8) return false;   // not a general-kernel size
    }
    // the general kernel: 4 or 8 waves, the workgroup's own entries within one wave
    pl.kind = kFusedGeneral;
    pl.waves = waves ? waves : fused_waves(items, steps, K);
    if (pl.waves != 4 && pl.waves != 8) return false;
    if (max_own_tokens(pl.waves, steps) * K > kWave) return false;
    pl.blocks = (unsigned)((items + pl.waves - 1) / pl.waves);
    *plan = pl;
    return true;
}

hipError_t launch_layout_dispatch(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K,
                                  int E, int P, int payload, int32_t* expert_count,
                                  int32_t* expert_offset, int32_t* part_count,
                                  int32_t* part_offset, int32_t* row_of_pair, int32_t* src_pair,
                                  uint32_t* status, void* recv_x, float* recv_scales,
                                  hipStream_t stream, int waves)
{
    FusedPlan pl;
    if (!plan_layout_dispatch(T, H, K, waves, &pl)) return hipErrorInvalidValue;  // checked first
    const int steps = (H + kStepCols - 1) / kStepCols;
    const int items = T * steps;
    const int n = T * K;
    if (pl.kind == kFusedTiny) {
        auto k = payload == 0 ? (K <= 8 ? layout_dispatch_tiny_kernel<0, 8> : layout_dispatch_tiny_kernel<0, 16>)
                              : (K <= 8 ? layout_dispatch_tiny_kernel<1, 8> : layout_dispatch_tiny_kernel<1, 16>);
        hipLaunchKernelGGL(k, dim3(pl.blocks), dim3(pl.waves * kWave), 0, stream, topk_idx, x, n, H,
                           K, E, P, expert_count, expert_offset, part_count, part_offset,
                           row_of_pair, src_pair, status, (uint8_t*)recv_x,
                           payload == 0 ? recv_scales : nullptr, steps, items);
        return hipGetLastError();
    }
    if (pl.kind == kFusedCount)
        return launch_count<false>(payload, pl.waves, pl.own8, topk_idx, x, n, H, K, E, P,
                                   expert_count, expert_offset, part_count, part_offset,
                                   row_of_pair, src_pair, status, recv_x, recv_scales, steps, items,
                                   DedupOutputs{}, stream);
    const DedupOutputs none{};
    return payload == 0
        ? launch_fused<0, false>(pl.waves, topk_idx, x, n, H, K, E, P, expert_count, expert_offset,
                                 part_count, part_offset, row_of_pair, src_pair, status, recv_x,
                                 recv_scales, steps, items, none, stream)
        : launch_fused<1, false>(pl.waves, topk_idx, x, n, H, K, E, P, expert_count, expert_offset,
                                 part_count, part_offset, row_of_pair, src_pair, status, recv_x,
                                 recv_scales, steps, items, none, stream);
}

bool plan_dedup_layout_dispatch(int T, int H, int K, int P, int waves, FusedPlan* plan)
{
    const int steps = (H + kStepCols - 1) / kStepCols;
    const int64_t items = (int64_t)T * steps;
    const int64_t n = (int64_t)T * K;
    if (T < 1 || n > kFusedMaxPairs || P > kMaxTopK || items > kMaxGridBlocks || waves < 0)
        return false;
    FusedPlan pl{};
    if (n <= kCountMaxPairs && (K & (K - 1)) == 0) {
        // the counting kernel: every workgroup inside one token (8, 7 or 6
        // waves dividing the steps per token, the largest by default), a
        // token's K entries on K aligned lanes (K a power of two, so K
        // divides 64)
        int W = 0;
        if (waves == 0) {
            for (int c = 8; c >= 6; --c)
                if (steps % c == 0) { W = c; break; }
        } else if (waves >= 6 && waves <= 8 && steps % waves == 0) {
            W = waves;
        }
        if (W != 0) {
            pl.kind = kFusedCount;
            pl.waves = W;
            pl.own8 = K <= 8;
            pl.blocks = (unsigned)((items + W - 1) / W) + 1;
            *plan = pl;
            return true;
        }
    }
    // the general kernel: 4 or 8 waves, the workgroup's own entries within one wave
    pl.kind = kFusedGeneral;
    pl.waves = waves ? waves : fused_waves(items, steps, K);
    if (pl.waves != 4 && pl.waves != 8) return false;
    if (max_own_tokens(pl.waves, steps) * K > kWave) return false;
    pl.blocks = (unsigned)((items + pl.waves - 1) / pl.waves);
    *plan = pl;
    return true;
}

hipError_t launch_dedup_layout_dispatch(const int32_t* topk_idx, const uint16_t* x, int T, int H,
                                        int K, int E, int P, int payload, int32_t* expert_count,
                                        int32_t* expert_offset, int32_t* part_count,
                                        int32_t* part_offset, int32_t* row_of_pair,
                                        int32_t* src_pair, int32_t* tp_row, int32_t* part_tokens,
                                        int32_t* part_token_offset, int32_t* tp_src,
                                        uint32_t* kmask, uint32_t* status, void* recv_x,
                                        float* recv_scales, hipStream_t stream, int waves)
{
    FusedPlan pl;
    if (!plan_dedup_layout_dispatch(T, H, K, P, waves, &pl)) return hipErrorInvalidValue;
    const int steps = (H + kStepCols - 1) / kStepCols;
    const int items = T * steps;
    const int n = T * K;
    const DedupOutputs dd{tp_row, part_tokens, part_token_offset, tp_src, kmask};
    if (pl.kind == kFusedCount)
        return launch_count<true>(payload, pl.waves, pl.own8, topk_idx, x, n, H, K, E, P,
                                  expert_count, expert_offset, part_count, part_offset,
                                  row_of_pair, src_pair, status, recv_x, recv_scales, steps, items,
                                  dd, stream);
    return payload == 0
        ? launch_fused<0, true>(pl.waves, topk_idx, x, n, H, K, E, P, expert_count, expert_offset,
                                part_count, part_offset, row_of_pair, src_pair, status, recv_x,
                                recv_scales, steps, items, dd, stream)
        : launch_fused<1, true>(pl.waves, topk_idx, x, n, H, K, E, P, expert_count, expert_offset,
                                part_count, part_offset, row_of_pair, src_pair, status, recv_x,
                                recv_scales, steps, items, dd, stream);
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
