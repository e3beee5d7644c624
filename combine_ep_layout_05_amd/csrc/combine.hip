// combine.hip -- gather each token's top-k expert outputs and reduce them in
// fp32 with the top-k weights, written out as bf16 (gfx950).
//
// out[t, c] = bf16_rne(acc); acc = 0.0f, then for k = 0..K-1 with
// r = row_of_pair[t*K+k] >= 0: acc = fmaf(w[t,k], y[r, c], acc).
// The expert outputs y are read in place from the caller's buffer, in the
// receive-row layout of the dispatch (MoRI PR #614 "perf(ep): InterNodeV1LL
// low-token latency on MI300X + CX7", zero-copy combine paragraph: no
// staging copy of the combine input).
//
// Work split: one wave per (token, 512-column step), items strided flatly
// over the whole grid (waves per workgroup and workgroup count from the
// launch geometry) -- partitioning by (token, hidden slice) rather than by
// token keeps every wave busy at small token counts (same PR, CombineSync
// paragraph), and 512 columns per wave is the floor the same PR measured
// best (MultiWarpIter paragraph).  Each lane owns 8 columns: it issues all of
// its K 16-byte loads (one per expert row, each wave-wide load a contiguous
// 1 KB) before the first FMA so the K rows are in flight together, then
// accumulates in k order and stores 16 bytes of bf16.
//
// The same kernel runs the two levels of the per-destination (dedup) combine
// (UCCL PR #749: tokens batched per destination; MoRI PR #614,
// DispatchIntraNode paragraph: one copy of a token per destination):
//   partial: for each partition holding a copy of the token, sums in k order
//            only the top-k entries whose bit is set in that copy's mask and
//            writes the bf16 partial to the copy's row;
//   reduce:  adds the token's partial rows in partition order (weight 1:
//            fmaf(1, v, acc) is the correctly rounded acc + v) and writes
//            the bf16 result.
#include "ep_device.h"
#include "ep_launch.h"
#include "ep_numerics.h"

namespace ep {
namespace {

enum CombineMode { kPlain = 0, kPartial = 1, kReduce = 2 };

// acc[0..7] = fmaf over k = 0..K-1 in order, for the k with bit k of `use`
// set and a source row (row_k >= 0), of w_k * y[row_k, 8 columns].  rows and
// weights are lane-k values of `myrow` / `myw`; v[k] holds the loaded columns.
template <int kMaxK>
__device__ __forceinline__ uint4 reduce_rows(const uint4 (&v)[kMaxK], int myrow, float myw, int K,
                                             uint32_t use)
{
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        if (k < K && ((use >> k) & 1u)) {
            const int r = read_lane(myrow, k);
            if (r >= 0) {
                const float wk = __builtin_bit_cast(float, read_lane(__builtin_bit_cast(int, myw), k));
                acc[0] = __builtin_fmaf(wk, bf16_lo(v[k].x), acc[0]);
                acc[1] = __builtin_fmaf(wk, bf16_hi(v[k].x), acc[1]);
                acc[2] = __builtin_fmaf(wk, bf16_lo(v[k].y), acc[2]);
                acc[3] = __builtin_fmaf(wk, bf16_hi(v[k].y), acc[3]);
                acc[4] = __builtin_fmaf(wk, bf16_lo(v[k].z), acc[4]);
                acc[5] = __builtin_fmaf(wk, bf16_hi(v[k].z), acc[5]);
                acc[6] = __builtin_fmaf(wk, bf16_lo(v[k].w), acc[6]);
                acc[7] = __builtin_fmaf(wk, bf16_hi(v[k].w), acc[7]);
            }
        }
    }
    uint4 o;
    o.x = pack2_bf16(acc[0], acc[1]);
    o.y = pack2_bf16(acc[2], acc[3]);
    o.z = pack2_bf16(acc[4], acc[5]);
    o.w = pack2_bf16(acc[6], acc[7]);
    return o;
}

// Combine level 1 for one item when every entry is in at most one partition's
// mask: lane k < K holds the entry's receive row `myrow`, weight `myw` and
// partition `pk` (-1: in no mask), lane p < P the couple's partial row `prow`
// (-1: no copy).  Entries are ranked by (partition, k); the rows are loaded in
// that order, so the reduction runs through them once with static register
// indices, storing a partition's bf16 sum after its last entry.  The fmaf
// order within a partition is ascending k, as in the general loop.  A copy
// none of whose entries has a row gets +0, as there.
template <int kMaxK, bool kStream>
__device__ __forceinline__ void partial_in_order(const uint16_t* __restrict__ y,
                                                 uint16_t* __restrict__ out, int H, int col0,
                                                 bool active, int lane, int myrow, float myw,
                                                 int pk, int prow, int4* __restrict__ ord)
{
    const bool valid = pk >= 0 && myrow >= 0;            // lanes >= K have pk = -1
    const int key = valid ? (pk << 5) | lane : 0x7FFFFFFF;
    int rank = 0;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) rank += (read_lane(key, k) < key) ? 1 : 0;
    const int nv = __builtin_popcountll(__ballot(valid));
    uint4 v[kMaxK];
    float w[kMaxK];
    int part[kMaxK + 1];
    // the loads in rank order with no branch around them (past nv: row 0;
    // past H: column 0; both in bounds and unused), so the reduction below
    // waits for one row at a time
    // The entries in that order through LDS (`ord`, this wave's kMaxTopK
    // slots): lane k writes its row, weight and partition to slot rank, lane
    // j reads slot j back (one wave: wave_lds_sync between write and read,
    // no workgroup barrier).
    if (valid) ord[rank] = make_int4(myrow, __builtin_bit_cast(int, myw), pk, 0);
    wave_lds_sync();
    const int4 o = lane < nv ? ord[lane] : make_int4(0, 0, -1, 0);
    const int cl = active ? col0 : 0;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        const int r = read_lane(o.x, j);
        w[j] = __builtin_bit_cast(float, read_lane(o.y, j));
        part[j] = read_lane(o.z, j);
        v[j] = load16<kStream>(y + (int64_t)r * H + cl);
        __builtin_amdgcn_sched_barrier(0);
    }
    part[kMaxK] = -1;
    uint64_t written = 0;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // The fmaf runs for every slot, so no load is sunk into a branch that
    // uses it (which would issue it last): slots past nv come after every
    // entry, and what they add is never stored.
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        acc[0] = __builtin_fmaf(w[j], bf16_lo(v[j].x), acc[0]);
        acc[1] = __builtin_fmaf(w[j], bf16_hi(v[j].x), acc[1]);
        acc[2] = __builtin_fmaf(w[j], bf16_lo(v[j].y), acc[2]);
        acc[3] = __builtin_fmaf(w[j], bf16_hi(v[j].y), acc[3]);
        acc[4] = __builtin_fmaf(w[j], bf16_lo(v[j].z), acc[4]);
        acc[5] = __builtin_fmaf(w[j], bf16_hi(v[j].z), acc[5]);
        acc[6] = __builtin_fmaf(w[j], bf16_lo(v[j].w), acc[6]);
        acc[7] = __builtin_fmaf(w[j], bf16_hi(v[j].w), acc[7]);
        if (j < nv) {
            if (j + 1 >= nv || part[j + 1] != part[j]) {     // last entry of this partition
                const int orow = read_lane(prow, part[j]);
                uint4 o;
                o.x = pack2_bf16(acc[0], acc[1]);
                o.y = pack2_bf16(acc[2], acc[3]);
                o.z = pack2_bf16(acc[4], acc[5]);
                o.w = pack2_bf16(acc[6], acc[7]);
                if (active) store16<kStream>(out + (int64_t)orow * H + col0, o);
                written |= 1ull << part[j];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
            }
        }
    }
    // copies with no entry that has a row: +0
    uint64_t empty = __ballot(prow >= 0) & ~written;
    while (empty) {
        const int p = __builtin_ctzll(empty);
        empty &= empty - 1;
        if (active) store16<kStream>(out + (int64_t)read_lane(prow, p) * H + col0,
                                     make_uint4(0, 0, 0, 0));
    }
}

// An item is (token t, 512-column step).  Its K source rows are
// row_of_pair[t*K ..] (tp_row with K = P for reduce, weight 1).
// Plain and reduce write row t of `out`.  Partial loads the token's K expert
// rows once and, for each partition p with a copy of t (tp_row[t*P+p] >= 0,
// taken in ascending p), reduces the entries of kmask[t*P+p] into row
// tp_row[t*P+p] of `out`: every expert row is read once, as in the plain
// combine, and no wave is spent on (token, partition) couples without a copy.
// kSub: 512-column steps per item (the slice of the launch geometry, 1 or 2;
// the partial mode takes 1), items_per_token = ceil(steps / kSub).
template <int kMaxK, bool kStream, int kMode, int kSub, bool kOnce>
__global__ __launch_bounds__(kMaxMoveWaves * kWave) void combine_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ row_of_pair,
    const float* __restrict__ topk_w, int H, int K, uint16_t* __restrict__ out,
    int items_per_token, int n_items, int n_rows,
    const int32_t* __restrict__ tp_row, const uint32_t* __restrict__ kmask, int P, int out_rows)
{
    static_assert(kSub == 1 || kMode != kPartial, "the partial mode takes one step per item");
    const int lane = threadIdx.x % kWave;
    const int waves = blockDim.x / kWave;
    const int stride = gridDim.x * waves;
    // cached regime: the XCD-contiguous block order, so a token's items run on
    // the XCD that wrote its metadata; streaming regime: launch order (there
    // the contiguous order measured slower, 88 -> 97 us at 4096 x 7168)
    const int block = kStream ? (int)blockIdx.x : xcd_block(blockIdx.x, gridDim.x);
    // partial mode: per wave, entry k -> partition of the copy whose mask holds it
    __shared__ int32_t s_pk[kMode == kPartial ? kMaxMoveWaves : 1][kMaxTopK];
    // partial mode: per wave, the entries in (partition, k) order
    __shared__ int4 s_ord[kMode == kPartial ? kMaxMoveWaves : 1][kMaxTopK];
    auto run = [&](int item) {
        const int t = item / items_per_token;
        const int col_base = (item - t * items_per_token) * (kSub * kStepCols);
        const int col0 = col_base + lane * kColsPerLane;
        const bool active = col0 < H;
        // metadata loads without a branch around them (lanes past K or P read
        // a valid entry, whose value is then dropped): a load under a branch
        // costs its own wait for the argument pointer and for the data.  One
        // empty asm statement takes every loaded value as an operand after
        // all are issued, so the compiler neither sinks a load into the lanes
        // that use it nor waits for one before issuing the next.
        const int kl = lane < K ? lane : 0;
        int myrow = row_of_pair[(int64_t)t * K + kl];
        float myw = 1.0f;
        if constexpr (kMode != kReduce) myw = topk_w[(int64_t)t * K + kl];
        int prow = -1;
        uint32_t pmask = 0u;
        if constexpr (kMode == kPartial) {
            const int pl = lane < P ? lane : 0;
            prow = tp_row[(int64_t)t * P + pl];
            pmask = kmask[(int64_t)t * P + pl];
        }
        // (y as an input: its argument load is issued with these too)
        asm volatile("" : "+v"(myrow), "+v"(myw), "+v"(prow), "+v"(pmask) : "s"(y));
        if (lane >= K || myrow >= n_rows) myrow = -1;   // past n_rows: treated as masked
        if (lane >= K) myw = 0.0f;
        if constexpr (kMode == kPartial)
            if (lane >= P || prow >= out_rows) { prow = -1; pmask = 0u; }

        if constexpr (kMode == kPartial) {
            // When no entry is in two masks (always, for the masks of
            // ep_dedup_layout) the K rows are loaded in (partition, k) order
            // and reduced in one pass, closing a partition's sum at its last
            // entry; overlapping masks take the general loop below.  The
            // masks overlap unless their popcounts add up to the popcount of
            // their OR, both reduced over the couple lanes p < P <= 16 (one
            // DPP row: the butterfly leaves the row's total in every lane).
            // The entry -> partition map is then transposed through LDS: each
            // couple lane writes its partition into the slot of every entry
            // of its mask, and lane k reads slot k back -- within one wave, so
            // wave_lds_sync orders the hand-offs and no workgroup barrier is
            // needed.
            const uint32_t kbits = (uint32_t)((1ull << K) - 1ull);
            uint32_t m = prow >= 0 ? (pmask & kbits) : 0u;
            int orv = (int)m, cnt = __builtin_popcount(m);
            orv |= __builtin_amdgcn_update_dpp(0, orv, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
            cnt += __builtin_amdgcn_update_dpp(0, cnt, 0xB1, 0xF, 0xF, false);
            orv |= __builtin_amdgcn_update_dpp(0, orv, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
            cnt += __builtin_amdgcn_update_dpp(0, cnt, 0x4E, 0xF, 0xF, false);
            orv |= __builtin_amdgcn_update_dpp(0, orv, 0x141, 0xF, 0xF, false);   // row_half_mirror
            cnt += __builtin_amdgcn_update_dpp(0, cnt, 0x141, 0xF, 0xF, false);
            orv |= __builtin_amdgcn_update_dpp(0, orv, 0x140, 0xF, 0xF, false);   // row_mirror
            cnt += __builtin_amdgcn_update_dpp(0, cnt, 0x140, 0xF, 0xF, false);
            const bool overlap =
                read_lane(cnt, 0) != __builtin_popcount((uint32_t)read_lane(orv, 0));
            if (!overlap) {
                int32_t* const slot = s_pk[threadIdx.x / kWave];
                if (lane < kMaxTopK) slot[lane] = -1;
                wave_lds_sync();
                while (m) {                       // this couple's entries
                    const int k = __builtin_ctz(m);
                    m &= m - 1u;
                    slot[k] = lane;
                }
                wave_lds_sync();
                const int pk = lane < K ? slot[lane] : -1;
                partial_in_order<kMaxK, kStream>(y, out, H, col0, active, lane, myrow, myw, pk,
                                                 prow, s_ord[threadIdx.x / kWave]);
                return;
            }
        }

        if constexpr (kMode == kReduce) {
            // Up to 8 copies of the token (always, when the top-k is 8 or
            // less): the present couples compacted in ascending p into 8
            // scalar rows, then 8 row loads issued back to back with no branch
            // around them (past the copies: row 0, in bounds, never added),
            // as in the plain mode, instead of P loads each behind its own
            // branch.  128 x 7168 top-8, 16 partitions, graphs of 50 launches
            // on MI355X: 3.60 -> 2.91 us per launch, dedup step 14.30 -> 13.71
            // us (E = 32, P = 8: 3.05 -> 2.88 and 13.17 -> 13.07 us).
            uint64_t present = __ballot(myrow >= 0);       // lanes < P only
            if (__builtin_popcountll(present) <= 8) {
                int rows[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int p = present ? (int)__builtin_ctzll(present) : 0;
                    rows[j] = present ? read_lane(myrow, p) : -1;
                    present &= present - 1;
                }
                const int cl = active ? col0 : 0;
                uint4 v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    v[j] = load16<kStream>(y + (int64_t)(rows[j] >= 0 ? rows[j] : 0) * H + cl);
                    __builtin_amdgcn_sched_barrier(0);     // issue in p order, the add order
                }
                float acc[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (rows[j] >= 0) {                    // fmaf(1, v, acc) = acc + v, rounded once
                        acc[0] = __builtin_fmaf(1.0f, bf16_lo(v[j].x), acc[0]);
                        acc[1] = __builtin_fmaf(1.0f, bf16_hi(v[j].x), acc[1]);
                        acc[2] = __builtin_fmaf(1.0f, bf16_lo(v[j].y), acc[2]);
                        acc[3] = __builtin_fmaf(1.0f, bf16_hi(v[j].y), acc[3]);
                        acc[4] = __builtin_fmaf(1.0f, bf16_lo(v[j].z), acc[4]);
                        acc[5] = __builtin_fmaf(1.0f, bf16_hi(v[j].z), acc[5]);
                        acc[6] = __builtin_fmaf(1.0f, bf16_lo(v[j].w), acc[6]);
                        acc[7] = __builtin_fmaf(1.0f, bf16_hi(v[j].w), acc[7]);
                    }
                }
                uint4 o;
                o.x = pack2_bf16(acc[0], acc[1]);
                o.y = pack2_bf16(acc[2], acc[3]);
                o.z = pack2_bf16(acc[4], acc[5]);
                o.w = pack2_bf16(acc[6], acc[7]);
                if (active) store16<true>(out + (int64_t)t * H + col0, o);
                return;
            }
        }
        if constexpr (kMode != kPartial) {
            // the K rows and weights moved to scalar registers once, then
            // every row load issued before the first fmaf, in k order.  Plain
            // mode: no branch around them (a missing row reads row 0 and a
            // column past H column 0, both in bounds, and the fmaf loop skips
            // what is not a row), so the loads go out back to back and the
            // loop waits for them one at a time.  Reduce mode with more than
            // 8 copies skips absent couples with a uniform branch instead.
            // With kSub = 2 each row's two 16-byte pieces (columns 512 apart)
            // are loaded together.
            int rows[kMaxK];
            float wts[kMaxK];
#pragma unroll
            for (int k = 0; k < kMaxK; ++k) {
                rows[k] = (k < K) ? read_lane(myrow, k) : -1;
                wts[k] = __builtin_bit_cast(float, read_lane(__builtin_bit_cast(int, myw), k));
            }
            int cl[kSub];
#pragma unroll
            for (int u = 0; u < kSub; ++u) {
                const int c = col0 + u * kStepCols;
                cl[u] = c < H ? c : 0;
            }
            uint4 v[kMaxK][kSub];
#pragma unroll
            for (int k = 0; k < kMaxK; ++k) {
#pragma unroll
                for (int u = 0; u < kSub; ++u) {
                    if constexpr (kMode == kReduce) {
                        v[k][u] = make_uint4(0, 0, 0, 0);
                        if (rows[k] >= 0) v[k][u] = load16<kStream>(y + (int64_t)rows[k] * H + cl[u]);
                    } else {
                        v[k][u] = load16<kStream>(y + (int64_t)(rows[k] >= 0 ? rows[k] : 0) * H + cl[u]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);      // issue in k order, the fmaf order
            }
#pragma unroll
            for (int u = 0; u < kSub; ++u) {
                float acc[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
                for (int k = 0; k < kMaxK; ++k) {
                    if (rows[k] >= 0) {
                        acc[0] = __builtin_fmaf(wts[k], bf16_lo(v[k][u].x), acc[0]);
                        acc[1] = __builtin_fmaf(wts[k], bf16_hi(v[k][u].x), acc[1]);
                        acc[2] = __builtin_fmaf(wts[k], bf16_lo(v[k][u].y), acc[2]);
                        acc[3] = __builtin_fmaf(wts[k], bf16_hi(v[k][u].y), acc[3]);
                        acc[4] = __builtin_fmaf(wts[k], bf16_lo(v[k][u].z), acc[4]);
                        acc[5] = __builtin_fmaf(wts[k], bf16_hi(v[k][u].z), acc[5]);
                        acc[6] = __builtin_fmaf(wts[k], bf16_lo(v[k][u].w), acc[6]);
                        acc[7] = __builtin_fmaf(wts[k], bf16_hi(v[k][u].w), acc[7]);
                    }
                }
                uint4 o;
                o.x = pack2_bf16(acc[0], acc[1]);
                o.y = pack2_bf16(acc[2], acc[3]);
                o.z = pack2_bf16(acc[4], acc[5]);
                o.w = pack2_bf16(acc[6], acc[7]);
                // the output row is nontemporal at every size: no later access
                // of this launch or the next one wants it in L2 (128 x 7168
                // top-8, graphs of 50 steps on MI355X: step 6.97 -> 6.78 us
                // warm, 9.94 -> 9.41 us over 16 rotating input sets; 4 and 4096
                // tokens unchanged)
                const int c = col0 + u * kStepCols;
                if (c < H) store16<true>(out + (int64_t)t * H + c, o);
            }
        } else {
            // level 1 with overlapping masks: for each copy in ascending p, the
            // entries of its mask in ascending k
            uint4 v[kMaxK];
#pragma unroll
            for (int k = 0; k < kMaxK; ++k) {
                v[k] = make_uint4(0, 0, 0, 0);
                if (k < K) {
                    const int r = read_lane(myrow, k);
                    if (r >= 0 && active) v[k] = load16<kStream>(y + (int64_t)r * H + col0);
                }
            }
            uint64_t present = __ballot(prow >= 0);   // lanes < P only: prow is -1 elsewhere
            while (present) {
                const int p = __builtin_ctzll(present);
                present &= present - 1;
                const uint32_t use = (uint32_t)read_lane((int)pmask, p);
                const int orow = read_lane(prow, p);
                const uint4 o = reduce_rows<kMaxK>(v, myrow, myw, K, use);
                if (active) store16<kStream>(out + (int64_t)orow * H + col0, o);
            }
        }
    };
    int item = block * waves + wave_uniform(threadIdx.x / kWave);
    if constexpr (kOnce) {               // the grid covers every item: no loop
        if (item < n_items) run(item);
    } else {
        for (; item < n_items; item += stride)   // n_items + stride < 2^31 (checked by the launcher)
            run(item);
    }
}

constexpr int64_t kMaxGridBlocks = 1 << 20;

// Streaming (nontemporal) expert-output reads (and partial-row writes) once
// the gathered rows exceed what the caches can usefully hold: measured on
// MI355X at 4096 x 7168 top-8 right after a dispatch, the combine went 132 ->
// 96 us because its once-read rows no longer evict the dispatch's fresh lines.
// Below that the reads stay cached: nontemporal reads of cache-resident rows
// measured slower (128 x 7168 step 6.97 -> 7.42 us).
// EP_FORCE_POLICY (build option for A/B runs): 1 = cached combine accesses,
// 2 or more = streaming ones, whatever the size.
bool combine_streams(int64_t gathered_rows, int H)
{
#if defined(EP_FORCE_POLICY)
    if (EP_FORCE_POLICY == 1) return false;
    if (EP_FORCE_POLICY >= 2) return true;
#endif
    return gathered_rows * H * 2 >= kStreamMinBytes;
}

}  // namespace

bool combine_streaming(int T, int H, int K)
{
    return combine_streams((int64_t)T * K, H);
}

// The streaming regime's combine in 2-wave workgroups, the cached one in
// kDefaultGeometry's 4: measured on MI355X with the step's own inputs
// (graphs of 20 steps, interleaved), 4096 x 7168 top-8 Zipf routing: step
// 146.0 -> 143.4 us (combine alone 90.8 -> 88.2 us), 16384 x 4096 bf16 with
// 10 % of entries masked: step 381.9 -> 373.7 us (189.5 -> 182.9 us); 1 and 8
// waves in between, 4 the slowest of the four in both.  At 4 to 128 tokens
// no geometry beat 4 waves by 2 % in the step.
MoveGeometry combine_default_geometry(int T, int H, int K)
{
    return combine_streaming(T, H, K) ? MoveGeometry{2, 0, 1} : kDefaultGeometry;
}

bool combine_launch_ok(int n_units, int H, MoveGeometry g)
{
    if (g.waves < 1 || g.waves > kMaxMoveWaves || g.max_blocks < 0) return false;
    if (g.slice_steps != 1 && g.slice_steps != 2) return false;
    const int64_t per_unit = (int64_t)(H + g.slice_steps * kStepCols - 1) / (g.slice_steps * kStepCols);
    return (int64_t)n_units * per_unit + kMaxGridBlocks * kMaxMoveWaves < ((int64_t)1 << 31);
}

namespace {

template <int kMode>
hipError_t launch_combine_mode(const uint16_t* y, const int32_t* row_of_pair,
                               const float* topk_w, int n_units, int H, int K, int n_rows,
                               const int32_t* tp_row, const uint32_t* kmask, int P, int out_rows,
                               int64_t gathered_rows, uint16_t* out, hipStream_t stream,
                               MoveGeometry g)
{
    if (!combine_launch_ok(n_units, H, g) || (kMode == kPartial && g.slice_steps != 1))
        return hipErrorInvalidValue;                   // checked by the API first
    const int per_unit = (H + g.slice_steps * kStepCols - 1) / (g.slice_steps * kStepCols);
    const int64_t items = (int64_t)n_units * per_unit;
    if (items == 0) return hipSuccess;
    int64_t blocks = (items + g.waves - 1) / g.waves;
    if (g.max_blocks > 0 && blocks > g.max_blocks) blocks = g.max_blocks;
    if (blocks > kMaxGridBlocks) blocks = kMaxGridBlocks;
    const bool stream_policy = combine_streams(gathered_rows, H);
    const bool once = blocks * g.waves >= items;
    constexpr int kS2 = kMode == kPartial ? 1 : 2;     // the partial mode has no 2-step slice
    using Kernel = decltype(&combine_kernel<8, true, kMode, 1, true>);
    // [K <= 8 ? 0 : 1][streaming][slice of 1 or 2 steps][one item per wave]
    const Kernel table[2][2][2][2] = {
        {{{combine_kernel<8, false, kMode, 1, false>, combine_kernel<8, false, kMode, 1, true>},
          {combine_kernel<8, false, kMode, kS2, false>, combine_kernel<8, false, kMode, kS2, true>}},
         {{combine_kernel<8, true, kMode, 1, false>, combine_kernel<8, true, kMode, 1, true>},
          {combine_kernel<8, true, kMode, kS2, false>, combine_kernel<8, true, kMode, kS2, true>}}},
        {{{combine_kernel<16, false, kMode, 1, false>, combine_kernel<16, false, kMode, 1, true>},
          {combine_kernel<16, false, kMode, kS2, false>, combine_kernel<16, false, kMode, kS2, true>}},
         {{combine_kernel<16, true, kMode, 1, false>, combine_kernel<16, true, kMode, 1, true>},
          {combine_kernel<16, true, kMode, kS2, false>, combine_kernel<16, true, kMode, kS2, true>}}}};
    const Kernel k = table[K <= 8 ? 0 : 1][stream_policy ? 1 : 0][g.slice_steps == 2 ? 1 : 0]
                          [once ? 1 : 0];
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(g.waves * kWave), 0, stream, y, row_of_pair,
                       topk_w, H, K, out, per_unit, (int)items, n_rows, tp_row, kmask, P, out_rows);
    return hipGetLastError();
}

// The two dedup combine levels: one wave per workgroup, uncapped.  In the
// XCD-contiguous order every XCD still holds one contiguous range of tokens,
// as in the fused dedup dispatch before them, so each level reads the masks,
// row maps and partial rows of a token on the XCD that wrote them.  Measured
// in graphs of 50 dedup steps on MI355X (top-8, hidden 7168, 16 partitions):
// 128 tokens 14.57 -> 14.50 us (another box 14.49 -> 14.33) against 8-wave
// workgroups, 16 tokens 11.10 -> 10.66, 256 tokens 23.85 -> 23.58; 2- and
// 4-wave workgroups in between (timed alone, without the launch before it,
// the reduce level is 0.1 us faster with 2 waves than with 1).  Also in the
// streaming regime: 4096 x 7168 fp8, 8 partitions, 255.2 -> 252.2 us; 16384 x
// 4096 bf16 600.1 -> 592.5 us; 1024 x 7168 80.8 -> 79.1 us.
MoveGeometry dedup_geometry()
{
    return MoveGeometry{1, 0, 1};
}

}  // namespace

hipError_t launch_combine(const uint16_t* y, const int32_t* row_of_pair, const float* topk_w,
                          int T, int H, int K, uint16_t* out, hipStream_t stream, MoveGeometry g)
{
    return launch_combine_mode<kPlain>(y, row_of_pair, topk_w, T, H, K, T * K, nullptr, nullptr,
                                       1, T, (int64_t)T * K, out, stream, g);
}

hipError_t launch_combine_partial(const uint16_t* y, const int32_t* row_of_pair,
                                  const float* topk_w, const int32_t* tp_row,
                                  const uint32_t* kmask, int T, int H, int K, int P,
                                  uint16_t* partial, hipStream_t stream)
{
    return launch_combine_mode<kPartial>(y, row_of_pair, topk_w, T, H, K, T * K, tp_row, kmask, P,
                                         T * P, (int64_t)T * K, partial, stream,
                                         dedup_geometry());
}

hipError_t launch_combine_reduce(const uint16_t* partial, const int32_t* tp_row, int T, int H,
                                 int P, uint16_t* out, hipStream_t stream)
{
    return launch_combine_mode<kReduce>(partial, tp_row, nullptr, T, H, P, T * P, nullptr, nullptr,
                                        1, T, (int64_t)T * P, out, stream, dedup_geometry());
}

}  // namespace ep
