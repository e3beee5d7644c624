// layout.hip -- per-expert / per-destination counts, exclusive scans and
// deterministic receive slots for MoE expert-parallel dispatch (gfx950).
//
// What is computed (UCCL PR #749 "[EP] Low-latency mode batch tokens per
// destination": a destination's batch is the sum of its local experts'
// counts; MoRI PR #614 "perf(ep): InterNodeV1LL low-token latency on MI300X +
// CX7", DispatchIntraNode paragraph: work items are the flat (t, k) entries
// t*K + i; routing-scan paragraph: negative ids are sentinels):
//   count[e], offset = exclusive scan of count, part_count[p] = sum of count
//   over experts p*L .. p*L+L-1, part_offset[p] = offset[p*L], and for every
//   valid entry row = offset[e] + (number of earlier entries, in flat (t, k)
//   order, with the same expert).
//
// The pages' systems learn each destination's size by spinning on
// per-expert completion counters and claim slots with atomics, which makes
// the slot order depend on timing.  Here the counts are known before any
// payload moves and slots come from prefix sums only:
//   - in-wave rank: the lanes holding the same expert ("peers") are found
//     with one ballot per bit of the expert id (match-any); a lane's rank is
//     the number of its peers in lower lanes (mbcnt), the lowest peer is the
//     group leader;
//   - across the 16 waves of a round: each leader writes its group size to
//     an LDS table [wave][expert]; one thread per expert turns its column
//     into an exclusive prefix over waves;
//   - across rounds: a running per-expert cursor in LDS;
//   - across workgroups (large batches): per-chunk histograms in the
//     workspace; each ranking workgroup derives its chunk's per-expert bases
//     from all chunk histograms (a separate scan launch only above 256
//     chunks).
// Plain entries up to 2048 skip the histogram-and-scan ranks: an entry's
// slot is the number of valid (expert, entry) keys below its own, counted
// with ballots by many workgroups at once (layout_count_kernel).
// Every id is loaded once, up front, and the match-any peers found while
// building the histogram are reused for the ranks.  Scans use DPP wave scans.
// No atomic's return value ever decides a slot, so the result is the same on
// every run.  LDS atomics are used only for order-free histogram sums.
#include <type_traits>

#include "ep_device.h"
#include "ep_launch.h"

namespace ep {
namespace {

constexpr int kSmallRounds = kSmallMaxPairs / kLayoutThreads;   // 2
constexpr int kChunkRounds = kChunkPairs / kLayoutThreads;      // 2

struct LayoutSmem {
    int32_t hist[kMaxExperts];
    int32_t cursor[kMaxExperts];
    uint16_t wtab[kLayoutWaves][kMaxExperts];   // per-wave group sizes / prefixes
    int32_t wsum[kLayoutWaves];
    uint32_t bad;
    int32_t total;
};

// Where a layout entry's id comes from.
//   Plain: entry p is the (t, k) pair p = t*K + k; its id is topk_idx[p] and an
//   id >= E is reported as bad.
//   Dedup: entry j is the (token, partition) couple j = t*P + p of the
//   per-destination layout (UCCL PR #749: tokens batched per destination;
//   MoRI PR #614, DispatchIntraNode paragraph: one copy of a token per
//   destination).  Its id is p when token t has a valid expert in partition
//   p, else -1, so the layout over ids 0..P-1 gives every present couple a
//   row in token order within its partition.  The top-k entries served by
//   that copy form a bit mask (bit k), written out when `kmask` is set; bad
//   ids of the token are reported by every couple of that token.
struct PlainEntries {
    const int32_t* idx;
    __device__ __forceinline__ int load(int64_t p, int E, bool& bad) const
    {
        const int e = idx[p];
        bad |= e >= E;
        return e;
    }
};

struct DedupEntries {
    const int32_t* idx;
    uint32_t* kmask;   // null: masks not wanted by this pass
    int K, E, L, P;    // the real routing: top-k, experts, experts per partition, partitions
    __device__ __forceinline__ int load(int64_t j, int, bool& bad) const
    {
        const int t = (int)j / P;              // T*P < 2^31 (checked by the caller)
        const int p = (int)j - t * P;
        const int lo = p * L, hi = lo + L;
        int e[kMaxTopK];
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) e[k] = (k < K) ? idx[(int64_t)t * K + k] : -1;
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            bad |= e[k] >= E;
            if (e[k] >= lo && e[k] < hi) m |= 1u << k;
        }
        if (kmask) kmask[j] = m;
        return m ? p : -1;
    }
};

__device__ __forceinline__ int id_bits(int E)
{
    // bits needed to tell apart ids 0..E-1
    return E <= 1 ? 0 : 32 - __builtin_clz((unsigned)(E - 1));
}

// Lanes of this wave whose valid expert id equals this lane's (0 if invalid).
// Must be called by all 64 lanes (ballots).
__device__ __forceinline__ uint64_t match_peers(int e, bool valid, int nbits)
{
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return valid ? peers : 0ull;
}

__device__ __forceinline__ void zero_smem(LayoutSmem& s, int E)
{
    const int tid = threadIdx.x;
    if (tid < E) {
        s.hist[tid] = 0;
        s.cursor[tid] = 0;
        for (int w = 0; w < kLayoutWaves; ++w) s.wtab[w][tid] = 0;
    }
    if (tid == 0) s.bad = 0u;
}

// Histogram contribution of one round: the lowest lane of each peer group adds
// the group's size (order-free integer sums).  Returns the peers for reuse by
// rank_round.  All threads call it.
__device__ __forceinline__ uint64_t hist_round(int e, int E, int nbits, int32_t* hist)
{
    const bool valid = (e >= 0) && (e < E);
    const uint64_t peers = match_peers(e, valid, nbits);
    if (valid && lanes_below(peers) == 0) atomicAdd(&hist[e], (int)__popcll(peers));
    return peers;
}

// Rank one round: entry p (this thread's, `real` when p < n) with expert id e
// and its in-wave peers.  On entry s.cursor[e] is the first free row of
// expert e; unless `last`, it has moved past this round's entries on exit.
// Writes row_of_pair for every real entry (-1 when masked) and src_pair for
// valid ones when src_pair is non-null (rows are below n_rows = T*K).
__device__ __forceinline__ void rank_round(int e, int64_t p, bool real, uint64_t peers,
                                           int64_t n_rows, int E, bool last, LayoutSmem& s,
                                           int32_t* __restrict__ row_of_pair,
                                           int32_t* __restrict__ src_pair)
{
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const bool valid = real && (e >= 0) && (e < E);
    const int rank = lanes_below(peers);
    if (valid && rank == 0) s.wtab[w][e] = (uint16_t)__popcll(peers);
    lds_barrier();

    int run = 0;
    if (tid < E) {
        for (int v = 0; v < kLayoutWaves; ++v) {
            const int c = s.wtab[v][tid];
            s.wtab[v][tid] = (uint16_t)run;
            run += c;
        }
    }
    lds_barrier();

    if (real) {
        int row = -1;
        if (valid) {
            row = s.cursor[e] + (int)s.wtab[w][e] + rank;
            if (src_pair && row < n_rows) src_pair[row] = (int32_t)p;
        }
        row_of_pair[p] = row;
    }
    if (last) return;
    lds_barrier();

    if (tid < E) {
        s.cursor[tid] += run;
        for (int v = 0; v < kLayoutWaves; ++v) s.wtab[v][tid] = 0;
    }
    lds_barrier();
}

// Exclusive scan of one value per thread over the whole workgroup; *total
// receives the sum.  Contains barriers: all threads must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, LayoutSmem& s, int* total)
{
    const int tid = threadIdx.x;
    const int lane = tid % kWave, w = tid / kWave;
    const int x = wave_inclusive_scan(v);
    if (lane == kWave - 1) s.wsum[w] = x;
    lds_barrier();
    if (w == 0) {
        const int t = wave_inclusive_scan(lane < kLayoutWaves ? s.wsum[lane] : 0);
        if (lane < kLayoutWaves) s.wsum[lane] = t;   // inclusive prefix of wave sums
    }
    lds_barrier();
    const int before = (w > 0) ? s.wsum[w - 1] : 0;
    *total = s.wsum[kLayoutWaves - 1];
    lds_barrier();
    return before + x - v;
}

// From per-expert counts (one per thread, tid < E): write expert_count,
// expert_offset, part_count, part_offset (skipped when part_count is null)
// and status; leave the exclusive offsets in s.cursor and N in s.total.
__device__ __forceinline__ void finish_counts(int count, int E, int P, uint32_t bad, LayoutSmem& s, bool write_out,
                              int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
                              int32_t* __restrict__ part_count, int32_t* __restrict__ part_offset,
                              uint32_t* __restrict__ status)
{
    const int tid = threadIdx.x;
    int N = 0;
    const int off = block_exclusive_scan(tid < E ? count : 0, s, &N);
    if (tid < E) s.cursor[tid] = off;
    if (tid == 0) s.total = N;
    if (write_out) {
        if (tid < E) {
            expert_count[tid] = count;
            expert_offset[tid] = off;
        }
        if (tid == 0) {
            expert_offset[E] = N;
            *status = bad ? 1u : 0u;
        }
    }
    lds_barrier();
    const int L = E / P;
    if (write_out && part_count && tid < P) {
        const int lo = s.cursor[tid * L];
        const int hi = (tid + 1 < P) ? s.cursor[(tid + 1) * L] : N;
        part_offset[tid] = lo;
        part_count[tid] = hi - lo;
    }
    if (write_out && part_count && tid == 0) part_offset[P] = N;
}

// ---------------------------------------------------------------------------
// Small batches of dedup couples (T*P <= kSmallMaxPairs): one workgroup does
// everything (plain entries take the counting kernel below).
template <class Entries>
__global__ __launch_bounds__(kLayoutThreads) void layout_single_kernel(
    const Entries src, int64_t n, int E, int P,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ part_count, int32_t* __restrict__ part_offset,
    int32_t* __restrict__ row_of_pair, int32_t* __restrict__ src_pair,
    uint32_t* __restrict__ status)
{
    __shared__ LayoutSmem s;
    const int tid = threadIdx.x;
    const int nbits = id_bits(E);
    const int rounds = (int)((n + kLayoutThreads - 1) / kLayoutThreads);
    int ids[kSmallRounds];
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kSmallRounds; ++r) {
        const int64_t p = (int64_t)r * kLayoutThreads + tid;
        ids[r] = (p < n) ? src.load(p, E, bad) : -1;
    }
    zero_smem(s, E);
    lds_barrier();

    // pass 1: histogram
    uint64_t peers[kSmallRounds];
#pragma unroll
    for (int r = 0; r < kSmallRounds; ++r) {
        peers[r] = 0ull;
        if (r < rounds) peers[r] = hist_round(ids[r], E, nbits, s.hist);
    }
    if (bad) s.bad = 1u;
    lds_barrier();

    finish_counts(tid < E ? s.hist[tid] : 0, E, P, s.bad, s, true, expert_count, expert_offset,
                  part_count, part_offset, status);
    lds_barrier();

    // pass 2: deterministic slots
#pragma unroll
    for (int r = 0; r < kSmallRounds; ++r) {
        if (r < rounds) {
            const int64_t p = (int64_t)r * kLayoutThreads + tid;
            rank_round(ids[r], p, p < n, peers[r], n, E, r == rounds - 1, s, row_of_pair, src_pair);
        }
    }

    for (int64_t r = (int64_t)s.total + tid; r < n; r += kLayoutThreads) src_pair[r] = -1;
}

// ---------------------------------------------------------------------------
// Medium batches of plain entries (kTinyLayoutPairs < n <= kSmallMaxPairs):
// the slot of entry (e, p) is the number of valid entries before it in
// (expert, entry) order -- keys e*2^12 + p below its own -- counted with
// ballots, so the ranking spreads over many workgroups instead of one.
// Launch block 0 builds the histogram (match-any groups into LDS) and writes
// the counts, offsets, partition sums, status and the src_pair tail; every
// other workgroup ranks kCountLayoutOwn consecutive entries: each of its 16
// waves holds kIds rounds of the ids (one id per lane and round) and counts,
// for each own entry, the keys below it with one ballot and popcount per
// round; one barrier later wave 0 sums the waves' counts and writes the rows.
// Outputs equal those of the single-workgroup kernel.
constexpr int kCountLayoutOwn = 8;

template <int kIds>
__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(
    const int32_t* __restrict__ idx, int n, int E, int P,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ part_count, int32_t* __restrict__ part_offset,
    int32_t* __restrict__ row_of_pair, int32_t* __restrict__ src_pair,
    uint32_t* __restrict__ status)
{
    static_assert(kIds * kLayoutThreads <= kSmallMaxPairs, "keys hold entries below 2^12");
    __shared__ LayoutSmem s;
    __shared__ int32_t part[kCountLayoutOwn][kLayoutWaves];   // own entry q: keys below, per wave
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int w = wave_uniform(tid / kWave);
    int id[kIds];                                              // addresses clamped, masked below
#pragma unroll
    for (int j = 0; j < kIds; ++j) {
        const int p = j * kLayoutThreads + tid;
        id[j] = idx[p < n ? p : n - 1];
    }
#pragma unroll
    for (int j = 0; j < kIds; ++j)
        if (j * kLayoutThreads + tid >= n) id[j] = -1;

    if (blockIdx.x == 0) {
        zero_smem(s, E);
        lds_barrier();
        bool bad = false;
#pragma unroll
        for (int j = 0; j < kIds; ++j) {
            (void)hist_round(id[j], E, id_bits(E), s.hist);
            bad |= id[j] >= E;
        }
        if (bad) s.bad = 1u;
        lds_barrier();
        finish_counts(tid < E ? s.hist[tid] : 0, E, P, s.bad, s, true, expert_count,
                      expert_offset, part_count, part_offset, status);
        lds_barrier();
        for (int r = s.total + tid; r < n; r += kLayoutThreads) src_pair[r] = -1;
        return;
    }

    const int p0 = (int)(blockIdx.x - 1) * kCountLayoutOwn;
    const int nq = n - p0 < kCountLayoutOwn ? n - p0 : kCountLayoutOwn;
    const int me = idx[p0 + (lane < nq ? lane : 0)];
    uint32_t key[kIds];
#pragma unroll
    for (int j = 0; j < kIds; ++j)
        key[j] = (id[j] >= 0 && id[j] < E)
                     ? (((uint32_t)id[j] << 12) | (uint32_t)(j * kLayoutThreads + tid))
                     : 0xFFFFFFFFu;
    const bool mvalid = lane < nq && me >= 0 && me < E;
    const uint32_t mkey = mvalid ? (((uint32_t)me << 12) | (uint32_t)(p0 + lane)) : 0u;
    int below = 0;
#pragma unroll
    for (int q = 0; q < kCountLayoutOwn; ++q) {   // lanes past nq hold key 0: nothing below it
        const uint32_t qk = (uint32_t)read_lane((int)mkey, q);
        int c = 0;
#pragma unroll
        for (int j = 0; j < kIds; ++j) c += __builtin_popcountll(__ballot(key[j] < qk));
        if (lane == q) below = c;
    }
    if (lane < kCountLayoutOwn) part[lane][w] = below;
    lds_barrier();
    if (w == 0 && lane < nq) {
        int row = 0;
#pragma unroll
        for (int u = 0; u < kLayoutWaves; ++u) row += part[lane][u];
        if (!mvalid) row = -1;
        row_of_pair[p0 + lane] = row;
        if (row >= 0) src_pair[row] = p0 + lane;
    }
}

// ---------------------------------------------------------------------------
// Tiny batches (n <= kTinyLayoutPairs = 128 entries): one wave does it all.
// A wave's LDS operations complete in program order, so the single-workgroup
// kernel's barriers are not needed (wave_lds_sync orders each hand-off
// between lanes): match-any groups add their sizes to the
// LDS histogram, a DPP wave scan over the experts (kMaxExperts / 64 per lane)
// turns it into offsets that stay in LDS as per-expert cursors, and each
// round's rows are cursor + in-wave rank, the group leaders then moving the
// cursor past their group.
constexpr int kTinyLayoutPairs = 2 * kWave;

template <class Entries>
__global__ __launch_bounds__(kWave) void layout_tiny_kernel(
    const Entries src, int n, int E, int P,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ part_count, int32_t* __restrict__ part_offset,
    int32_t* __restrict__ row_of_pair, int32_t* __restrict__ src_pair,
    uint32_t* __restrict__ status)
{
    constexpr int kPerLane = kMaxExperts / kWave;
    __shared__ int32_t cur[kMaxExperts];
    const int lane = threadIdx.x;
    const int nbits = id_bits(E);
    bool bad = false;
    const int e0 = lane < n ? src.load(lane, E, bad) : -1;
    const int e1 = kWave + lane < n ? src.load(kWave + lane, E, bad) : -1;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int e = lane * kPerLane + j;
        if (e < E) cur[e] = 0;
    }
    const bool v0 = e0 >= 0 && e0 < E;
    const bool v1 = e1 >= 0 && e1 < E;
    const uint64_t peers0 = match_peers(e0, v0, nbits);
    const uint64_t peers1 = (n > kWave) ? match_peers(e1, v1, nbits) : 0ull;
    const int rank0 = lanes_below(peers0), rank1 = lanes_below(peers1);
    wave_lds_sync();                              // counters cleared
    if (v0 && rank0 == 0) atomicAdd(&cur[e0], (int)__popcll(peers0));
    if (v1 && rank1 == 0) atomicAdd(&cur[e1], (int)__popcll(peers1));
    wave_lds_sync();                              // histogram complete

    int c[kPerLane], sum = 0;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int e = lane * kPerLane + j;
        c[j] = (e < E) ? cur[e] : 0;
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
            cur[e] = o;                          // per-expert cursor: first free row
        }
        o += c[j];
    }
    wave_lds_sync();                              // offsets written
    if (part_count) {
        const int L = E / P;
        for (int p = lane; p < P; p += kWave) {
            const int lo = cur[p * L];
            const int hi = (p + 1 < P) ? cur[(p + 1) * L] : N;
            part_offset[p] = lo;
            part_count[p] = hi - lo;
        }
    }
    const bool anybad = __ballot(bad) != 0ull;
    if (lane == 0) {
        expert_offset[E] = N;
        if (part_count) part_offset[P] = N;
        *status = anybad ? 1u : 0u;
    }

    // rows: round 0, then its group leaders move the cursors past their
    // groups (after every lane of the wave has read them), then round 1
    const int row0 = v0 ? cur[e0] + rank0 : -1;
    wave_lds_sync();                              // every lane has read its cursor
    if (v0 && rank0 == 0) cur[e0] = row0 + (int)__popcll(peers0);
    wave_lds_sync();                              // cursors moved past round 0
    const int row1 = v1 ? cur[e1] + rank1 : -1;
    if (lane < n) {
        row_of_pair[lane] = row0;
        if (v0 && src_pair) src_pair[row0] = lane;
    }
    if (kWave + lane < n) {
        row_of_pair[kWave + lane] = row1;
        if (v1 && src_pair) src_pair[row1] = kWave + lane;
    }
    if (src_pair)
        for (int r = N + lane; r < n; r += kWave) src_pair[r] = -1;
}

// ---------------------------------------------------------------------------
// Large batches, pass 1: one workgroup per chunk of kChunkPairs entries
// writes the chunk's histogram into ws_hist[chunk][E] and a bad-id flag into
// ws_bad[chunk] (ballot-aggregated LDS atomics: a hot expert costs one atomic
// per wave, not one per entry).
template <class Entries>
__global__ __launch_bounds__(kLayoutThreads) void layout_hist_kernel(
    const Entries src, int64_t n, int E, int32_t* __restrict__ ws_hist,
    uint32_t* __restrict__ ws_bad)
{
    __shared__ int32_t hist[kMaxExperts];
    __shared__ uint32_t bad;
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const int nbits = id_bits(E);
    const int64_t c0 = (int64_t)chunk * kChunkPairs;
    const int64_t c1 = (c0 + kChunkPairs < n) ? c0 + kChunkPairs : n;
    int ids[kChunkRounds];
    bool b = false;
#pragma unroll
    for (int r = 0; r < kChunkRounds; ++r) {
        const int64_t p = c0 + (int64_t)r * kLayoutThreads + tid;
        ids[r] = (p < c1) ? src.load(p, E, b) : -1;
    }
    if (tid < E) hist[tid] = 0;
    if (tid == 0) bad = 0u;
    lds_barrier();
#pragma unroll
    for (int r = 0; r < kChunkRounds; ++r) (void)hist_round(ids[r], E, nbits, hist);
    if (b) bad = 1u;
    lds_barrier();
    if (tid < E) ws_hist[(int64_t)chunk * E + tid] = hist[tid];
    if (tid == 0) ws_bad[chunk] = bad;
}

// Large batches with many chunks, pass 2: one workgroup turns the chunk
// histograms into totals, the scans and partition sums, and each chunk's base
// row per expert (offset[e] + rows of expert e in earlier chunks), written
// back over ws_hist.
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(kLayoutThreads) void layout_scan_kernel(
    int nchunks, int E, int P, int32_t* __restrict__ ws_hist,
    const uint32_t* __restrict__ ws_bad,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ part_count, int32_t* __restrict__ part_offset,
    uint32_t* __restrict__ status)
{
    __shared__ LayoutSmem s;
    const int tid = threadIdx.x;
    if (tid == 0) s.bad = 0u;
    lds_barrier();
    uint32_t b = 0;
    for (int c = tid; c < nchunks; c += kLayoutThreads) b |= ws_bad[c];
    if (b) s.bad = 1u;

    // exclusive prefix over chunks, per expert (loads batched so they overlap)
    int run = 0;
    if (tid < E) {
        for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
            int h[kScanBatch];
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                h[j] = (c0 + j < nchunks) ? ws_hist[(int64_t)(c0 + j) * E + tid] : 0;
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) {
                if (c0 + j < nchunks) ws_hist[(int64_t)(c0 + j) * E + tid] = run;
                run += h[j];
            }
        }
    }
    lds_barrier();
    finish_counts(run, E, P, s.bad, s, true, expert_count, expert_offset, part_count, part_offset,
                  status);
    lds_barrier();
    if (tid < E) {
        const int off = s.cursor[tid];
        for (int c = 0; c < nchunks; ++c) ws_hist[(int64_t)c * E + tid] += off;
    }
}

// Large batches, last pass: one workgroup per chunk ranks its entries.
// With bases_ready == 0 (few chunks) every workgroup first derives, from all
// chunk histograms, the per-expert totals (-> scans; workgroup 0 also writes
// the count outputs) and the rows of each expert taken by earlier chunks --
// reading C*E integers from L2 is cheaper than another launch.  With
// bases_ready == 1 the scan kernel has already put the bases in ws_hist.
template <class Entries>
__global__ __launch_bounds__(kLayoutThreads) void layout_rank_kernel(
    const Entries src, int64_t n, int E, int P, int nchunks, int bases_ready,
    const int32_t* __restrict__ ws_hist, const uint32_t* __restrict__ ws_bad,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ part_count, int32_t* __restrict__ part_offset,
    int32_t* __restrict__ row_of_pair, int32_t* __restrict__ src_pair,
    uint32_t* __restrict__ status)
{
    __shared__ LayoutSmem s;
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const int nbits = id_bits(E);
    const int64_t c0 = (int64_t)chunk * kChunkPairs;
    const int64_t c1 = (c0 + kChunkPairs < n) ? c0 + kChunkPairs : n;
    int ids[kChunkRounds];
    bool unused_bad = false;   // bad ids were collected by the histogram pass
#pragma unroll
    for (int r = 0; r < kChunkRounds; ++r) {
        const int64_t p = c0 + (int64_t)r * kLayoutThreads + tid;
        ids[r] = (p < c1) ? src.load(p, E, unused_bad) : -1;
    }
    (void)unused_bad;
    zero_smem(s, E);
    lds_barrier();

    if (!bases_ready) {
        // groups of E threads split the chunks; partial sums meet in LDS
        const int groups = kLayoutThreads / E;
        const int g = tid / E, e = tid - g * E;
        if (g < groups) {
            // kScanBatch loads in flight per batch (addresses clamped, values
            // masked: no branch around a load, so one wait covers the batch)
            int tot = 0, bef = 0;
            for (int cb = g; cb < nchunks; cb += groups * kScanBatch) {
                int h[kScanBatch];
#pragma unroll
                for (int j = 0; j < kScanBatch; ++j) {
                    const int c = cb + j * groups;
                    h[j] = ws_hist[(int64_t)(c < nchunks ? c : nchunks - 1) * E + e];
                }
#pragma unroll
                for (int j = 0; j < kScanBatch; ++j) {
                    const int c = cb + j * groups;
                    const int v = c < nchunks ? h[j] : 0;
                    tot += v;
                    bef += c < chunk ? v : 0;
                }
            }
            atomicAdd(&s.hist[e], tot);
            atomicAdd(&s.cursor[e], bef);
        }
        uint32_t b = 0;
        for (int c = tid; c < nchunks; c += kLayoutThreads) b |= ws_bad[c];
        if (b) s.bad = 1u;
        lds_barrier();
        const int before = (tid < E) ? s.cursor[tid] : 0;
        lds_barrier();
        finish_counts(tid < E ? s.hist[tid] : 0, E, P, s.bad, s, chunk == 0, expert_count,
                      expert_offset, part_count, part_offset, status);
        lds_barrier();                     // partition sums above read s.cursor
        if (tid < E) s.cursor[tid] += before;
    } else {
        if (tid < E) s.cursor[tid] = ws_hist[(int64_t)chunk * E + tid];
        if (tid == 0) s.total = expert_offset[E];
    }
    lds_barrier();

    const int rounds = (int)((c1 - c0 + kLayoutThreads - 1) / kLayoutThreads);
#pragma unroll
    for (int r = 0; r < kChunkRounds; ++r) {
        if (r < rounds) {
            const int64_t p = c0 + (int64_t)r * kLayoutThreads + tid;
            const bool valid = ids[r] >= 0 && ids[r] < E;
            const uint64_t peers = match_peers(ids[r], valid, nbits);
            rank_round(ids[r], p, p < c1, peers, n, E, r == rounds - 1, s, row_of_pair,
                       src_pair);
        }
    }

    const int64_t stride = (int64_t)gridDim.x * kLayoutThreads;
    for (int64_t r = (int64_t)s.total + (int64_t)chunk * kLayoutThreads + tid; r < n; r += stride)
        src_pair[r] = -1;
}

// ---------------------------------------------------------------------------
// Workgroup size of the dedup counting kernel: 8 waves, every id loaded in two
// (four) rounds, measured faster than 16 waves in one (two) and than 4 waves
// (graphs of 50 launches on MI355X, top-8, hidden 7168: 128 tokens with 16
// partitions 3.24 -> 3.14 us, with E = 32, P = 8 3.10 -> 2.98 us; 4 to 256
// tokens 1-3 % faster; 4 waves 4-16 % slower): its two barriers wait on half as
// many waves.
constexpr int kDedupCountThreads = 512;

// ---------------------------------------------------------------------------
// Dedup layout by counting, for T*K <= kSmallMaxPairs entries with K and P
// powers of two.  Couple (t, p) is present when token t has a valid expert in
// partition p; its row is the partition's offset plus the number of earlier
// tokens present in p.  Every workgroup loads all T*K ids (coalesced, one per
// thread and round); a token's K entries are K aligned lanes of one wave, so
// an entry knows from a DPP prefix OR over its group whether a lower entry of
// its token is in the same partition, and the entry that is first counts the
// token for that partition, in LDS: in all, and before the workgroup's
// tokens (e / L by an exact multiply-shift, as in the fused kernels).  One
// barrier later wave 0 takes the workgroup's couples, one per lane in couple
// order -- 64 / P tokens, lane u*P + p for couple (t_lo + u, p) -- derives
// each couple's top-k mask from its token's ids, ranks it among the
// workgroup's earlier tokens with one ballot and writes tp_row, kmask and
// tp_src with consecutive lanes on consecutive couples.  Launch block 0
// writes the per-partition totals and offsets, status and the tp_src tail.
// Spreading the work this way keeps every global access coalesced and each
// workgroup's share small: one workgroup doing all of it (a thread per
// token, its P couples' writes strided by P) took 6-8 us at 128 x top-8 / 16
// partitions on one CU's memory pipeline.
template <int kIds, int kMaxK>
__global__ __launch_bounds__(kDedupCountThreads) void dedup_layout_count_kernel(
    const int32_t* __restrict__ idx, int T, int K, int E, int P, int32_t* __restrict__ tp_row,
    int32_t* __restrict__ part_tokens, int32_t* __restrict__ part_token_offset,
    int32_t* __restrict__ tp_src, uint32_t* __restrict__ kmask, uint32_t* __restrict__ status)
{
    static_assert(kIds * kDedupCountThreads <= kSmallMaxPairs, "the launcher's bound");
    __shared__ int32_t cnt[2][kMaxTopK];        // tokens present per partition: all, before t_lo
    __shared__ uint32_t sbad;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int n = T * K;
    const int kshift = __builtin_ctz((unsigned)K);          // K is a power of two
    const int tpw = kWave / P;                              // tokens per workgroup (P a power of two)
    const int t_lo = blockIdx.x == 0 ? T : (int)(blockIdx.x - 1) * tpw;
    // e / L for e < 1024 and L <= 1024: (e * magic) >> 20 with magic =
    // floor(2^20 / L) + 1, exact since e * (L - 2^20 mod L) < 2^20
    const uint32_t magic = (1u << 20) / (uint32_t)(E / P) + 1u;

    int id[kIds];                                           // loads first, addresses clamped
#pragma unroll
    for (int j = 0; j < kIds; ++j) {
        const int p = j * kDedupCountThreads + tid;
        id[j] = idx[p < n ? p : n - 1];
    }
    // wave 0 of a couple workgroup: couple (t_lo + u, pc) on lane u * P + pc;
    // its token's ids loaded now, with the others (uniform branch)
    const int u = lane / P;                                 // P a power of two: a shift
    const int pc = lane - u * P;
    const int t = t_lo + u;
    const bool own = t < T;                                 // lanes of tokens past T: nothing
    int ids[kMaxK];
    if (blockIdx.x != 0 && tid < kWave) {
        const int64_t row = (int64_t)(own ? t : T - 1) * K;
#pragma unroll
        for (int k = 0; k < kMaxK; ++k) ids[k] = idx[row + (k < K ? k : K - 1)];
    }
    if (tid < 2 * kMaxTopK) cnt[tid / kMaxTopK][tid % kMaxTopK] = 0;
    if (tid == 0) sbad = 0u;
    lds_barrier();                                          // (1) counters cleared
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kIds; ++j) {
        const int p = j * kDedupCountThreads + tid;
        const int e = p < n ? id[j] : -1;
        bad |= e >= E;
        const bool valid = e >= 0 && e < E;
        const uint32_t pp = valid ? ((uint32_t)e * magic) >> 20 : 0u;
        const uint32_t bit = valid ? 1u << pp : 0u;
        const uint32_t lower = group_excl_or(bit, K, lane);   // every lane: DPP sources
        if (valid && !(lower & bit)) {                      // the token's first entry in pp
            atomicAdd(&cnt[0][pp], 1);
            if ((p >> kshift) < t_lo) atomicAdd(&cnt[1][pp], 1);
        }
    }
    if (__ballot(bad) != 0ull && lane == 0) sbad = 1u;
    lds_barrier();                                          // (2) counts complete

    const int tot = lane < P ? cnt[0][lane] : 0;
    const int incl = wave_inclusive_scan(tot);              // partition offsets
    const int M = read_lane(incl, P - 1);
    if (blockIdx.x == 0) {
        if (tid < P) {
            part_tokens[tid] = tot;
            part_token_offset[tid] = incl - tot;
        }
        if (tid == 0) {
            part_token_offset[P] = M;
            *status = sbad ? 1u : 0u;
        }
        for (int r = M + tid; r < T * P; r += kDedupCountThreads) tp_src[r] = -1;
        return;
    }
    if (tid >= kWave) return;                               // wave 0 takes the couples
    uint32_t m = 0u;                                        // top-k mask of the couple
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
        const bool valid = k < K && ids[k] >= 0 && ids[k] < E;
        const uint32_t pp = valid ? ((uint32_t)ids[k] * magic) >> 20 : 32u;
        m |= (pp == (uint32_t)pc ? 1u : 0u) << k;
    }
    if (!own) m = 0u;
    // earlier tokens of this workgroup present in pc: the lanes u' * P + pc, u' < u
    const uint64_t same = (~0ull / ((1ull << P) - 1ull)) << pc;
    const uint64_t b = __ballot(m != 0u) & same & ((1ull << lane) - 1ull);
    const int before = __shfl(incl - tot, pc) + cnt[1][pc] + __builtin_popcountll(b);
    if (own) {
        const int j = t * P + pc;
        const int r = m ? before : -1;
        tp_row[j] = r;
        kmask[j] = m;
        if (r >= 0) tp_src[r] = j;
    }
}

int64_t num_chunks(int64_t n) { return (n + kChunkPairs - 1) / kChunkPairs; }

}  // namespace

size_t layout_workspace_bytes(int T, int K, int E)
{
    const int64_t n = (int64_t)T * K;
    if (n <= kSmallMaxPairs) return 0;
    const int64_t c = num_chunks(n);
    const size_t hist = (size_t)c * E * sizeof(int32_t);
    const size_t hist_padded = (hist + 255) & ~(size_t)255;
    return hist_padded + (size_t)c * sizeof(uint32_t);
}

namespace {

// n entries with ids in 0..E-1 (E <= kMaxExperts) and P partitions; the
// workspace sizing of layout_workspace_bytes for the same n and E.
template <class Entries>
hipError_t launch_layout_entries(const Entries& src, int64_t n, int E, int P,
                                 int32_t* expert_count, int32_t* expert_offset,
                                 int32_t* part_count, int32_t* part_offset,
                                 int32_t* row_of_pair, int32_t* src_pair, uint32_t* status,
                                 void* ws, hipStream_t stream)
{
    if (n <= kTinyLayoutPairs) {
        hipLaunchKernelGGL(layout_tiny_kernel<Entries>, dim3(1), dim3(kWave), 0, stream, src,
                           (int)n, E, P, expert_count, expert_offset, part_count, part_offset,
                           row_of_pair, src_pair, status);
        return hipGetLastError();
    }
    if constexpr (std::is_same_v<Entries, PlainEntries>) {
        // here n > kTinyLayoutPairs: the counting kernel clamps its id
        // addresses to n - 1 and must never see the empty batch, whose
        // topk_idx may be null
        if (n <= kSmallMaxPairs) {
            const unsigned blocks = (unsigned)((n + kCountLayoutOwn - 1) / kCountLayoutOwn) + 1;
            hipLaunchKernelGGL(n <= kLayoutThreads ? layout_count_kernel<1> : layout_count_kernel<2>,
                               dim3(blocks), dim3(kLayoutThreads), 0, stream, src.idx, (int)n, E,
                               P, expert_count, expert_offset, part_count, part_offset,
                               row_of_pair, src_pair, status);
            return hipGetLastError();
        }
    } else {
        if (n <= kSmallMaxPairs) {
            hipLaunchKernelGGL(layout_single_kernel<Entries>, dim3(1), dim3(kLayoutThreads), 0,
                               stream, src, n, E, P, expert_count, expert_offset, part_count,
                               part_offset, row_of_pair, src_pair, status);
            return hipGetLastError();
        }
    }
    const int64_t c = num_chunks(n);
    const size_t hist = (size_t)c * E * sizeof(int32_t);
    int32_t* ws_hist = (int32_t*)ws;
    uint32_t* ws_bad = (uint32_t*)((char*)ws + ((hist + 255) & ~(size_t)255));
    Entries hist_src = src;
    if constexpr (std::is_same_v<Entries, DedupEntries>) hist_src.kmask = nullptr;
    hipLaunchKernelGGL(layout_hist_kernel<Entries>, dim3((unsigned)c), dim3(kLayoutThreads), 0,
                       stream, hist_src, n, E, ws_hist, ws_bad);
    const int bases_ready = c > kMaxChunksTwoPass ? 1 : 0;
    if (bases_ready)
        hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kLayoutThreads), 0, stream,
                           (int)c, E, P, ws_hist, ws_bad, expert_count, expert_offset, part_count,
                           part_offset, status);
    hipLaunchKernelGGL(layout_rank_kernel<Entries>, dim3((unsigned)c), dim3(kLayoutThreads), 0,
                       stream, src, n, E, P, (int)c, bases_ready, ws_hist, ws_bad, expert_count,
                       expert_offset, part_count, part_offset, row_of_pair, src_pair, status);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_layout(const int32_t* idx, int T, int K, int E, int P,
                         int32_t* expert_count, int32_t* expert_offset,
                         int32_t* part_count, int32_t* part_offset,
                         int32_t* row_of_pair, int32_t* src_pair, uint32_t* status,
                         void* ws, hipStream_t stream)
{
    return launch_layout_entries(PlainEntries{idx}, (int64_t)T * K, E, P, expert_count,
                                 expert_offset, part_count, part_offset, row_of_pair, src_pair,
                                 status, ws, stream);
}

size_t dedup_layout_workspace_bytes(int T, int P) { return layout_workspace_bytes(T, P, P); }

hipError_t launch_dedup_layout(const int32_t* idx, int T, int K, int E, int P, int32_t* tp_row,
                               int32_t* part_tokens, int32_t* part_token_offset, int32_t* tp_src,
                               uint32_t* kmask, uint32_t* status, void* ws, hipStream_t stream)
{
    const bool pow2 = (K & (K - 1)) == 0 && (P & (P - 1)) == 0;
    if (T >= 1 && pow2 && (int64_t)T * K <= kSmallMaxPairs) {
        const unsigned blocks = (unsigned)((T + kWave / P - 1) / (kWave / P)) + 1;
        // ids per thread: 2 up to 1024 entries, 4 up to kSmallMaxPairs
        constexpr int kR = kSmallMaxPairs / kDedupCountThreads;
        const bool half = (int64_t)T * K <= kSmallMaxPairs / 2;
        hipLaunchKernelGGL(K <= 8 ? (half ? dedup_layout_count_kernel<kR / 2, 8> : dedup_layout_count_kernel<kR, 8>)
                                  : (half ? dedup_layout_count_kernel<kR / 2, 16> : dedup_layout_count_kernel<kR, 16>),
                           dim3(blocks), dim3(kDedupCountThreads), 0, stream, idx, T, K, E, P, tp_row,
                           part_tokens, part_token_offset, tp_src, kmask, status);
        return hipGetLastError();
    }
    // ids 0..P-1 with one partition per id: the per-"expert" counts and scan
    // are the per-partition token counts and offsets.
    const DedupEntries src{idx, kmask, K, E, E / P, P};
    return launch_layout_entries(src, (int64_t)T * P, P, P, part_tokens, part_token_offset,
                                 nullptr, nullptr, tp_row, tp_src, status, ws, stream);
}

}  // namespace ep
