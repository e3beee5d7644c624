/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel low-latency
 * layout / dispatch / combine library (libep_mi355x.so).
 *
 * One GPU's share of the expert-parallel traffic: the P destination "ranks"
 * of an EP group are P contiguous partitions of the receive buffers in this
 * GPU's HBM.  The method:
 *   - layout: count tokens per expert and per destination before any
 *     payload moves, then give every (token, k) entry a slot.  The sources
 *     show the cost of learning a destination's batch size by waiting on
 *     per-expert completion counters (UCCL PR #749 "[EP] Low-latency mode
 *     batch tokens per destination", review comment); here the counts come
 *     from a histogram and an exclusive scan, and slots are deterministic;
 *   - dispatch: each token's hidden vector, quantised to fp8 with one scale
 *     per 128 columns, is written to the receive row of each of its top-k
 *     experts (DeepEP PR #693 "Pipeline direct NVLink dispatch with
 *     triple-buffered prefetch", Summary: a token carries hidden data, scale
 *     factors and routing); a bf16 passthrough mode copies the row as is;
 *   - combine: each token gathers its top-k expert outputs, reads straight
 *     from the caller's buffer (MoRI PR #614 "perf(ep): InterNodeV1LL
 *     low-token latency on MI300X + CX7", zero-copy combine paragraph), and
 *     reduces them in fp32 with the top-k weights, written out as bf16.
 *
 * Conventions (all entry points):
 *   - Device pointers unless stated.  The caller owns every buffer; the
 *     library allocates nothing, keeps no pointer after a call returns and
 *     holds no global state, so calls on different streams are independent
 *     (the one exception, ep_layout_dispatch_noalloc, holds a scratch buffer
 *     per device).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work; none synchronises the host.  Buffers must stay
 *     alive until the stream has run the work.
 *   - Return 0 on success.  EP_EINVAL (bad argument), EP_ENOTSUP
 *     (unsupported payload) and EP_ESCRATCH (ep_layout_dispatch_noalloc
 *     only: the batch needs more scratch than the library holds) mean a
 *     host-side check failed and NOTHING was enqueued: every check, those of
 *     the kernel launches included, runs before the first launch.  EP_EHIP
 *     means HIP refused a launch (see ep_last_hip_error()); the launches of
 *     the same call before it may have been enqueued.
 *   - Every call can be captured into a HIP graph: no call allocates,
 *     memsets or synchronises; counters the kernels need are cleared by
 *     the kernels themselves.
 *
 * Notation: T tokens, H hidden size, K top-k (1..16), E experts (1..1024),
 * P partitions (E % P == 0), L = E / P experts per partition, expert e
 * belongs to partition e / L (UCCL PR #749 review excerpt: a rank owns a
 * contiguous block of experts).  A "pair" is a (t, k) entry, flat index
 * t*K + k.  N = number of valid pairs (0 <= id < E).
 */
#ifndef EP_MI355X_H
#define EP_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_OK 0
#define EP_EINVAL (-1)
#define EP_ENOTSUP (-2)
#define EP_EHIP (-3)

#define EP_PAYLOAD_FP8_E4M3FN 0   /* OCP e4m3fn bytes + fp32 scale per 128 columns */
#define EP_PAYLOAD_BF16 1         /* bf16 passthrough, no scales */

#define EP_MAX_TOPK 16
#define EP_MAX_EXPERTS 1024

/* status word bit set by ep_layout when some id >= E was seen (that entry is
 * then treated as masked). */
#define EP_STATUS_BAD_EXPERT_ID 1u

/*
 * Size in bytes of the workspace ep_layout needs for T tokens, top-K, E
 * experts.  Host-only.  0 means no workspace is needed (small batches).
 * Returns 0 as well for arguments ep_layout would reject.
 */
size_t ep_layout_workspace_bytes(int T, int K, int E);

/*
 * Layout: per-expert and per-destination counts, their exclusive scans and
 * the slot of every pair.
 *
 *   topk_idx      int32 [T, K] row-major.  Negative = masked entry (the
 *                 sentinel of MoRI PR #614, routing-scan paragraph); an id
 *                 >= E sets EP_STATUS_BAD_EXPERT_ID in *status and is masked.
 *   expert_count  int32 [E]    out: pairs routed to each expert.
 *   expert_offset int32 [E+1]  out: exclusive scan, expert_offset[E] = N.
 *   part_count    int32 [P]    out: pairs per destination partition (the
 *                              batch size a sender needs, UCCL PR #749).
 *   part_offset   int32 [P+1]  out: part_offset[p] = expert_offset[p*L],
 *                              part_offset[P] = N.
 *   row_of_pair   int32 [T*K]  out: receive row of pair t*K+k, -1 if masked.
 *                              Rows of expert e are expert_offset[e] ..
 *                              expert_offset[e+1]-1 in ascending (t, k)
 *                              order, so the layout is deterministic and
 *                              partition p owns rows part_offset[p] ..
 *                              part_offset[p+1]-1.
 *   src_pair      int32 [T*K]  out: src_pair[row] = t*K+k for row < N, -1
 *                              for row in [N, T*K).
 *   status        uint32 [1]   out: cleared, then EP_STATUS_* bits.
 *   ws, ws_bytes  workspace of at least ep_layout_workspace_bytes(T,K,E)
 *                 bytes, 16-byte aligned (may be NULL when that is 0).
 *                 Contents need no initialisation and are scratch after the
 *                 call; one workspace must not be shared by calls that can
 *                 run concurrently.
 * Errors: EP_EINVAL for T < 0, K outside 1..16, E outside 1..1024, P < 1,
 * E % P != 0, T*K >= 2^31, NULL or misaligned (4 B; ws 16 B) pointers where
 * T > 0 needs them (expert_count, expert_offset, part_count, part_offset and
 * status are always needed), or ws_bytes too small.
 */
int ep_layout(const int32_t* topk_idx, int T, int K, int E, int P,
              int32_t* expert_count, int32_t* expert_offset,
              int32_t* part_count, int32_t* part_offset,
              int32_t* row_of_pair, int32_t* src_pair, uint32_t* status,
              void* ws, size_t ws_bytes, void* stream);

/*
 * Dispatch: scatter each token's hidden vector into the receive rows of its
 * valid pairs, fp8 with its per-128-column scales travelling with the row
 * (DeepEP PR #693 "Pipeline direct NVLink dispatch with triple-buffered
 * prefetch", Summary: a token's hidden data, scale factors and routing are
 * sent together; MoRI PR #614 "perf(ep): InterNodeV1LL low-token latency on
 * MI300X + CX7" dispatches fp8 and combines bf16), or bf16 as is.
 *
 *   x            bf16 bits [T, H], 16-byte aligned.
 *   row_of_pair  int32 [T*K] from ep_layout.
 *   payload      EP_PAYLOAD_FP8_E4M3FN: for every token and 128-column block,
 *                amax = max |x| (NaN ignored), scale = amax / 448 (IEEE fp32
 *                division), byte = e4m3fn(x / scale) (IEEE fp32 division,
 *                round to nearest even, saturating at +-448, NaN -> 0x7F|sign,
 *                sign kept on zero); amax = 0 gives scale 0 and zero bytes.
 *                recv_x is uint8 [T*K, H] and recv_scales fp32 [T*K, H/128],
 *                both row-major; H % 128 == 0.
 *                EP_PAYLOAD_BF16: the row is copied verbatim, recv_x is bf16
 *                [T*K, H], recv_scales is ignored (may be NULL); H % 8 == 0.
 *   Only rows named by row_of_pair are written; every other row (masked
 *   entries, rows >= N) is left untouched.
 * Errors: EP_EINVAL for T < 0, H <= 0, the H divisibility above, K outside
 * 1..16, T*K >= 2^31, NULL or misaligned pointers (x, recv_x 16 B;
 * row_of_pair, recv_scales 4 B) when T > 0; EP_ENOTSUP for another payload.
 */
int ep_dispatch(const uint16_t* x, int T, int H, int K,
                const int32_t* row_of_pair, int payload,
                void* recv_x, float* recv_scales, void* stream);

/*
 * Layout and dispatch in one call: the same results as ep_layout followed by
 * ep_dispatch (every output of both, bit for bit), with the same arguments
 * and errors as those two calls together.  For small batches (T*K <= 4096
 * and T * ceil(H/512) <= 2^20) it is ONE kernel launch: each dispatch
 * workgroup derives the layout values it needs from the T*K ids, so no
 * separate layout launch precedes it -- at a few tokens the step is paced by
 * launches, not by bytes (MoRI PR #614, view-cache paragraph).  Larger
 * batches run the layout and dispatch kernels back to back.
 */
int ep_layout_dispatch(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K, int E,
                       int P, int payload, int32_t* expert_count, int32_t* expert_offset,
                       int32_t* part_count, int32_t* part_offset, int32_t* row_of_pair,
                       int32_t* src_pair, uint32_t* status, void* ws, size_t ws_bytes,
                       void* recv_x, float* recv_scales, void* stream);

/*
 * ep_layout_dispatch without a workspace argument, for callers that cannot
 * allocate device memory (code recorded into a HIP graph, serving loops that
 * forbid allocation, harnesses without an allocator).  Same arguments,
 * results and errors as ep_layout_dispatch minus ws / ws_bytes: batches that
 * need a layout workspace (ep_layout_workspace_bytes(T, K, E) > 0) use a
 * buffer of EP_NOALLOC_SCRATCH_BYTES that the library holds on each device
 * from its first such call until the process ends.  The call allocates
 * nothing.
 *   - A batch whose workspace exceeds EP_NOALLOC_SCRATCH_BYTES is rejected
 *     with EP_ESCRATCH before anything else happens (for E = 1024 that is
 *     T*K above about 10^6 entries).
 *   - `stream` must belong to the current device (EP_EINVAL otherwise).
 *   - The first call on a device that needs the buffer looks up its address
 *     there (a host call, not stream work): make that first call outside
 *     stream capture.
 *   - Every call on one device shares that device's buffer, so calls that
 *     can overlap on one device (concurrent streams, other host threads)
 *     race; serialise them.  The buffer needs no initialisation and keeps
 *     the last call's scratch contents.
 */
#define EP_ESCRATCH (-4)
#define EP_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

int ep_layout_dispatch_noalloc(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K,
                               int E, int P, int payload, int32_t* expert_count,
                               int32_t* expert_offset, int32_t* part_count, int32_t* part_offset,
                               int32_t* row_of_pair, int32_t* src_pair, uint32_t* status,
                               void* recv_x, float* recv_scales, void* stream);

/*
 * Combine (MoRI PR #614 "perf(ep): InterNodeV1LL low-token latency on MI300X
 * + CX7": the expert outputs are gathered back to their tokens and reduced,
 * read in place from the receive rows -- zero-copy combine paragraph):
 * out[t, c] = bf16_rne(acc), acc = 0.0f, then for k = 0..K-1 with
 * r = row_of_pair[t*K+k] >= 0: acc = fmaf(topk_w[t*K+k], y[r, c], acc)
 * (fp32, fixed k order; masked entries are skipped, weights used as given).
 * A token with every entry masked gives +0.  bf16 rounding is to nearest
 * even; NaN stays NaN.
 *
 *   expert_out  bf16 bits y [T*K, H] in the receive-row layout of
 *               ep_dispatch (read in place, no staging copy), 16-B aligned;
 *               all T*K rows must be readable (for a masked entry the kernel
 *               reads row 0 instead and does not use it).
 *   topk_w      fp32 [T, K].   out  bf16 bits [T, H], 16-B aligned.
 * Errors: EP_EINVAL for T < 0, H <= 0 or H % 8 != 0, K outside 1..16,
 * T*K >= 2^31, NULL or misaligned pointers when T > 0.
 */
int ep_combine(const uint16_t* expert_out, const int32_t* row_of_pair,
               const float* topk_w, int T, int H, int K,
               uint16_t* out, void* stream);

/*
 * Per-destination (dedup) variant.  A token whose top-k experts share a
 * destination is sent there once, with a bit mask of the top-k entries that
 * copy serves, and the destination sums its share of the combine before
 * sending one partial row back (UCCL PR #749 "[EP] Low-latency mode batch
 * tokens per destination"; MoRI PR #614, DispatchIntraNode paragraph: the
 * flat work split leaves the dedup unchanged).  A "couple" is (t, p), flat
 * index t*P + p; it is present when token t has at least one valid expert
 * in partition p.  M = number of present couples.  P <= 16.
 *
 * The dedup dispatch is ep_dispatch with K = P and row_of_pair = tp_row:
 * each present couple's row gets one copy of the token (fp8 + scales, or
 * bf16), M rows in all instead of N.
 */
#define EP_MAX_DEDUP_PARTITIONS 16

/* Workspace bytes ep_dedup_layout needs (0: none).  Host-only; 0 as well for
 * arguments ep_dedup_layout would reject. */
size_t ep_dedup_layout_workspace_bytes(int T, int K, int E, int P);

/*
 * Dedup layout.
 *   topk_idx          int32 [T, K], as for ep_layout (negative = masked, id >= E
 *                     sets EP_STATUS_BAD_EXPERT_ID and is masked).
 *   tp_row            int32 [T*P] out: dedup row of couple t*P+p, -1 when absent.
 *                     Partition p owns rows part_token_offset[p] ..
 *                     part_token_offset[p+1]-1, in ascending token order.
 *   part_tokens       int32 [P]   out: present couples (distinct tokens) per partition.
 *   part_token_offset int32 [P+1] out: exclusive scan; part_token_offset[P] = M.
 *   tp_src            int32 [T*P] out: tp_src[row] = t*P+p for row < M, -1 for
 *                     rows M .. T*P-1.
 *   kmask             uint32 [T*P] out: bit k set when topk_idx[t, k] is a valid
 *                     expert of partition p (0 for absent couples).
 *   status            uint32 [1] out: cleared, then EP_STATUS_* bits.
 *   ws, ws_bytes      workspace of ep_dedup_layout_workspace_bytes(T, K, E, P)
 *                     bytes, 16-byte aligned; scratch, not shared by concurrent calls.
 * Errors: EP_EINVAL for the routing errors of ep_layout, P outside 1..16,
 * E % P != 0, T*P >= 2^31, NULL or misaligned (4 B; ws 16 B) pointers, or
 * ws_bytes too small.
 */
int ep_dedup_layout(const int32_t* topk_idx, int T, int K, int E, int P,
                    int32_t* tp_row, int32_t* part_tokens, int32_t* part_token_offset,
                    int32_t* tp_src, uint32_t* kmask, uint32_t* status,
                    void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes ep_dedup_layout_dispatch needs (0: none); host-only. */
size_t ep_dedup_layout_dispatch_workspace_bytes(int T, int K, int E, int P);

/*
 * The sender's whole dedup step in one call: the per-expert layout (every
 * output of ep_layout), the dedup layout (every output of ep_dedup_layout)
 * and the dedup dispatch (ep_dispatch with K = P over tp_row), bit for bit
 * the same as those three calls.  For T*K <= 4096 (and T * ceil(H/512) <=
 * 2^20) it is ONE kernel launch (each workgroup derives both layouts' values
 * for its own tokens from the T*K ids); larger batches run the three calls'
 * kernels back to back.
 *   recv_x / recv_scales are sized for T*P rows (only rows < M are written).
 *   ws: ep_dedup_layout_dispatch_workspace_bytes(T, K, E, P) bytes.
 * Errors: those of the three calls.
 */
int ep_dedup_layout_dispatch(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K, int E,
                             int P, int payload, int32_t* expert_count, int32_t* expert_offset,
                             int32_t* part_count, int32_t* part_offset, int32_t* row_of_pair,
                             int32_t* src_pair, int32_t* tp_row, int32_t* part_tokens,
                             int32_t* part_token_offset, int32_t* tp_src, uint32_t* kmask,
                             uint32_t* status, void* ws, size_t ws_bytes, void* recv_x,
                             float* recv_scales, void* stream);

/*
 * Combine level 1, at the destination: for every present couple (t, p),
 * partial[tp_row[t*P+p], c] = bf16_rne(acc), acc = 0.0f, then for k = 0..K-1
 * in order with bit k of kmask[t*P+p] set and r = row_of_pair[t*K+k] >= 0:
 * acc = fmaf(topk_w[t*K+k], expert_out[r, c], acc).  Rows of absent couples
 * are not written.
 *   expert_out  bf16 [T*K, H] in the receive-row layout of ep_layout (the
 *               per-expert rows the experts computed), 16-B aligned; all T*K
 *               rows must be readable (row 0 is read, unused, in place of
 *               entries without a row).
 *   row_of_pair int32 [T*K] from ep_layout; topk_w fp32 [T, K];
 *   tp_row, kmask from ep_dedup_layout;  partial bf16 [T*P, H], 16-B aligned.
 * Errors: EP_EINVAL for T < 0, K outside 1..16, P outside 1..16, T*K or
 * T*P >= 2^31, H <= 0 or H % 8 != 0, NULL or misaligned pointers when T > 0.
 */
int ep_combine_partial(const uint16_t* expert_out, const int32_t* row_of_pair,
                       const float* topk_w, const int32_t* tp_row, const uint32_t* kmask,
                       int T, int H, int K, int P, uint16_t* partial, void* stream);

/*
 * Combine level 2, at the token's home: out[t, c] = bf16_rne(acc), acc = 0.0f,
 * then for p = 0..P-1 in order with r = tp_row[t*P+p] >= 0:
 * acc = acc + partial[r, c] (fp32).  A token with no present couple gives +0.
 *   partial bf16 [T*P, H] from ep_combine_partial, all T*P rows readable
 *               (row 0 is read, unused, in place of absent couples);
 *   tp_row int32 [T*P]; out bf16 [T, H]; 16-B aligned rows.
 * Errors: EP_EINVAL for T < 0, P outside 1..16, T*P >= 2^31, H <= 0 or
 * H % 8 != 0, NULL or misaligned pointers when T > 0.
 */
int ep_combine_reduce(const uint16_t* partial, const int32_t* tp_row, int T, int H, int P,
                      uint16_t* out, void* stream);

/*
 * Launch geometry (for tuning).  ep_dispatch and ep_combine launch 4 waves
 * (256 threads) per workgroup and one wave per work item, a work item being
 * one token's 512-column slice.  These variants take the geometry
 * explicitly:
 *   waves_per_block  1, 2, 4 or 8;
 *   max_blocks       0 (one wave per item) or a cap on the number of
 *                    workgroups, whose waves then stride over the items;
 *   slice_cols       0 or 512 (512 columns per item) or 1024 (two
 *                    512-column halves of one token per wave, loaded
 *                    together).
 * The outputs do not depend on the geometry (bit for bit); only the time
 * does.  The sources found that the best geometry moves with token count and
 * phase, that items below 512 columns starve, and pick the geometry by
 * measurement (MoRI PR #614, tuner and MultiWarpIter paragraphs).
 * Errors: those of ep_dispatch / ep_combine, and EP_EINVAL for another
 * waves_per_block, a negative max_blocks or another slice_cols.
 */
#define EP_MAX_WAVES_PER_BLOCK 8

int ep_dispatch_geom(const uint16_t* x, int T, int H, int K, const int32_t* row_of_pair,
                     int payload, void* recv_x, float* recv_scales, int waves_per_block,
                     int max_blocks, int slice_cols, void* stream);

int ep_combine_geom(const uint16_t* expert_out, const int32_t* row_of_pair, const float* topk_w,
                    int T, int H, int K, uint16_t* out, int waves_per_block, int max_blocks,
                    int slice_cols, void* stream);

/*
 * Host-only: the geometry an ep_combine of T tokens x top-k K at hidden size
 * H runs with, written to plan[4]:
 *   plan[0]  waves per workgroup, plan[1] max_blocks, plan[2] columns per
 *            work item, as ep_combine_geom takes them;
 *   plan[3]  1 when the combine streams (the gathered rows T*K*H*2 bytes
 *            reach 64 MiB: nontemporal loads and stores), else 0.
 * With waves_per_block = 0 (then max_blocks and slice_cols 0 too) it is
 * ep_combine's own choice: 2 waves per workgroup when the combine streams,
 * 4 otherwise, uncapped, 512 columns (the geometry found fastest by
 * measurement, as the sources pick theirs: MoRI PR #614 "perf(ep):
 * InterNodeV1LL low-token latency on MI300X + CX7", tuner paragraphs);
 * otherwise the geometry given, as ep_combine_geom would launch it.
 * Returns EP_EINVAL (plan untouched) for arguments or a geometry
 * ep_combine / ep_combine_geom would reject.  Nothing touches the GPU.
 */
int ep_combine_plan(int T, int H, int K, int waves_per_block, int max_blocks, int slice_cols,
                    int32_t* plan);

/*
 * ep_layout_dispatch with an explicit launch geometry (0 = the library's
 * choice for each of the three values).  Same results, bit for bit, as
 * ep_layout_dispatch.
 *   - A batch that runs fused (T*K <= 4096, one launch) takes only a
 *     workgroup size: max_blocks must be 0 and slice_cols 0 or 512.  The
 *     workgroup sizes the fused kernels take depend on the batch:
 *       T*K <= 128 (EP_PLAN_FUSED_TINY): 1, 2, 4 or 8 waves (default 4);
 *       T*K <= 1024 (EP_PLAN_FUSED_COUNT): 4, 6, 7 or 8 waves when a
 *         workgroup's items then touch at most 16 entries (the default is
 *         the largest of 8, 7, 6 that divides the 512-column steps per
 *         token); 4 or 8 waves otherwise (EP_PLAN_FUSED_GENERAL);
 *       T*K <= 4096 (EP_PLAN_FUSED_GENERAL): 4 or 8 waves when a
 *         workgroup's items touch at most 64 entries.
 *   - A larger batch runs the layout kernels and then the dispatch kernel,
 *     which takes (waves_per_block, max_blocks, slice_cols) as
 *     ep_dispatch_geom does.
 * Errors: those of ep_layout_dispatch, and EP_EINVAL for a geometry the
 * batch's kernels do not take (nothing is enqueued).
 */
int ep_layout_dispatch_geom(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K, int E,
                            int P, int payload, int32_t* expert_count, int32_t* expert_offset,
                            int32_t* part_count, int32_t* part_offset, int32_t* row_of_pair,
                            int32_t* src_pair, uint32_t* status, void* ws, size_t ws_bytes,
                            void* recv_x, float* recv_scales, int waves_per_block, int max_blocks,
                            int slice_cols, void* stream);

/*
 * Host-only: how ep_layout_dispatch_geom would run a batch with the given
 * geometry (0s = ep_layout_dispatch's own choice), written to plan[4]:
 *   plan[0]  EP_PLAN_FUSED_TINY, EP_PLAN_FUSED_COUNT, EP_PLAN_FUSED_GENERAL
 *            (one fused launch) or EP_PLAN_LAYOUT_THEN_DISPATCH;
 *   plan[1]  waves per workgroup (of the fused kernel, or of the dispatch);
 *   plan[2]  fused: workgroups launched; otherwise the dispatch's max_blocks;
 *   plan[3]  columns per work item (512, or the dispatch's slice).
 * Returns EP_EINVAL (plan untouched) for arguments or a geometry
 * ep_layout_dispatch_geom would reject, EP_ENOTSUP for another payload.
 * Pointers are not involved; nothing touches the GPU.
 */
#define EP_PLAN_FUSED_TINY 0
#define EP_PLAN_FUSED_COUNT 1
#define EP_PLAN_FUSED_GENERAL 2
#define EP_PLAN_LAYOUT_THEN_DISPATCH 3

int ep_layout_dispatch_plan(int T, int H, int K, int E, int P, int payload, int waves_per_block,
                            int max_blocks, int slice_cols, int32_t* plan);

/*
 * ep_dedup_layout_dispatch with an explicit launch geometry (0 = the
 * library's choice for each value); same results, bit for bit.  Same
 * arguments as ep_dedup_layout_dispatch, then the geometry, then the stream.
 *   - A batch that runs fused (T*K <= 4096) takes only a workgroup size
 *     (max_blocks 0, slice_cols 0 or 512):
 *       K a power of two and T*K <= 1024 (EP_PLAN_FUSED_COUNT): 6, 7 or 8
 *         waves that divide the 512-column steps per token, so that every
 *         workgroup lies inside one token (default: the largest); when
 *         none does, or another size is asked for, the general kernel;
 *       otherwise (EP_PLAN_FUSED_GENERAL): 4 or 8 waves when a workgroup's
 *         items touch at most 64 entries.
 *   - A larger batch runs the two layouts and then the dispatch to the
 *     couple rows (P entries per token over tp_row), which takes
 *     (waves_per_block, max_blocks, slice_cols) as ep_dispatch_geom does.
 * Errors: those of ep_dedup_layout_dispatch, and EP_EINVAL for a geometry
 * the batch's kernels do not take (nothing is enqueued).
 */
int ep_dedup_layout_dispatch_geom(const int32_t* topk_idx, const uint16_t* x, int T, int H, int K,
                                  int E, int P, int payload, int32_t* expert_count,
                                  int32_t* expert_offset, int32_t* part_count,
                                  int32_t* part_offset, int32_t* row_of_pair, int32_t* src_pair,
                                  int32_t* tp_row, int32_t* part_tokens,
                                  int32_t* part_token_offset, int32_t* tp_src, uint32_t* kmask,
                                  uint32_t* status, void* ws, size_t ws_bytes, void* recv_x,
                                  float* recv_scales, int waves_per_block, int max_blocks,
                                  int slice_cols, void* stream);

/*
 * Host-only: how ep_dedup_layout_dispatch_geom would run a batch, written to
 * plan[4] as by ep_layout_dispatch_plan (plan[0] EP_PLAN_FUSED_COUNT,
 * EP_PLAN_FUSED_GENERAL or EP_PLAN_LAYOUT_THEN_DISPATCH).  EP_EINVAL (plan
 * untouched) for arguments or a geometry ep_dedup_layout_dispatch_geom would
 * reject, EP_ENOTSUP for another payload.  Nothing touches the GPU.
 */
int ep_dedup_layout_dispatch_plan(int T, int H, int K, int E, int P, int payload,
                                  int waves_per_block, int max_blocks, int slice_cols,
                                  int32_t* plan);

/*
 * HIP graph capture for the small-token regime, where host enqueue paces the
 * GPU (MoRI PR #614, view-cache paragraph: at 4 tokens most of a round's
 * wall time was host work, and stable buffers are what make the op
 * capturable).  Between ep_graph_begin(stream) and ep_graph_end(stream, &g)
 * every ep_* call (and any other work) enqueued on `stream` is recorded, not
 * run; `stream` must not be the null stream.  ep_graph_launch replays the
 * recorded work on any stream with the pointers and sizes it was recorded
 * with.  ep_graph_destroy frees the graph (host call; the graph must not be
 * running).  Return codes as above; *graph is set only on success.
 */
int ep_graph_begin(void* stream);
int ep_graph_end(void* stream, void** graph);
int ep_graph_launch(void* graph, void* stream);
int ep_graph_destroy(void* graph);

/*
 * Encode n fp32 values with the same e4m3fn encoder the fp8 dispatch uses
 * (round to nearest even, saturating, NaN -> 0x7F|sign; below 464 in
 * magnitude the conversion instruction alone, from there on after a clamp to
 * +-448).  in: fp32 [n], out: uint8 [n], both device pointers (4 B / 1 B
 * aligned).  For checking the encoder against the format definition over
 * whole ranges of inputs.
 */
int ep_e4m3fn_encode(const float* in, int64_t n, uint8_t* out, void* stream);

/*
 * int64 expert ids (the index type a framework's top-k returns) to the int32
 * ids the layout calls take, on the GPU: topk_idx32[i] = -1 for a negative
 * topk_idx64[i] (negative ids are the sentinel for a dropped entry: MoRI PR
 * #614 "perf(ep): InterNodeV1LL low-token latency on MI300X + CX7", routing
 * scan paragraph), INT32_MAX for one above INT32_MAX (a bad id the layout then
 * reports in its status), the value itself otherwise.  n entries;
 * topk_idx64 8-B and topk_idx32 4-B aligned device pointers.  One extra
 * launch: a router that emits int32 ids needs none.
 * Errors: EP_EINVAL for n < 0, NULL or misaligned pointers when n > 0.
 */
int ep_topk_idx_narrow(const int64_t* topk_idx64, int64_t n, int32_t* topk_idx32, void* stream);

/* Message for a return code; static storage. */
const char* ep_strerror(int code);
/* hipError_t of the last failed launch in the calling thread (0 if none). */
int ep_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* EP_MI355X_H */
