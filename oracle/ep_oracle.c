/*
 * ep_oracle.c -- CPU oracle for MoE expert-parallel low-latency layout,
 * dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and
 * the bench's cpu_baseline leg load this file's library.  The product path
 * (the HIP library) never calls it, and the two share no code: no headers,
 * helpers, tables or constants.
 *
 * Plain, single-threaded, slow on purpose: every step is the definition of
 * what it computes, in the order the sources state it, with nothing blocked,
 * fused or reordered.  Floating point is fp32 because the method fixes it:
 * the per-128-column scale is an fp32 amax/448 and the combine accumulates in
 * fp32 before writing bf16 (UCCL PR #749 "[EP] Low-latency mode batch tokens
 * per destination" and DeepEP PR #693 "Pipeline direct NVLink dispatch with
 * triple-buffered prefetch", Summary: a dispatched token carries its hidden
 * vector plus scale factors; MoRI PR #614 "perf(ep): InterNodeV1LL low-token
 * latency on MI300X + CX7", tuned-rules paragraph: fp8 dispatch / bf16
 * combine).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off (no -ffast-math).
 * On x86-64 `float` arithmetic is IEEE binary32 on SSE, so `/` is the
 * correctly rounded division and fmaf() is the fused multiply-add.
 *
 * Readings of points the sources leave open (each is also listed with the
 * design notes of the repository):
 *  - slot order: token-ascending within an expert, ties (duplicate ids in
 *    one token) by k, i.e. rows follow the row-major (t,k) order;
 *  - expert->partition map is contiguous, p = e / L with L = E / P
 *    (UCCL PR #749 review excerpt: expert index = rank * experts-per-rank + e);
 *  - "per destination" counts are counts of (t,k) pairs (UCCL PR #749 sums
 *    the per-expert counts of a destination's experts);
 *  - a negative id is a masked entry (MoRI PR #614, routing-scan paragraph:
 *    negative sentinel); an id >= E is reported in status bit 0 and masked;
 *  - fp8 is OCP E4M3 "fn" (bias 7, max 448, no infinities, S.1111.111 NaN),
 *    with saturation and round-to-nearest-even;
 *  - q = E(x / scale) with IEEE fp32 division by the stored scale;
 *    amax = 0 gives scale 0 and all-zero bytes;
 *  - combine: acc = 0, then acc = fmaf(w[t,k], y[row], acc) for k = 0..K-1,
 *    skipping masked entries, then bf16 round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> fp32 is exact: a bf16 is the upper half of an fp32. */
float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/*
 * fp32 -> bf16, round to nearest, ties to even (IEEE 754 roundTiesToEven
 * applied to the 16 discarded low bits).  The two candidates are the
 * truncation `hi` and the next bf16 away from zero `hi + 1` (bit pattern;
 * past the largest finite value that pattern is infinity, which is the IEEE
 * overflow result).  NaN stays NaN, quiet, sign kept.
 */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u = bits_from_f32(f);
    if (isnan(f))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint16_t hi = (uint16_t)(u >> 16);
    uint32_t discarded = u & 0xFFFFu;
    if (discarded > 0x8000u || (discarded == 0x8000u && (hi & 1u)))
        hi = (uint16_t)(hi + 1u);
    return hi;
}

/*
 * OCP OFP8 E4M3 ("fn") value of a code: sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits.  exponent field 0 is subnormal: 2^-6 * m/8.
 * S.1111.111 is NaN; there are no infinities.  Used by tests only.
 */
float oracle_e4m3fn_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return s ? -NAN : NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/*
 * fp32 -> OCP E4M3 "fn", round to nearest with ties to even, saturating.
 *  - NaN -> 0x7F with the sign bit kept;
 *  - |v| >= 448 (the largest finite value; also +-inf) -> 0x7E with sign;
 *  - otherwise |v| is rounded to the nearest representable value, ties to
 *    the even mantissa, with a mantissa carry moving into the exponent;
 *    the sign is kept when the result is zero.
 * Written from the value set: in the subnormal range the representable
 * values are m * 2^-9 (m = 0..8, m = 8 being the smallest normal 2^-6); in
 * binade [2^E, 2^(E+1)) they are m * 2^(E-3), m = 8..16.  Scaling |v| by a
 * power of two is exact, and nearbyint() in the default rounding mode is
 * round-half-to-even.
 */
uint8_t oracle_e4m3fn_encode(float v)
{
    uint8_t sign = (bits_from_f32(v) >> 31) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {
        double m = nearbyint(ldexp(a, 9));           /* 0..8 */
        return (uint8_t)(sign | (uint8_t)m);         /* m = 8 is 0x08 = 2^-6 */
    }
    int fe;
    (void)frexp(a, &fe);                             /* a in [2^(fe-1), 2^fe) */
    int E = fe - 1;                                  /* -6 .. 8 */
    double m = nearbyint(ldexp(a, 3 - E));           /* 8 .. 16 */
    if (m == 16.0) { m = 8.0; E += 1; }
    /* a < 448 keeps the result at or below 448 = 2^8 * 14/8. */
    return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)((int)m - 8));
}

/* Array forms for the tests. */
void oracle_e4m3fn_encode_array(const float* in, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3fn_encode(in[i]);
}
void oracle_bf16_rne_array(const float* in, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(in[i]);
}

/* Argument validation shared by the three steps' conventions. */
static int check_routing(int T, int K, int E, int P)
{
    if (T < 0 || K < 1 || K > 16 || E < 1 || E > 1024 || P < 1 || E % P != 0)
        return ORACLE_EINVAL;
    if ((int64_t)T * K > INT32_MAX)
        return ORACLE_EINVAL;
    return ORACLE_OK;
}

/*
 * Layout: counts per expert and per destination partition, their exclusive
 * scans, and the deterministic slot of every (t,k) pair.
 *
 *  count[e]      = #{(t,k) : idx[t,k] = e}           (negative ids masked;
 *                                                     ids >= E set status
 *                                                     bit 0 and are masked)
 *  offset[0] = 0, offset[e+1] = offset[e] + count[e], N = offset[E]
 *  part_count[p] = sum of count over experts p*L .. p*L+L-1
 *  part_offset[p] = offset[p*L], part_offset[P] = N
 *  row_of_pair[t*K+k] = offset[e] + #{(t',k') before (t,k) in row-major
 *                       order with idx = e}, or -1 for a masked entry
 *  src_pair[row] = t*K+k for row < N, -1 for row in [N, T*K)
 *
 * The per-destination count is the quantity a sender needs before it moves
 * any payload (UCCL PR #749: a destination's batch size is the sum of its
 * local experts' counts); the row-major (t,k) order is the flat work-item
 * order t*K + i of MoRI PR #614 (DispatchIntraNode paragraph).
 */
int oracle_layout(const int32_t* idx, int T, int K, int E, int P,
                  int32_t* expert_count, int32_t* expert_offset,
                  int32_t* part_count, int32_t* part_offset,
                  int32_t* row_of_pair, int32_t* src_pair, uint32_t* status)
{
    if (check_routing(T, K, E, P) != ORACLE_OK)
        return ORACLE_EINVAL;
    const int L = E / P;
    const int64_t npairs = (int64_t)T * K;
    uint32_t st = 0;

    for (int e = 0; e < E; ++e) expert_count[e] = 0;
    for (int64_t i = 0; i < npairs; ++i) {
        int32_t e = idx[i];
        if (e < 0) continue;
        if (e >= E) { st |= 1u; continue; }
        expert_count[e] += 1;
    }

    expert_offset[0] = 0;
    for (int e = 0; e < E; ++e) expert_offset[e + 1] = expert_offset[e] + expert_count[e];
    const int32_t N = expert_offset[E];

    for (int p = 0; p < P; ++p) {
        int32_t s = 0;
        for (int e = p * L; e < p * L + L; ++e) s += expert_count[e];
        part_count[p] = s;
        part_offset[p] = expert_offset[p * L];
    }
    part_offset[P] = N;

    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) return ORACLE_EINVAL;
    for (int e = 0; e < E; ++e) cursor[e] = expert_offset[e];
    for (int64_t i = 0; i < npairs; ++i) {
        int32_t e = idx[i];
        if (e < 0 || e >= E) { row_of_pair[i] = -1; continue; }
        int32_t r = cursor[e]++;
        row_of_pair[i] = r;
        src_pair[r] = (int32_t)i;
    }
    for (int64_t r = N; r < npairs; ++r) src_pair[r] = -1;
    free(cursor);
    *status = st;
    return ORACLE_OK;
}

/*
 * fp8 dispatch of tokens [t0, t1).  For each token and each block of 128
 * columns: amax = max |x| (fmaxf, which ignores NaN), scale = amax / 448 in
 * fp32, q = E(x / scale) (0x00 for the whole block when amax = 0).  The same
 * bytes and scale are written to every valid row of the token; rows of
 * masked entries and rows >= N are not touched.
 * recv_x is [rows, H] bytes, recv_scales is [rows, H/128] fp32, row-major.
 */
int oracle_dispatch_fp8_range(const uint16_t* x, int T, int H, int K,
                              const int32_t* row_of_pair, int t0, int t1,
                              uint8_t* recv_x, float* recv_scales)
{
    if (T < 0 || H <= 0 || H % 128 != 0 || K < 1 || K > 16 || t0 < 0 || t1 > T || t0 > t1)
        return ORACLE_EINVAL;
    const int nb = H / 128;
    uint8_t q[128];
    for (int t = t0; t < t1; ++t) {
        for (int b = 0; b < nb; ++b) {
            const uint16_t* xb = x + (int64_t)t * H + (int64_t)b * 128;
            float amax = 0.0f;
            for (int j = 0; j < 128; ++j) amax = fmaxf(amax, fabsf(oracle_bf16_to_f32(xb[j])));
            float scale = amax / 448.0f;
            for (int j = 0; j < 128; ++j)
                q[j] = (amax == 0.0f) ? 0x00 : oracle_e4m3fn_encode(oracle_bf16_to_f32(xb[j]) / scale);
            if (amax == 0.0f) scale = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t r = row_of_pair[(int64_t)t * K + k];
                if (r < 0) continue;
                memcpy(recv_x + (int64_t)r * H + (int64_t)b * 128, q, 128);
                recv_scales[(int64_t)r * nb + b] = scale;
            }
        }
    }
    return ORACLE_OK;
}

int oracle_dispatch_fp8(const uint16_t* x, int T, int H, int K, const int32_t* row_of_pair,
                        uint8_t* recv_x, float* recv_scales)
{
    return oracle_dispatch_fp8_range(x, T, H, K, row_of_pair, 0, T, recv_x, recv_scales);
}

/* bf16 passthrough dispatch: the token's H bf16 values copied verbatim into
 * every valid row (no scales). */
int oracle_dispatch_bf16(const uint16_t* x, int T, int H, int K, const int32_t* row_of_pair,
                         uint16_t* recv_x)
{
    if (T < 0 || H <= 0 || K < 1 || K > 16)
        return ORACLE_EINVAL;
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int32_t r = row_of_pair[(int64_t)t * K + k];
            if (r < 0) continue;
            memcpy(recv_x + (int64_t)r * H, x + (int64_t)t * H, (size_t)H * 2);
        }
    return ORACLE_OK;
}

/*
 * Combine of tokens [t0, t1): out[t,c] = bf16_rne(acc) where acc starts at
 * 0.0f and, for k = 0..K-1 with r = row_of_pair[t,k] >= 0,
 * acc = fmaf(w[t,k], y[r,c], acc).  A token whose entries are all masked
 * gives +0.  y has the same row layout as the dispatch receive buffer.
 */
int oracle_combine_range(const uint16_t* y, const int32_t* row_of_pair, const float* w,
                         int T, int H, int K, int t0, int t1, uint16_t* out)
{
    if (T < 0 || H <= 0 || K < 1 || K > 16 || t0 < 0 || t1 > T || t0 > t1)
        return ORACLE_EINVAL;
    for (int t = t0; t < t1; ++t)
        for (int c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t r = row_of_pair[(int64_t)t * K + k];
                if (r < 0) continue;
                acc = fmaf(w[(int64_t)t * K + k], oracle_bf16_to_f32(y[(int64_t)r * H + c]), acc);
            }
            out[(int64_t)t * H + c] = oracle_bf16_rne(acc);
        }
    return ORACLE_OK;
}

int oracle_combine(const uint16_t* y, const int32_t* row_of_pair, const float* w,
                   int T, int H, int K, uint16_t* out)
{
    return oracle_combine_range(y, row_of_pair, w, T, H, K, 0, T, out);
}

/*
 * Per-destination deduplicated layout (a token travels once to each partition
 * that holds any of its valid experts; UCCL PR #749: tokens batched per
 * destination; MoRI PR #614, DispatchIntraNode paragraph: the dispatch
 * de-duplicates a token's copies per destination).
 *
 *  kmask[t*P+p]        = bit k set iff idx[t,k] is a valid id in partition p
 *  present(t,p)        = kmask[t*P+p] != 0
 *  part_tokens[p]      = #{t : present(t,p)}
 *  part_token_off[0]=0, part_token_off[p+1] = part_token_off[p] + part_tokens[p]; M = part_token_off[P]
 *  tp_row[t*P+p]       = part_token_off[p] + #{t' < t : present(t',p)}, or -1
 *  tp_src[row]         = t*P+p for row < M, -1 for row in [M, T*P)
 *  status bit 0        = some id >= E
 */
int oracle_dedup_layout(const int32_t* idx, int T, int K, int E, int P,
                        int32_t* tp_row, int32_t* part_tokens, int32_t* part_token_off,
                        int32_t* tp_src, uint32_t* kmask, uint32_t* status)
{
    if (check_routing(T, K, E, P) != ORACLE_OK || P > 16)
        return ORACLE_EINVAL;
    const int L = E / P;
    uint32_t st = 0;
    for (int64_t i = 0; i < (int64_t)T * P; ++i) kmask[i] = 0;
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int32_t e = idx[(int64_t)t * K + k];
            if (e < 0) continue;
            if (e >= E) { st |= 1u; continue; }
            kmask[(int64_t)t * P + e / L] |= 1u << k;
        }
    for (int p = 0; p < P; ++p) {
        int32_t c = 0;
        for (int t = 0; t < T; ++t) c += kmask[(int64_t)t * P + p] != 0;
        part_tokens[p] = c;
    }
    part_token_off[0] = 0;
    for (int p = 0; p < P; ++p) part_token_off[p + 1] = part_token_off[p] + part_tokens[p];
    const int64_t M = part_token_off[P];
    for (int p = 0; p < P; ++p) {
        int32_t cursor = part_token_off[p];
        for (int t = 0; t < T; ++t) {
            int64_t i = (int64_t)t * P + p;
            if (kmask[i] == 0) { tp_row[i] = -1; continue; }
            tp_row[i] = cursor;
            tp_src[cursor] = (int32_t)i;
            ++cursor;
        }
    }
    for (int64_t r = M; r < (int64_t)T * P; ++r) tp_src[r] = -1;
    *status = st;
    return ORACLE_OK;
}

/*
 * Two-level combine, level 1 (at the destination): for every present (t,p),
 * acc = 0.0f, then acc = fmaf(w[t,k], y[row_of_pair[t,k], c], acc) for the k
 * of kmask[t*P+p] in ascending order whose row is a receive row (>= 0; a
 * masked entry contributes nothing, as in the plain combine);
 * partial[tp_row[t,p], c] = bf16_rne(acc).  y is in the pair-row layout of
 * the plain dispatch.
 */
int oracle_combine_partial(const uint16_t* y, const int32_t* row_of_pair, const float* w,
                           const int32_t* tp_row, const uint32_t* kmask,
                           int T, int H, int K, int P, uint16_t* partial)
{
    if (T < 0 || H <= 0 || K < 1 || K > 16 || P < 1 || P > 16)
        return ORACLE_EINVAL;
    for (int t = 0; t < T; ++t)
        for (int p = 0; p < P; ++p) {
            int64_t i = (int64_t)t * P + p;
            int32_t dst = tp_row[i];
            if (dst < 0) continue;
            for (int c = 0; c < H; ++c) {
                float acc = 0.0f;
                for (int k = 0; k < K; ++k) {
                    if (!(kmask[i] >> k & 1u)) continue;
                    int32_t r = row_of_pair[(int64_t)t * K + k];
                    if (r < 0) continue;
                    acc = fmaf(w[(int64_t)t * K + k], oracle_bf16_to_f32(y[(int64_t)r * H + c]), acc);
                }
                partial[(int64_t)dst * H + c] = oracle_bf16_rne(acc);
            }
        }
    return ORACLE_OK;
}

/*
 * Two-level combine, level 2 (at the source): acc = 0.0f, then
 * acc = acc + partial[tp_row[t,p], c] for p ascending over present (t,p)
 * (fp32 adds); out[t,c] = bf16_rne(acc).  A token present nowhere gives +0.
 */
int oracle_combine_reduce(const uint16_t* partial, const int32_t* tp_row, int T, int H, int P,
                          uint16_t* out)
{
    if (T < 0 || H <= 0 || P < 1 || P > 16)
        return ORACLE_EINVAL;
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int p = 0; p < P; ++p) {
                int32_t r = tp_row[(int64_t)t * P + p];
                if (r < 0) continue;
                acc = acc + oracle_bf16_to_f32(partial[(int64_t)r * H + c]);
            }
            out[(int64_t)t * H + c] = oracle_bf16_rne(acc);
        }
    return ORACLE_OK;
}
