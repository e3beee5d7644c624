/* Drives every function of oracle/ep_oracle.c over random small cases and
 * edge cases, with buffers of exactly the documented sizes, so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (host code only) fails
 * on any out-of-bounds access, shift or overflow.  Prints "ok" at the end. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_layout(const int32_t*, int, int, int, int, int32_t*, int32_t*, int32_t*, int32_t*,
                  int32_t*, int32_t*, uint32_t*);
int oracle_dispatch_fp8(const uint16_t*, int, int, int, const int32_t*, uint8_t*, float*);
int oracle_dispatch_bf16(const uint16_t*, int, int, int, const int32_t*, uint16_t*);
int oracle_combine(const uint16_t*, const int32_t*, const float*, int, int, int, uint16_t*);
int oracle_dedup_layout(const int32_t*, int, int, int, int, int32_t*, int32_t*, int32_t*,
                        int32_t*, uint32_t*, uint32_t*);
int oracle_combine_partial(const uint16_t*, const int32_t*, const float*, const int32_t*,
                           const uint32_t*, int, int, int, int, uint16_t*);
int oracle_combine_reduce(const uint16_t*, const int32_t*, int, int, int, uint16_t*);
void oracle_e4m3fn_encode_array(const float*, int64_t, uint8_t*);
void oracle_bf16_rne_array(const float*, int64_t, uint16_t*);
float oracle_e4m3fn_decode(uint8_t);

static uint64_t s = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return (uint32_t)(s >> 16);
}

static void* xmalloc(size_t n) { return malloc(n ? n : 1); }

static int one_case(int T, int K, int E, int P, int H)
{
    const int n = T * K;
    int32_t* idx = xmalloc((size_t)n * 4);
    for (int i = 0; i < n; ++i) idx[i] = (int32_t)(rnd() % (unsigned)(E + 4)) - 2;
    int32_t *cnt = xmalloc((size_t)E * 4), *off = xmalloc((size_t)(E + 1) * 4);
    int32_t *pc = xmalloc((size_t)P * 4), *po = xmalloc((size_t)(P + 1) * 4);
    int32_t *rop = xmalloc((size_t)n * 4), *src = xmalloc((size_t)n * 4);
    uint32_t st;
    if (oracle_layout(idx, T, K, E, P, cnt, off, pc, po, rop, src, &st)) return 1;

    uint16_t* x = xmalloc((size_t)T * H * 2);
    for (int i = 0; i < T * H; ++i) x[i] = (uint16_t)rnd();      /* any bf16, NaN and inf included */
    uint8_t* rx = xmalloc((size_t)n * H);
    float* rs = xmalloc((size_t)n * (H / 128) * 4);
    if (oracle_dispatch_fp8(x, T, H, K, rop, rx, rs)) return 2;
    uint16_t* rb = xmalloc((size_t)n * H * 2);
    if (oracle_dispatch_bf16(x, T, H, K, rop, rb)) return 3;

    uint16_t* y = xmalloc((size_t)n * H * 2);
    for (int i = 0; i < n * H; ++i) y[i] = (uint16_t)(rnd() & 0x7F7Fu);
    float* w = xmalloc((size_t)n * 4);
    for (int i = 0; i < n; ++i) w[i] = (float)(rnd() % 1000) / 1000.0f;
    uint16_t* out = xmalloc((size_t)T * H * 2);
    if (oracle_combine(y, rop, w, T, H, K, out)) return 4;

    if (P <= 16) {
        int32_t *tpr = xmalloc((size_t)T * P * 4), *pt = xmalloc((size_t)P * 4);
        int32_t *pto = xmalloc((size_t)(P + 1) * 4), *tps = xmalloc((size_t)T * P * 4);
        uint32_t* km = xmalloc((size_t)T * P * 4);
        uint32_t st2;
        if (oracle_dedup_layout(idx, T, K, E, P, tpr, pt, pto, tps, km, &st2)) return 5;
        if (st2 != st) return 6;
        uint16_t* part = xmalloc((size_t)T * P * H * 2);
        if (oracle_combine_partial(y, rop, w, tpr, km, T, H, K, P, part)) return 7;
        uint16_t* out2 = xmalloc((size_t)T * H * 2);
        if (oracle_combine_reduce(part, tpr, T, H, P, out2)) return 8;
        uint8_t* dx = xmalloc((size_t)T * P * H);
        float* ds = xmalloc((size_t)T * P * (H / 128) * 4);
        if (oracle_dispatch_fp8(x, T, H, P, tpr, dx, ds)) return 9;
        free(tpr); free(pt); free(pto); free(tps); free(km); free(part); free(out2); free(dx); free(ds);
    }
    free(idx); free(cnt); free(off); free(pc); free(po); free(rop); free(src); free(x); free(rx);
    free(rs); free(rb); free(y); free(w); free(out);
    return 0;
}

int main(void)
{
    static const int Es[] = {1, 2, 4, 8, 12, 16, 32, 64, 1024};
    for (int c = 0; c < 400; ++c) {
        const int E = Es[rnd() % (sizeof Es / sizeof Es[0])];
        int P = 1 + (int)(rnd() % (unsigned)(E < 32 ? E : 32));
        while (E % P) --P;
        const int T = (int)(rnd() % 24);
        const int K = 1 + (int)(rnd() % 16);
        const int H = 128 * (1 + (int)(rnd() % 3));
        const int rc = one_case(T, K, E, P, H);
        if (rc) {
            printf("case %d (T=%d K=%d E=%d P=%d H=%d) failed at step %d\n", c, T, K, E, P, H, rc);
            return 1;
        }
    }
    /* the encoders on special values and a stride of all fp32 patterns */
    enum { M = 1 << 16 };
    float* v = malloc(M * sizeof(float));
    uint8_t* q = malloc(M);
    uint16_t* b = malloc(M * 2);
    for (uint64_t base = 0; base < (1ull << 32); base += (uint64_t)M * 4099) {
        for (int i = 0; i < M; ++i) {
            uint32_t bits = (uint32_t)(base + (uint64_t)i * 4099);
            memcpy(&v[i], &bits, 4);
        }
        oracle_e4m3fn_encode_array(v, M, q);
        oracle_bf16_rne_array(v, M, b);
    }
    for (int c = 0; c < 256; ++c) (void)oracle_e4m3fn_decode((uint8_t)c);
    free(v); free(q); free(b);
    printf("ok\n");
    return 0;
}
