/*
 * Exhaustive check of the quotient shortcut the fp8 dispatch kernel uses
 * (test infrastructure; linked with the oracle's encoder).
 *
 * For every pair of finite bf16 values with 0 <= |x| <= amax (amax > 0), with
 * scale = amax / 448 in IEEE fp32: if scale >= 2^-90, the shortcut
 *     y = 1/scale, q0 = |x|*y, r = fma(-q0, scale, |x|), q = sign(x)*fma(r, y, q0)
 * must give the same OCP e4m3fn byte as the IEEE-rounded quotient x / scale.
 * argv[3] = -1 or +1 runs the same check with y one ulp below or above
 * RN(1/scale); passing for -1, 0 and +1 shows that any reciprocal within one
 * ulp of the correctly rounded one (a faithful v_rcp_f32, or one refined by a
 * Newton step) gives the same bytes.
 * Prints the pair count and the number of differing bytes; exit status 1 if
 * any byte differs.  argv[1] = stride over amax codes (1 = all), argv[2] = 1
 * to also run the negative x values.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint8_t oracle_e4m3fn_encode(float v);

static float from_bf16(uint32_t h) { uint32_t u = h << 16; float f; memcpy(&f, &u, 4); return f; }

int main(int argc, char** argv)
{
    const unsigned stride = argc > 1 ? (unsigned)atoi(argv[1]) : 1u;
    const int negatives = argc > 2 ? atoi(argv[2]) : 0;
    const int yoff = argc > 3 ? atoi(argv[3]) : 0;
    long long pairs = 0, bad = 0, fast_blocks = 0;
    for (uint32_t m = 1; m <= 0x7F7Fu; m += stride) {
        const float amax = from_bf16(m);
        const float scale = amax / 448.0f;
        if (!(scale >= 0x1p-90f && isfinite(scale))) continue;
        ++fast_blocks;
        volatile float one = 1.0f;
        const float yrn = one / scale;
        const float y = yoff < 0 ? nextafterf(yrn, 0.0f) : yoff > 0 ? nextafterf(yrn, INFINITY) : yrn;
        for (uint32_t a16 = 0; a16 <= m; ++a16) {
            for (int sg = 0; sg <= negatives; ++sg) {
                const float x = from_bf16(a16 | (sg ? 0x8000u : 0u));
                const float a = fabsf(x);
                const float q0 = a * y;
                const float r = fmaf(-q0, scale, a);
                const float q = copysignf(fmaf(r, y, q0), x);
                ++pairs;
                if (oracle_e4m3fn_encode(q) != oracle_e4m3fn_encode(x / scale)) {
                    if (++bad <= 5)
                        printf("differs: amax=%a x=%a y=%a ieee=%a shortcut=%a\n", amax, x, y,
                               x / scale, q);
                }
            }
        }
    }
    printf("amax values %lld checks %lld differing bytes %lld\n", fast_blocks, pairs, bad);
    return bad != 0;
}
