// ep_numerics.h -- fp8 (OCP e4m3fn) quantisation and bf16 rounding on gfx950.
//
// e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; largest finite 448;
// S.1111.111 is NaN; no infinities.  gfx950's v_cvt_pk_fp8_f32 converts to
// this format with round-to-nearest-even.  Values beyond +-448 (only reachable
// from a non-finite or degenerate scale) are clamped first so the result
// saturates; NaN is passed through the clamp untouched.
#pragma once

#include "ep_device.h"

namespace ep {

constexpr float kE4m3Max = 448.0f;

// Saturating clamp to [-448, 448] that leaves NaN as NaN.
__device__ __forceinline__ float clamp_e4m3(float q)
{
    const float c = __builtin_fminf(__builtin_fmaxf(q, -kE4m3Max), kE4m3Max);
    return (q != q) ? q : c;
}

// Pack four fp32 values (already divided by the scale) into four e4m3fn bytes,
// little-endian in column order.
__device__ __forceinline__ uint32_t pack4_e4m3fn(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), clamp_e4m3(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c), clamp_e4m3(d), w, true);
    return (uint32_t)w;
}

// One value, as the dispatch encodes it: below 464 in magnitude the bare
// instruction (the quotient fast path), from 464 up and for NaN after the
// clamp (the IEEE-division path) -- so a range check of this function covers
// the instruction's rounding of (448, 464) to 448 that the fast path relies on.
__device__ __forceinline__ uint8_t encode_e4m3fn_one(float a)
{
    const float c = (__builtin_fabsf(a) < 464.0f) ? a : clamp_e4m3(a);
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false);
    return (uint8_t)(w & 0xFF);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Max over the 16 lanes of this lane's DPP row of non-negative, non-NaN fp32
// values (per-lane maxima that start from 0 and take fmaxf, which drops NaN),
// taken on their bit patterns, which order like the values.  Integer max
// lets each step be one DPP-fused v_max_i32 (a float max would first have to
// quiet the moved operand).
__device__ __forceinline__ float row16_max(float a)
{
    int k = __builtin_bit_cast(int, a);
    // the DPP control must be a constant expression, hence the spelled-out steps
    k = __builtin_elementwise_max(k, __builtin_amdgcn_update_dpp(0, k, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    k = __builtin_elementwise_max(k, __builtin_amdgcn_update_dpp(0, k, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    k = __builtin_elementwise_max(k, __builtin_amdgcn_update_dpp(0, k, 0x141, 0xF, 0xF, false));  // row_half_mirror
    k = __builtin_elementwise_max(k, __builtin_amdgcn_update_dpp(0, k, 0x140, 0xF, 0xF, false));  // row_mirror
    return __builtin_bit_cast(float, k);
}

// amax / 448 correctly rounded without a division: with c = RN(1/448),
// q0 = amax*c, r = fma(-q0, 448, amax) (exact remainder), scale = fma(r, c, q0).
// Equal to the IEEE quotient for every finite bf16 amax (all 32640 checked on
// the CPU and on gfx950); an infinite or NaN amax makes r NaN and keeps q0,
// which is then amax*c = amax/448 (inf or NaN).
constexpr float kInv448 = 0x1.24924ap-9f;
__device__ __forceinline__ float block_scale(float amax)
{
    const float q0 = amax * kInv448;
    const float r = __builtin_fmaf(-q0, kE4m3Max, amax);
    return (r == r) ? __builtin_fmaf(r, kInv448, q0) : q0;
}

// Smallest scale for which the quotient shortcut below reproduces the IEEE
// division's fp8 byte for every bf16 input.
constexpr float kFastQuotientMinScale = 0x1p-90f;

// Quantise this lane's 8 bf16 values (16 bytes) with the scale of its
// 128-column block (= its 16-lane DPP row).  Must be called by all 64 lanes.
// scale = amax / 448 (the IEEE fp32 quotient; 0 when amax is 0); each byte is
// e4m3fn(x / scale) with x / scale the IEEE-rounded fp32 quotient; a zero block
// gives zero bytes.
//
// The quotient: y = RN(1/scale) per lane, then per element q0 = |x|*y,
// r = fma(-q0, scale, |x|) (the exact remainder), q = fma(r, y, q0) with x's
// sign -- the reciprocal-and-remainder correction step of IA-64-style
// division (Markstein).  Checked exhaustively on the CPU: over every pair of
// bf16 values x, amax with |x| <= amax and scale >= 2^-90 it yields the same
// e4m3fn byte as IEEE division (its fp32 result can differ only below 2^-10,
// where both encode to a signed zero).  y itself is v_rcp_f32 (within 1 ulp)
// plus one Newton step with fma, which gives RN(1/scale) for every scale a
// bf16 amax can produce (checked on gfx950 against the IEEE reciprocal).
// There |q| < 448.0001, which v_cvt_pk_fp8_f32 rounds to +-448 (it returns
// NaN only from 464 up), so this path needs no clamp.  Smaller (or
// non-finite) scales take the IEEE division and the saturating clamp.
__device__ __forceinline__ uint2 quantise_e4m3fn_block8(uint4 v, float& scale)
{
    float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
    amax = row16_max(amax);
    scale = block_scale(amax);
    uint2 q = make_uint2(0u, 0u);
    if (amax != 0.0f) {
        if (scale >= kFastQuotientMinScale && scale <= 0x1.fffffep+127f) {
            const float y0 = __builtin_amdgcn_rcpf(scale);
            const float y = __builtin_fmaf(__builtin_fmaf(-scale, y0, 1.0f), y0, y0);
            float d[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float a = __builtin_fabsf(f[i]);
                const float q0 = a * y;
                const float r = __builtin_fmaf(-q0, scale, a);
                d[i] = __builtin_copysignf(__builtin_fmaf(r, y, q0), f[i]);
            }
            int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(d[0], d[1], 0, false);
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(d[2], d[3], w0, true);
            int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(d[4], d[5], 0, false);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(d[6], d[7], w1, true);
            q = make_uint2((uint32_t)w0, (uint32_t)w1);
        } else {
            float d[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) d[i] = f[i] / scale;
            q.x = pack4_e4m3fn(d[0], d[1], d[2], d[3]);
            q.y = pack4_e4m3fn(d[4], d[5], d[6], d[7]);
        }
    }
    return q;
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi)
{
    const uint16_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
    const uint16_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
    return (uint32_t)a | ((uint32_t)b << 16);
}

}  // namespace ep
