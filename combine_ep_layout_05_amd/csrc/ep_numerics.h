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

__device__ __forceinline__ uint8_t encode_e4m3fn_one(float a)
{
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), 0.0f, 0, false);
    return (uint8_t)(w & 0xFF);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Max over the 16 lanes of this lane's DPP row (rows are lanes 16r .. 16r+15).
__device__ __forceinline__ float row16_max(float a)
{
    // the DPP control must be a constant expression, hence the spelled-out steps
    a = __builtin_fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                               0, __builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, false)));   // quad_perm [1,0,3,2]
    a = __builtin_fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                               0, __builtin_bit_cast(int, a), 0x4E, 0xF, 0xF, false)));   // quad_perm [2,3,0,1]
    a = __builtin_fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                               0, __builtin_bit_cast(int, a), 0x141, 0xF, 0xF, false)));  // row_half_mirror
    a = __builtin_fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                               0, __builtin_bit_cast(int, a), 0x140, 0xF, 0xF, false)));  // row_mirror
    return a;
}

// Smallest scale for which the quotient shortcut below reproduces the IEEE
// division's fp8 byte for every bf16 input.
constexpr float kFastQuotientMinScale = 0x1p-90f;

// Quantise this lane's 8 bf16 values (16 bytes) with the scale of its
// 128-column block (= its 16-lane DPP row).  Must be called by all 64 lanes.
// scale = amax / 448 (IEEE fp32 division; 0 when amax is 0); each byte is
// e4m3fn(x / scale) with x / scale the IEEE-rounded fp32 quotient; a zero block
// gives zero bytes.
//
// The quotient: one IEEE reciprocal y = 1/scale per lane, then per element
// q0 = |x|*y, r = fma(-q0, scale, |x|) (the exact remainder), q = fma(r, y, q0)
// with x's sign -- the reciprocal-and-remainder correction step of
// IA-64-style division (Markstein).  Checked exhaustively on the CPU: over
// every pair of bf16 values x, amax with |x| <= amax and scale >= 2^-90 it
// yields the same e4m3fn byte as IEEE division (its fp32 result can differ
// only below 2^-10, where both encode to a signed zero).  Smaller (or
// non-finite) scales take the IEEE division.
__device__ __forceinline__ uint2 quantise_e4m3fn_block8(uint4 v, float& scale)
{
    float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
    amax = row16_max(amax);
    scale = amax / kE4m3Max;
    uint2 q = make_uint2(0u, 0u);
    if (amax != 0.0f) {
        float d[8];
        if (scale >= kFastQuotientMinScale && scale <= 0x1.fffffep+127f) {
            const float y = 1.0f / scale;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float a = __builtin_fabsf(f[i]);
                const float q0 = a * y;
                const float r = __builtin_fmaf(-q0, scale, a);
                d[i] = __builtin_copysignf(__builtin_fmaf(r, y, q0), f[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) d[i] = f[i] / scale;
        }
        q.x = pack4_e4m3fn(d[0], d[1], d[2], d[3]);
        q.y = pack4_e4m3fn(d[4], d[5], d[6], d[7]);
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
