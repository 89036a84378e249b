// Device-side helpers shared by the gq8 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define GQ8_DEV __device__ __forceinline__

namespace gq8 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: the weight bytes are read once)
GQ8_DEV u32x4 ld_nt16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ------------------------------------------------------------------ number formats

GQ8_DEV float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default rounding mode)
GQ8_DEV uint16_t f2h_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

GQ8_DEV float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN
GQ8_DEV uint16_t f2bf_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// round to nearest integer, ties away from zero; trunc(v) and v - trunc(v) are exact in fp32
GQ8_DEV int round_half_away(float v) {
    const float t = truncf(v);
    const float r = fabsf(v - t) >= 0.5f ? t + copysignf(1.0f, v) : t;
    return (int)r;
}

// Q8_0 / q8_1 block scale: fp16 bits of amax / 127 (round to nearest even)
GQ8_DEV uint16_t q8_scale_bits(float amax) { return f2h_bits(amax / 127.0f); }

// one quant of a block with (fp16-exact) scale d: round(v / d), clamped to +-127; 0 when d = 0
GQ8_DEV int q8_quant(float v, float d) {
    if (d == 0.f) return 0;
    const int qi = round_half_away(v / d);
    return qi > 127 ? 127 : (qi < -127 ? -127 : qi);
}

// q8_quant for a bf16 value v (8-bit significand) and a block scale d = fp16 (11-bit significand)
// without the division: v / d = (a / m) 2^e with a < 2^8 and m < 2^11 integers, so unless v / d
// is a half-integer it lies at least 2^-12 from every half-integer, while t = |v| * rcp(d) is
// within 2^-15 of it (|v / d| <= 128, v_rcp_f32 within 1 ulp): rounding t half up gives the same
// integer, and an exact tie (|v| = (q + 0.5) d, a product exact in fp32) goes away from zero.
// The result is q8_quant(v, d) bit for bit; d must be finite (callers take q8_quant otherwise).
GQ8_DEV int q8_quant_bf16(float v, float d, float rd) {
    if (d == 0.f) return 0;
    const float av = fabsf(v);
    int q = (int)(av * rd + 0.5f);
    if (((float)q + 0.5f) * d == av) q += 1;
    q = q > 127 ? 127 : q;
    return v < 0.f ? -q : q;
}

// signed byte i (0..3) of a dword, as float
template <int I>
GQ8_DEV float sbyte_f(uint32_t w) { return (float)(int)(int8_t)(uint8_t)(w >> (8 * I)); }

// sum_{i<4} byte_i(w) * x[i] added to acc, in order
GQ8_DEV float dot4_i8_f32(uint32_t w, const float* x, float acc) {
    acc = fmaf(sbyte_f<0>(w), x[0], acc);
    acc = fmaf(sbyte_f<1>(w), x[1], acc);
    acc = fmaf(sbyte_f<2>(w), x[2], acc);
    acc = fmaf(sbyte_f<3>(w), x[3], acc);
    return acc;
}

// 16 signed bytes dotted with x[0..16), sequential fp32
GQ8_DEV float dot16_i8_f32(u32x4 w, const float* x) {
    float s = 0.f;
    s = dot4_i8_f32(w.x, x + 0, s);
    s = dot4_i8_f32(w.y, x + 4, s);
    s = dot4_i8_f32(w.z, x + 8, s);
    s = dot4_i8_f32(w.w, x + 12, s);
    return s;
}

// ------------------------------------------------------------------ bf16 MFMA fragments
//
// v_mfma_f32_16x16x32_bf16: D[16][16] += A[16][32] * B[32][16]. Lane l supplies row l%16 of A
// and column l%16 of B as 8 bf16 of k-group l/16; D lane l holds column l%16, rows 4*(l/16) + v
// for v = 0..3. Which k an (k-group, element) slot stands for is the same for A and B, so any
// assignment of k's to slots gives the full 32-term sum: one Q8_0 block (32 k) is one MFMA.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

GQ8_DEV f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// two fp32 whose low 16 bits are zero -> packed bf16 pair (lo in bits 0..15)
GQ8_DEV uint32_t pack_bf16_trunc(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 8 signed bytes (two dwords) -> 8 bf16, exact (|q| <= 128 fits the bf16 significand)
GQ8_DEV bf16x8 i8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    u32x4 r;
    r.x = pack_bf16_trunc(sbyte_f<0>(w0), sbyte_f<1>(w0));
    r.y = pack_bf16_trunc(sbyte_f<2>(w0), sbyte_f<3>(w0));
    r.z = pack_bf16_trunc(sbyte_f<0>(w1), sbyte_f<1>(w1));
    r.w = pack_bf16_trunc(sbyte_f<2>(w1), sbyte_f<3>(w1));
    return __builtin_bit_cast(bf16x8, r);
}

// ------------------------------------------------------------------ wave64 reductions

template <int CTRL>
GQ8_DEV float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Lane l's value from lane l ^ 16 / l ^ 32 (v_permlane16_swap / v_permlane32_swap, no LDS), from
// l ^ 8 (DPP row rotate by 8 within a 16-lane row), and from l ^ 1 / l ^ 2 (DPP quad_perm).
GQ8_DEV uint32_t lane_xor16(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
}
GQ8_DEV uint32_t lane_xor32(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
}
template <int CTRL>
GQ8_DEV uint32_t dpp_u32(uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true); }
GQ8_DEV uint32_t lane_xor8(uint32_t v) { return dpp_u32<0x128>(v); }      // row_ror:8
GQ8_DEV uint32_t lane_xor1(uint32_t v) { return dpp_u32<0xB1>(v); }       // quad_perm [1,0,3,2]
GQ8_DEV uint32_t lane_xor2(uint32_t v) { return dpp_u32<0x4E>(v); }       // quad_perm [2,3,0,1]
GQ8_DEV float lane_xor16f(float v) { return __uint_as_float(lane_xor16(__float_as_uint(v))); }
GQ8_DEV float lane_xor32f(float v) { return __uint_as_float(lane_xor32(__float_as_uint(v))); }
GQ8_DEV float lane_xor8f(float v) { return __uint_as_float(lane_xor8(__float_as_uint(v))); }
GQ8_DEV float lane_xor1f(float v) { return __uint_as_float(lane_xor1(__float_as_uint(v))); }
GQ8_DEV float lane_xor2f(float v) { return __uint_as_float(lane_xor2(__float_as_uint(v))); }

// Max over the 64 lanes of unsigned values (every lane gets it)
GQ8_DEV uint32_t wave_max_u32(uint32_t v) {
    v = max(v, lane_xor1(v));
    v = max(v, lane_xor2(v));
    v = max(v, dpp_u32<0x141>(v));   // row_half_mirror: the other quad of the half-row
    v = max(v, lane_xor8(v));
    v = max(v, lane_xor16(v));
    v = max(v, lane_xor32(v));
    return v;
}

// Sum over the 64 lanes; every lane gets the same bits (each step adds a symmetric pair): the DPP
// steps within each 16-lane row, then v_permlane16_swap and v_permlane32_swap (gfx950) bring in
// the neighbouring row and the other half, with no LDS round trip.
GQ8_DEV float wave_sum(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);  // row_half_mirror
    v += dpp_mov<0x140>(v);  // row_mirror
    const int lane = threadIdx.x & 63;
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v += __uint_as_float((lane & 16) ? r[0] : r[1]);          // lane l ^ 16
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v += __uint_as_float((lane & 32) ? h[0] : h[1]);          // lane l ^ 32
    return v;
}

}  // namespace gq8
