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
// v_mfma_f32_32x32x16_bf16: D[32][32] += A[32][16] * B[16][32]. Lane l supplies row l%32 of A
// and column l%32 of B, each as 8 bf16 of the k-group l/32; D lane l holds column l%32, rows
// 8*(v/4) + 4*(l/32) + v%4 for v = 0..15. Which k an (k-group, element) slot stands for is the
// same for A and B, so any assignment of k's to slots gives the full 16-term sum; a Q8_0 block
// (32 k) is one pair of MFMAs when lane group g holds the block's bytes [16g, 16g+16) and MFMA
// m in {0,1} takes bytes [8m, 8m+8) of them.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

GQ8_DEV f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// row of D held in accumulator slot v by lane l
GQ8_DEV int mfma32_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// ------------------------------------------------------------------ wave64 reductions

template <int CTRL>
GQ8_DEV float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes; every lane gets the same bits (each step adds a symmetric pair).
GQ8_DEV float wave_sum(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);  // row_half_mirror
    v += dpp_mov<0x140>(v);  // row_mirror
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

GQ8_DEV int wave_sum_i32(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, true);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// ------------------------------------------------------------------ split-K arrival
//
// Partial sums that another work-group (possibly on another XCD, behind another L2) will read
// are written and read with device-scope atomic stores / loads (the sc1 cache policy): they are
// coherent across the L2s without a full-cache writeback or invalidate, which is what an
// agent-scope fence costs on this chip (tens of microseconds per kernel when every wave
// fences). Ordering: each thread waits for its own stores to complete (vmcnt(0)) before the
// work-group barrier, so every partial of the work-group is device-visible before thread 0's
// counter increment; the last arriver's loads are issued after it has read the counter.

template <typename V>
GQ8_DEV void st_dev(V* p, V v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename V>
GQ8_DEV V ld_dev(const V* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Wait until this thread's outstanding memory operations have completed (vmcnt(0)).
GQ8_DEV void wait_stores() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // gfx9 encoding: vmcnt(0) expcnt(7) lgkmcnt(15)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Sum of S device-coherent values p[0], p[stride], ..., ascending, with the loads issued in
// groups of 8 so their latencies overlap.
template <typename V>
GQ8_DEV V sum_planes(const V* p, size_t stride, int S) {
    V acc = 0;
    for (int s0 = 0; s0 < S; s0 += 8) {
        V v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = s0 + i < S ? ld_dev(p + (size_t)(s0 + i) * stride) : (V)0;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += v[i];
    }
    return acc;
}

// Called by every thread of a work-group after it has stored its partial sums with st_dev().
// Returns true in every thread of the work-group that arrives last among `nsplit` work-groups
// sharing `counter`; that work-group then reads all partial sums with ld_dev() and the counter
// is reset to zero. Nobody waits for anybody: no co-residency is assumed, and a graph replay
// starts from the zero the previous call left.
GQ8_DEV bool splitk_last_arrival(unsigned* counter, unsigned nsplit, int* s_flag) {
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = atomicAdd(counter, 1u);
        const int last = (prev == nsplit - 1u);
        if (last) atomicExch(counter, 0u);
        *s_flag = last;
    }
    __syncthreads();
    return *s_flag != 0;
}

}  // namespace gq8
