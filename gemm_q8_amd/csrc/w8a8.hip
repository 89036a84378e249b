// W8A8 decode product (W8A8 page, operator statement): int8 x_q[M][K] @ int8 W[K][N] -> int32,
// * x_scale[M] * w_scale[N] -> bf16, M = 1..32.
//
// The weight is read as packed 16-column x 64-k fragments (one contiguous 1 KiB wave load,
// 16 bytes per lane). One work-group owns one 16-column tile and ALL of K: its NW waves (up to
// 16) take k-steps w, w+NW, ... and their int32 tiles are added through LDS in wave order, so
// there is no split-K across work-groups, no workspace and no atomics (the W8A8 page splits K
// across blocks because its chip had 120 CUs per 40-160 tiles; here a work-group of 16 waves
// has the same bytes in flight without the combine round trip). Every load of a wave is issued,
// clamped to valid addresses, before the first MFMA / dot.
//   every M: v_mfma_i32_16x16x64_i8 (rows past M are zero), one MFMA row tile for M <= 16 and
//            two (sharing the weight fragment) for M <= 32. One x load per k-step per lane. With
//            at most 128 tiles and M <= 16, two work-groups share a tile, eight columns each, so
//            that twice as many CUs stream the weight (measured: M = 16, N = 1536, K = 4096
//            5.16 -> 5.00 us).
//   the alternative for M <= 15: v_dot4_i32_i8 on the VALU over the same fragments, which needs
//            M x loads per k-step per lane. The environment variable GQ8_W8A8_KERNEL=dot forces
//            it, for comparison (the results are bitwise the same); measured slower at every M,
//            by 0.05 to 0.3 us at M = 1 and from 1.8x at M = 8.
// int32 sums are exact, so every order gives the one correct accumulator; the epilogue is
// bf16( (fp32(acc) * x_scale[m]) * w_scale[n] ), two rounded fp32 products.
#include "gq8_device.h"
#include "gq8_internal.h"

namespace gq8 {

typedef int v4i __attribute__((ext_vector_type(4)));

struct W8Args {
    const int8_t* xq;
    const float* xs;
    const uint16_t* xb;     // bf16 x [M][K] (the variant that quantizes x itself)
    int8_t* xq_out;         //   its quantized x (written by work-group 0; nullable)
    float* xs_out;          //   its x_scale (nullable)
    const int8_t* wp;
    const float* wsc;
    void* out;
    int i32_out;
    int M, N, K;
    int ksteps;
};

GQ8_DEV int imin8(int a, int b) { return a < b ? a : b; }
GQ8_DEV uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// x_scale[m] * ... of the thread's first output (i = thread of the M x 16 tile), loaded at kernel
// start so that the epilogue does not wait for a global load after the reduction.
struct W8Scales {
    float xs, ws;
};

GQ8_DEV W8Scales w8a8_prefetch_scales(const W8Args& a, int n0) {
    const int i = (int)threadIdx.x;
    const int m = imin8(i >> 4, a.M - 1), n = imin8(n0 + (i & 15), a.N - 1);
    W8Scales sc;
    sc.xs = (a.i32_out || a.xs == nullptr) ? 0.f : a.xs[m];
    sc.ws = a.i32_out ? 0.f : a.wsc[n];
    return sc;
}

// The WG's int32 tiles [NW][32][16] -> sum over waves (in wave order) -> epilogue. xs_lds: the
// x scales computed in the work-group (the variant that quantizes x), else a.xs.
GQ8_DEV void w8a8_finish(const W8Args& a, int n0, int ncols, int nw, int (*tile)[32][16], W8Scales sc,
                         const float* xs_lds = nullptr) {
    __syncthreads();
    for (int i = threadIdx.x; i < a.M * 16; i += blockDim.x) {
        const int m = i >> 4, nl = i & 15;
        if (nl >= ncols) continue;
        const int n = n0 + nl;
        int p[16];
#pragma unroll
        for (int w = 0; w < 16; ++w) p[w] = tile[w][m][nl];     // all reads in flight
        int v = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) v += w < nw ? p[w] : 0;
        if (n < a.N) {
            if (a.i32_out) {
                reinterpret_cast<int*>(a.out)[(size_t)m * a.N + n] = v;
            } else {
                const bool first = i == (int)threadIdx.x;
                float f = (float)v;
                f = f * (xs_lds != nullptr ? xs_lds[m] : (first ? sc.xs : a.xs[m]));
                f = f * (first ? sc.ws : a.wsc[n]);
                reinterpret_cast<uint16_t*>(a.out)[(size_t)m * a.N + n] = f2bf_bits(f);
            }
        }
    }
}

// k-steps of wave w: w, w + NW, ..., KPW of them (clamped; steps >= ksteps are masked)
template <int KPW>
GQ8_DEV void load_frags(const W8Args& a, int nt, int wave, int nw, int lane, v4i* b, bool* ok) {
    const v4i* f = reinterpret_cast<const v4i*>(a.wp) + (size_t)nt * a.ksteps * 64 + lane;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int ks = wave + i * nw;
        ok[i] = ks < a.ksteps;
        b[i] = __builtin_nontemporal_load(f + (size_t)imin8(ks, a.ksteps - 1) * 64);
    }
}

// x row m, 16 bytes at k (clamped row and k; masked by the caller)
GQ8_DEV v4i load_x16(const W8Args& a, int m, int k) {
    const int mc = imin8(m, a.M - 1), kc = imin8(k, a.K - 16);
    return *reinterpret_cast<const v4i*>(a.xq + (size_t)mc * a.K + kc);
}

// 8 bf16 (one 16-byte load) -> 8 int8 quants round_half_away(v * inv), which stay in [-127, 127].
// y = v * inv is rounded to fp32 first (contraction off), then round half away from zero is
// trunc(y + copysign(0.5 - 2^-25, y)): for |y| >= 0.25 the sum is exact or rounds without crossing
// an integer, except where y is exactly a half-integer, which the bias 0.5 - 2^-25 then carries
// over (checked against the definition on every fp32 in [0.25, 128]); below 0.25 both give 0.
// |v| <= amax and inv = fl(127 / amax) give |y| <= 127 (1 + 2^-24)^2 < 127.5 - 2^-25, so the
// quant never leaves [-127, 127] (a zero row has inv = 0 and all quants 0).
GQ8_DEV uint2 quant8_bf16(u32x4 r, float inv) {
#pragma clang fp contract(off)
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t h = r[e >> 1];
        const float v = __uint_as_float(e & 1 ? (h & 0xffff0000u) : (h << 16));
        const float y = v * inv;
        q[e] = (int)(y + copysignf(0x1.fffffep-2f, y));
    }
    // low bytes of q0..q3 -> one word (byte select 0x0c gives zero)
    const uint32_t p01 = __builtin_amdgcn_perm((uint32_t)q[1], (uint32_t)q[0], 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm((uint32_t)q[3], (uint32_t)q[2], 0x0c0c0400u);
    const uint32_t p45 = __builtin_amdgcn_perm((uint32_t)q[5], (uint32_t)q[4], 0x0c0c0400u);
    const uint32_t p67 = __builtin_amdgcn_perm((uint32_t)q[7], (uint32_t)q[6], 0x0c0c0400u);
    return uint2{__builtin_amdgcn_perm(p23, p01, 0x05040100u), __builtin_amdgcn_perm(p67, p45, 0x05040100u)};
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// max |v| of 8 bf16 as its bit pattern (non-negative bf16 order as unsigned 16-bit integers;
// packed max, two values an instruction)
GQ8_DEV uint32_t absmax8_bf16_bits(u32x4 r) {
    us2 m = {0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, r[e] & 0x7fff7fffu));
    return (uint32_t)(m.x > m.y ? m.x : m.y);
}

GQ8_DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// HALF: two work-groups per 16-column tile, eight columns each (twice the work-groups when the
// tiles are fewer than the CUs): lane l loads the fragment lane of column 8h + l%8, so lanes l
// and l + 8 load the same bytes (one cache-line request) and the MFMA computes each of the
// work-group's eight columns twice.
template <int MT, int KPW, bool HALF = false>
__global__ void __launch_bounds__(1024) w8a8_mfma_kernel(W8Args a) {
    __shared__ int tile[16][32][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int nt = HALF ? (int)blockIdx.x >> 1 : (int)blockIdx.x;
    const int hf = HALF ? (int)blockIdx.x & 1 : 0;
    const int n0 = nt * 16 + 8 * hf;
    v4i b[KPW];
    bool ok[KPW];
    load_frags<KPW>(a, nt, wave, nw, HALF ? ((lane & 48) | (8 * hf + (lane & 7))) : lane, b, ok);
    const W8Scales sc = w8a8_prefetch_scales(a, n0);
    const int mrow = lane & 15;
    v4i x0[KPW], x1[KPW];
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int k = (wave + i * nw) * 64 + 16 * (lane >> 4);
        x0[i] = load_x16(a, mrow, k);
        if (MT == 2) x1[i] = load_x16(a, mrow + 16, k);
    }
    __builtin_amdgcn_sched_barrier(0);
    const v4i z = {0, 0, 0, 0};
    v4i acc0 = z, acc1 = z;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int k = (wave + i * nw) * 64 + 16 * (lane >> 4);
        const bool kin = ok[i] && k < a.K;
        const v4i xa = (kin && mrow < a.M) ? x0[i] : z;
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, ok[i] ? b[i] : z, acc0, 0, 0, 0);
        if (MT == 2) {
            const v4i xb = (kin && mrow + 16 < a.M) ? x1[i] : z;
            acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(xb, ok[i] ? b[i] : z, acc1, 0, 0, 0);
        }
    }
    // D layout: lane l holds column l%16, rows 4*(l/16) + v
    const int col = lane & 15, r0 = 4 * (lane >> 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        tile[wave][r0 + v][col] = acc0[v];
        if (MT == 2) tile[wave][16 + r0 + v][col] = acc1[v];
    }
    w8a8_finish(a, n0, HALF ? 8 : 16, nw, tile, sc);
}

// x is bf16 [M][K], M <= 8, M * K <= 16384 (the variant that quantizes x per token in the
// work-group). Every work-group makes the whole x_q, so the quantization is spread over all its
// threads (thread t takes the 8-value chunks t, t + threads, ... of x in memory order) and the
// bytes are staged in LDS, where the MFMA waves read their A operands. Order: w_scale, x, then
// the weights (loads complete in issue order: the quantization waits only for x and overlaps
// the weight stream); row maxes through LDS atomics (one per wave when a wave's chunks lie in
// one row); x_scale and 127 / amax per row; the quants; then the MFMA and the epilogue of the
// int8 product. Work-group 0 also writes x_q and x_scale out when asked.
constexpr int kBxMaxM = kFusedBf16xM;
constexpr int kBxRow = 16;                   // LDS row padding (bytes): rows start on other banks

template <int KPW, int XC>
__global__ void __launch_bounds__(1024) w8a8_bf16x_kernel(W8Args a) {
    __shared__ __attribute__((aligned(16))) int8_t xl[kFusedBf16xElems + kBxMaxM * kBxRow];
    __shared__ int tile[16][32][16];
    __shared__ uint32_t am_s[kBxMaxM];
    __shared__ float inv_s[kBxMaxM], xs_s[kBxMaxM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nthr = blockDim.x, nw = nthr >> 6, nt = blockIdx.x;
    const int cpr = a.K >> 3, nch = a.M * cpr, ldk = a.K + kBxRow;
    W8Scales sc;
    sc.xs = 0.f;
    sc.ws = a.wsc[imin8(nt * 16 + (tid & 15), a.N - 1)];
    u32x4 r[XC];
    int c[XC];
#pragma unroll
    for (int j = 0; j < XC; ++j) {           // past the end: the last chunk again (same row)
        c[j] = imin8(tid + j * nthr, nch - 1);
        r[j] = *reinterpret_cast<const u32x4*>(a.xb + (size_t)c[j] * 8);
    }
    v4i b[KPW];
    bool ok[KPW];
    load_frags<KPW>(a, nt, wave, nw, lane, b, ok);
    __builtin_amdgcn_sched_barrier(0);       // keep every load issued ahead of the maxes
    if (tid < kBxMaxM) am_s[tid] = 0u;
    __syncthreads();
    int row[XC];
#pragma unroll
    for (int j = 0; j < XC; ++j) {
        row[j] = (int)((uint32_t)c[j] / (uint32_t)cpr);
        uint32_t m = absmax8_bf16_bits(r[j]);
        const int rlo = __builtin_amdgcn_readfirstlane(row[j]);
        if (rlo == __shfl(row[j], 63, 64)) {             // chunks ascend with the lane
            m = wave_max_u32(m);
            if (lane == 0) atomicMax(&am_s[rlo], m);
        } else {
            atomicMax(&am_s[row[j]], m);
        }
    }
    __syncthreads();
    if (tid < a.M) {
        const float f = bf16_bits_to_f32(am_s[tid]);
        xs_s[tid] = f / 127.0f;
        inv_s[tid] = f > 0.f ? 127.0f / f : 0.f;
        if (nt == 0 && a.xs_out != nullptr) a.xs_out[tid] = f / 127.0f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < XC; ++j) {
        const uint2 q = quant8_bf16(r[j], inv_s[row[j]]);
        const int col = (c[j] - row[j] * cpr) * 8;
        *reinterpret_cast<uint2*>(xl + row[j] * ldk + col) = q;
        if (nt == 0 && a.xq_out != nullptr && tid + j * nthr < nch)
            *reinterpret_cast<uint2*>(a.xq_out + (size_t)c[j] * 8) = q;
    }
    __syncthreads();
    const int mrow = lane & 15;
    const v4i z = {0, 0, 0, 0};
    v4i acc = z;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int k = (wave + i * nw) * 64 + 16 * (lane >> 4);
        const bool in = ok[i] && k < a.K && mrow < a.M;
        const v4i xv = *reinterpret_cast<const v4i*>(xl + (in ? mrow * ldk + k : 0));
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(in ? xv : z, ok[i] ? b[i] : z, acc, 0, 0, 0);
    }
    const int col = lane & 15, r0 = 4 * (lane >> 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) tile[wave][r0 + v][col] = acc[v];
    w8a8_finish(a, nt * 16, 16, nw, tile, sc, xs_s);
}

template <int MC, int KPW>
__global__ void __launch_bounds__(1024) w8a8_dot_kernel(W8Args a) {
    __shared__ int tile[16][32][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int nt = blockIdx.x;
    v4i b[KPW];
    bool ok[KPW];
    load_frags<KPW>(a, nt, wave, nw, lane, b, ok);
    const W8Scales sc = w8a8_prefetch_scales(a, nt * 16);
    int acc[MC];
#pragma unroll
    for (int m = 0; m < MC; ++m) acc[m] = 0;
    // x rows are L2-resident; with 16 waves a work-group keeps them per k-step (register budget)
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int k = (wave + i * nw) * 64 + 16 * (lane >> 4);
        v4i xv[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) xv[m] = load_x16(a, m, k);
        if (ok[i] && k < a.K) {
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                int t = acc[m];
                t = __builtin_amdgcn_sdot4(xv[m].x, b[i].x, t, false);
                t = __builtin_amdgcn_sdot4(xv[m].y, b[i].y, t, false);
                t = __builtin_amdgcn_sdot4(xv[m].z, b[i].z, t, false);
                t = __builtin_amdgcn_sdot4(xv[m].w, b[i].w, t, false);
                acc[m] = t;
            }
        }
    }
    // lanes l, l+16, l+32, l+48 hold the four 16-wide k quarters of column l%16
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        int t = acc[m];
        t += (int)lane_xor16((uint32_t)t);
        t += (int)lane_xor32((uint32_t)t);
        if (lane < 16 && m < a.M) tile[wave][m][lane] = t;
    }
    w8a8_finish(a, nt * 16, 16, nw, tile, sc);
}

// ------------------------------------------------------------------------------------ planning

W8Plan plan_w8a8(int M, int N, int K) {
    W8Plan p{};
    const int choice = w8a8_kernel_choice();
    p.mfma = !(choice == 1 && M <= 15);            // MFMA by default, at every M (measured)
    p.ntiles = (N + 15) / 16;
    p.half = p.mfma && M <= 16 && 2 * p.ntiles <= 256;
    p.ksteps = (K + 63) / 64;
    p.nw = p.ksteps < 16 ? p.ksteps : 16;
    p.kpw = (p.ksteps + p.nw - 1) / p.nw;
    return p;
}

template <int KPW>
static int launch_w8a8_kpw(const W8Plan& p, W8Args a, hipStream_t st) {
    const dim3 g(p.ntiles), g2(2 * p.ntiles), b(64 * p.nw);
    if (a.xb != nullptr) {                 // bf16 x quantized in the work-group
        const int nch = a.M * (a.K >> 3), nthr = 64 * p.nw, xc = (nch + nthr - 1) / nthr;
        if (xc <= 1) hipLaunchKernelGGL((w8a8_bf16x_kernel<KPW, 1>), g, b, 0, st, a);
        else if (xc <= 2) hipLaunchKernelGGL((w8a8_bf16x_kernel<KPW, 2>), g, b, 0, st, a);
        else return GQ8_ESHAPE;
    } else if (p.mfma) {
        if (p.half) hipLaunchKernelGGL((w8a8_mfma_kernel<1, KPW, true>), g2, b, 0, st, a);
        else if (a.M <= 16) hipLaunchKernelGGL((w8a8_mfma_kernel<1, KPW>), g, b, 0, st, a);
        else hipLaunchKernelGGL((w8a8_mfma_kernel<2, KPW>), g, b, 0, st, a);
    } else if (a.M <= 1) {
        hipLaunchKernelGGL((w8a8_dot_kernel<1, KPW>), g, b, 0, st, a);
    } else if (a.M <= 2) {
        hipLaunchKernelGGL((w8a8_dot_kernel<2, KPW>), g, b, 0, st, a);
    } else if (a.M <= 4) {
        hipLaunchKernelGGL((w8a8_dot_kernel<4, KPW>), g, b, 0, st, a);
    } else if (a.M <= 8) {
        hipLaunchKernelGGL((w8a8_dot_kernel<8, KPW>), g, b, 0, st, a);
    } else {
        hipLaunchKernelGGL((w8a8_dot_kernel<15, KPW>), g, b, 0, st, a);
    }
    return launch_status();
}

int launch_w8a8(const W8Plan& p, const int8_t* xq, const float* xs, const int8_t* wp,
                const float* ws_scale, void* out, bool i32_out, int M, int N, int K, hipStream_t st,
                const uint16_t* xb, int8_t* xq_out, float* xs_out) {
    if (xb != nullptr && !bf16x_fused(M, K)) return GQ8_ESHAPE;
    if (xb != nullptr && i32_out) return GQ8_EINVAL;
    W8Args a{};
    a.xq = xq; a.xs = xs; a.wp = wp; a.wsc = ws_scale; a.out = out; a.i32_out = i32_out ? 1 : 0;
    a.xb = xb; a.xq_out = xq_out; a.xs_out = xs_out;
    a.M = M; a.N = N; a.K = K; a.ksteps = p.ksteps;
    switch (p.kpw) {
        case 1: return launch_w8a8_kpw<1>(p, a, st);
        case 2: return launch_w8a8_kpw<2>(p, a, st);
        case 3: return launch_w8a8_kpw<3>(p, a, st);
        case 4: return launch_w8a8_kpw<4>(p, a, st);
        // K > 4096: one variant per step count, since every wave issues KPW loads of each kind
        // (clamped past the last step), so a larger KPW than needed multiplies the loads
        case 5: return launch_w8a8_kpw<5>(p, a, st);
        case 6: return launch_w8a8_kpw<6>(p, a, st);
        case 7: return launch_w8a8_kpw<7>(p, a, st);
        case 8: return launch_w8a8_kpw<8>(p, a, st);
        default: return GQ8_ESHAPE;
    }
}

// ------------------------------------------------------------------------- per-token quantize

// One work-group per row: amax over the row (lane maxes, wave max, then the four waves), then
// the quants of each 8-value chunk with quant8_bf16 (the arithmetic of the W8A8 kernel that
// quantizes x itself, so the bytes agree).
__global__ void __launch_bounds__(256) per_token_quantize_kernel(const uint16_t* __restrict__ x, int K,
                                                                 int8_t* __restrict__ xq,
                                                                 float* __restrict__ xs) {
    __shared__ uint32_t wmax[4];
    const int m = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint16_t* row = x + (size_t)m * K;
    uint32_t ab = 0u;
    for (int k = 8 * (int)threadIdx.x; k < K; k += 8 * 256)
        ab = umax32(ab, absmax8_bf16_bits(*reinterpret_cast<const u32x4*>(row + k)));
    ab = wave_max_u32(ab);
    if (lane == 0) wmax[wave] = ab;
    __syncthreads();
    const float am = bf16_bits_to_f32(umax32(umax32(wmax[0], wmax[1]), umax32(wmax[2], wmax[3])));
    const float inv = am > 0.f ? 127.0f / am : 0.f;
    if (threadIdx.x == 0) xs[m] = am / 127.0f;
    for (int k = 8 * (int)threadIdx.x; k < K; k += 8 * 256)
        *reinterpret_cast<uint2*>(xq + (size_t)m * K + k) =
            quant8_bf16(*reinterpret_cast<const u32x4*>(row + k), inv);
}

int launch_per_token_quantize(const uint16_t* x, int M, int K, int8_t* xq, float* xs, hipStream_t st) {
    hipLaunchKernelGGL(per_token_quantize_kernel, dim3(M), dim3(256), 0, st, x, K, xq, xs);
    return launch_status();
}

}  // namespace gq8
