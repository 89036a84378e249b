// Q8_0 reads (HC-Q8 page, "What changed"): the Q8_0 matrix-vector product with fp32 x, the fused
// RMSNorm + Q8_0 hyper-connection down read and the Q8_0 up read.
//
// Every weight byte is read once from HBM with 16-byte non-temporal loads. Each wave issues all
// of its loads (clamped to valid addresses, never behind a branch) before its first arithmetic,
// so a wave costs one memory latency, not one per load; a kernel launch costs more than most of
// these reads, so each operation is one kernel where the shape allows it.
//
//  * GEMV (fp32 x): a work-group owns RW rows and all of K; wave w reads 1024-column chunks
//    w, w+NW, ... (one 1 KiB contiguous load per row per chunk); lane partials are reduced over
//    the wave (DPP) and the waves' sums are added through LDS in wave order. No split-K.
//  * down read: 32 rows x 32 columns (one Q8_0 block) per bf16 MFMA pair. u = R * w_norm is
//    exact in fp32 (8-bit x 8-bit significands) and is split exactly into bf16 hi + lo, so the
//    MFMA products are exact. A work-group holds up to 16 row tiles and one 128-column slab and
//    stages u (and the slab's sums of R^2) in LDS once for all of them. The partial sums of the
//    K slabs go to the workspace; a second kernel adds them in ascending slab order, applies
//    rs = 1/sqrt(mean R^2 + eps) and rounds to bf16.
//  * up read: lo is bf16, exact as an MFMA operand; one wave owns 32 rows and all of K.
#include "gq8_device.h"
#include "gq8_internal.h"

namespace gq8 {

GQ8_DEV void load16_f32(const float* p, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 f = *reinterpret_cast<const float4*>(p + 4 * i);
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
}

GQ8_DEV int imin(int a, int b) { return a < b ? a : b; }

// ------------------------------------------------------------------------------ GEMV, fp32 x

// MAXW: most waves per work-group (4 when K <= 4096, else 16); it sets the register budget.
template <int T, int RW, int MAXW>
__global__ void __launch_bounds__(64 * MAXW) gemv_rows_kernel(GemvArgs a) {
    constexpr int TG = MAXW <= 4 ? (T <= 8 ? T : 8) : (T <= 2 ? T : 2);   // x rows in registers
    __shared__ float red[16][RW * T];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int NW = blockDim.x >> 6;
    const int N = a.N, K = a.K, nblk = K >> 5;
    const int row0 = blockIdx.x * RW;
    const int nchunk = (K + 1023) >> 10;
    const float* x = reinterpret_cast<const float*>(a.x);

    float acc[RW][T];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[r][t] = 0.f;

    for (int c = wave; c < nchunk; c += NW) {
        const int k = c * 1024 + lane * 16;
        const bool kok = k < K;                             // K % 32 == 0: k + 16 <= K
        const int kc = kok ? k : K - 16;
        u32x4 wq[RW];
        uint16_t wd[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int row = imin(row0 + r, N - 1);
            wq[r] = ld_nt16(a.q + (size_t)row * K + kc);
            wd[r] = a.d[(size_t)row * nblk + (kc >> 5)];
        }
#pragma unroll
        for (int t0 = 0; t0 < T; t0 += TG) {
            // rows t0 + t >= T exist only when TG does not divide T: those are skipped at
            // compile time (no load, no accumulator)
            float xv[TG][16];
#pragma unroll
            for (int t = 0; t < TG; ++t)
                if (t0 + t < T) load16_f32(x + (size_t)(t0 + t) * K + kc, xv[t]);
            __builtin_amdgcn_sched_barrier(0);
            if (!kok) {
#pragma unroll
                for (int t = 0; t < TG; ++t)
#pragma unroll
                    for (int i = 0; i < 16; ++i) xv[t][i] = 0.f;
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const float dsc = kok ? h2f(wd[r]) : 0.f;
#pragma unroll
                for (int t = 0; t < TG; ++t)
                    if (t0 + t < T)
                        acc[r][t0 + t] = fmaf(dot16_i8_f32(wq[r], xv[t]), dsc, acc[r][t0 + t]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float v = wave_sum(acc[r][t]);
            if (lane == 0) red[wave][r * T + t] = v;
        }
    __syncthreads();
    for (int i = threadIdx.x; i < RW * T; i += blockDim.x) {
        const int t = i / RW, r = i - t * RW;
        const int row = row0 + r;
        if (row >= N) continue;
        float v = 0.f;
        for (int w = 0; w < NW; ++w) v += red[w][r * T + t];
        reinterpret_cast<float*>(a.out)[(size_t)t * N + row] = v;
    }
}

template <int T> constexpr int gemv_rw() { return T <= 2 ? 8 : (T <= 4 ? 4 : (T <= 8 ? 2 : 1)); }

template <int T>
static int launch_gemv_t(GemvArgs a, hipStream_t st) {
    constexpr int RW = gemv_rw<T>();
    int nw = (a.K + 1023) / 1024;
    if (nw <= 4) {
        hipLaunchKernelGGL((gemv_rows_kernel<T, RW, 4>), dim3((a.N + RW - 1) / RW), dim3(64 * nw), 0, st, a);
    } else {
        nw = nw > 16 ? 16 : nw;
        constexpr int RW16 = RW < 2 ? RW : 2;
        hipLaunchKernelGGL((gemv_rows_kernel<T, RW16, 16>), dim3((a.N + RW16 - 1) / RW16), dim3(64 * nw), 0, st, a);
    }
    return launch_status();
}

#define GQ8_T_SWITCH(FN, ...)                                                                    \
    switch (a.T) {                                                                                \
        case 1: return FN<1>(__VA_ARGS__);   case 2: return FN<2>(__VA_ARGS__);                   \
        case 3: return FN<3>(__VA_ARGS__);   case 4: return FN<4>(__VA_ARGS__);                   \
        case 5: return FN<5>(__VA_ARGS__);   case 6: return FN<6>(__VA_ARGS__);                   \
        case 7: return FN<7>(__VA_ARGS__);   case 8: return FN<8>(__VA_ARGS__);                   \
        case 9: return FN<9>(__VA_ARGS__);   case 10: return FN<10>(__VA_ARGS__);                 \
        case 11: return FN<11>(__VA_ARGS__); case 12: return FN<12>(__VA_ARGS__);                 \
        case 13: return FN<13>(__VA_ARGS__); case 14: return FN<14>(__VA_ARGS__);                 \
        case 15: return FN<15>(__VA_ARGS__); case 16: return FN<16>(__VA_ARGS__);                 \
        default: return GQ8_ESHAPE;                                                               \
    }

int launch_q8_0_gemv(GemvArgs a, hipStream_t st) { GQ8_T_SWITCH(launch_gemv_t, a, st) }

// ------------------------------------------------------------------------------ down read

constexpr int kDnNB = kDownSlab / 32;     // Q8_0 blocks per slab

template <int T> constexpr int vmax_for() { return T <= 8 ? 4 : (T <= 16 ? 8 : 16); }

// One work-group: slab blockIdx.x (128 columns) x up to 16 row tiles of 32 (one per wave).
template <int T>
__global__ void __launch_bounds__(1024) hc_down_partial_kernel(GemvArgs a) {
    constexpr int VMAX = vmax_for<T>();
    __shared__ u32x4 ua[2][kDnNB][2][64];           // u hi / lo pieces in MFMA A layout
    __shared__ float sq[kDnNB][2][2][32];           // sum of R^2 of each staged 8-column piece
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int N = a.N, K = a.K, nblk = K >> 5;
    const int s = blockIdx.x;
    const int k0 = s * kDownSlab;
    const int rt = blockIdx.y * 16 + wave;
    const int g = lane >> 5;
    const int n = rt * 32 + (lane & 31);
    const int nc = imin(n, N - 1);
    const uint16_t* R = reinterpret_cast<const uint16_t*>(a.x);

    // 1. weight quants and scales of this wave's 32 rows x 4 blocks (clamped, masked later)
    u32x4 wq[kDnNB];
    uint16_t wd[kDnNB];
#pragma unroll
    for (int b = 0; b < kDnNB; ++b) {
        const int kb = imin(k0 + 32 * b, K - 32);
        wq[b] = ld_nt16(a.q + (size_t)nc * K + kb + 16 * g);
        wd[b] = a.d[(size_t)nc * nblk + (kb >> 5)];
    }

    // 2. stage u = R * w_norm for the slab as exact bf16 hi + lo, and R^2 sums
    for (int it = threadIdx.x; it < kDnNB * 2 * 64; it += blockDim.x) {
        const int b = it >> 7, m = (it >> 6) & 1, l = it & 63;
        const int t = l & 31, gg = l >> 5;
        const int k = k0 + 32 * b + 16 * gg + 8 * m;
        const bool ok = t < a.T && k < K;
        const int kc = ok ? k : 0, tc = ok ? t : 0;
        const uint4 rv = *reinterpret_cast<const uint4*>(R + (size_t)tc * K + kc);
        const uint4 wv = *reinterpret_cast<const uint4*>(a.wnorm + kc);
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
        uint32_t hi[4], lo[4];
        float r2 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float r0 = __uint_as_float(rw[i] << 16), r1 = __uint_as_float(rw[i] & 0xffff0000u);
            const float w0 = __uint_as_float(ww[i] << 16), w1 = __uint_as_float(ww[i] & 0xffff0000u);
            const float u0 = ok ? r0 * w0 : 0.f, u1 = ok ? r1 * w1 : 0.f;   // exact products
            const uint16_t h0 = f2bf_bits(u0), h1 = f2bf_bits(u1);
            const float l0 = u0 - bf2f(h0), l1 = u1 - bf2f(h1);             // exact residuals
            hi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lo[i] = pack_bf16_trunc(l0, l1);                                // exact in bf16
            r2 = fmaf(r0, r0, r2);
            r2 = fmaf(r1, r1, r2);
        }
        ua[0][b][m][l] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        ua[1][b][m][l] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        sq[b][m][gg][t] = ok ? r2 : 0.f;
    }
    __syncthreads();

    // 3. per block: four exact-product MFMAs, then the block scale
    f32x16 acc = {};
#pragma unroll
    for (int b = 0; b < kDnNB; ++b) {
        const bool bok = k0 + 32 * b < K;
        const float dsc = bok ? h2f(wd[b]) : 0.f;
        const bf16x8 b0 = i8x8_to_bf16x8(wq[b].x, wq[b].y);
        const bf16x8 b1 = i8x8_to_bf16x8(wq[b].z, wq[b].w);
        f32x16 D = {};
        D = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, ua[0][b][0][lane]), b0, D);
        D = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, ua[1][b][0][lane]), b0, D);
        D = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, ua[0][b][1][lane]), b1, D);
        D = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, ua[1][b][1][lane]), b1, D);
#pragma unroll
        for (int v = 0; v < VMAX; ++v) acc[v] = fmaf(dsc, D[v], acc[v]);
    }

    // 4. partial sums of this slab: part[s][t][n], and the slab's sum of R^2 per row t
#pragma unroll
    for (int v = 0; v < VMAX; ++v) {
        const int t = mfma32_row(v, lane);
        if (t < a.T && n < N) a.part[((size_t)s * a.T + t) * N + n] = acc[v];
    }
    if (blockIdx.y == 0 && threadIdx.x < a.T) {
        const int t = threadIdx.x;
        float v = 0.f;
        for (int b = 0; b < kDnNB; ++b)
            for (int m = 0; m < 2; ++m)
                for (int gg = 0; gg < 2; ++gg) v += sq[b][m][gg][t];
        a.ssq[(size_t)s * a.T + t] = v;
    }
}

// lo[t][n] = bf16(rs[t] * sum_s part[s][t][n]); one work-group per (32 rows, t). The S slab sums
// are added in ascending order within each of 8 contiguous slab groups, then the groups in order.
__global__ void __launch_bounds__(256) hc_down_combine_kernel(GemvArgs a) {
    __shared__ float red[8][32];
    __shared__ float s_rs;
    const int t = blockIdx.y;
    const int sg = threadIdx.x >> 5, nl = threadIdx.x & 31;
    const int n = blockIdx.x * 32 + nl;
    const int S = a.S, N = a.N;
    const int per = (S + 7) / 8;
    const int s0 = sg * per, s1 = imin(S, s0 + per);
    if (threadIdx.x < 64) {            // rs[t]: lane-strided sums, then the wave sum
        float ss = 0.f;
        for (int s = threadIdx.x; s < S; s += 64) ss += a.ssq[(size_t)s * a.T + t];
        ss = wave_sum(ss);
        if (threadIdx.x == 0) {
            const float rs = 1.0f / sqrtf(ss / (float)a.K + a.eps);
            s_rs = rs;
            if (blockIdx.x == 0 && a.rs_out != nullptr) a.rs_out[t] = rs;
        }
    }
    float v = 0.f;
    if (n < N) {
        for (int s = s0; s < s1; s += 16) {
            float p[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                p[i] = s + i < s1 ? a.part[((size_t)(s + i) * a.T + t) * N + n] : 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) v += p[i];
        }
    }
    red[sg][nl] = v;
    __syncthreads();
    if (threadIdx.x < 32 && n < N && a.out != nullptr) {
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) tot += red[i][nl];
        reinterpret_cast<uint16_t*>(a.out)[(size_t)t * N + n] = f2bf_bits(s_rs * tot);
    }
}

size_t hc_down_workspace_bytes(int T, int N, int K) {
    const size_t S = hc_down_slabs(K);
    return round_up(S * T * N * sizeof(float), kCounterAlign) +
           round_up(S * T * sizeof(float), kCounterAlign);
}

template <int T>
static int launch_down_t(GemvArgs a, void* ws, hipStream_t st) {
    const int S = hc_down_slabs(a.K);
    const int ntile = (a.N + 31) / 32;
    char* w = static_cast<char*>(ws);
    a.S = S;
    a.part = reinterpret_cast<float*>(w);
    a.ssq = reinterpret_cast<float*>(w + round_up((size_t)S * T * a.N * sizeof(float), kCounterAlign));
    const int waves = ntile < 16 ? ntile : 16;
    hipLaunchKernelGGL((hc_down_partial_kernel<T>), dim3(S, (ntile + 15) / 16), dim3(64 * waves), 0, st, a);
    int rc = launch_status();
    if (rc != GQ8_OK) return rc;
    hipLaunchKernelGGL(hc_down_combine_kernel, dim3(ntile, T), dim3(256), 0, st, a);
    return launch_status();
}

int launch_hc_down(GemvArgs a, void* ws, hipStream_t st) { GQ8_T_SWITCH(launch_down_t, a, ws, st) }

// ------------------------------------------------------------------------------ up read

constexpr int kUpCB = 10;                 // Q8_0 blocks per register batch (K = 320 in one)

template <int T>
__global__ void __launch_bounds__(256) hc_up_kernel(GemvArgs a) {
    constexpr int VMAX = vmax_for<T>();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int N = a.N, K = a.K, nblk = K >> 5;
    const int rt = blockIdx.x * 4 + wave;
    const int g = lane >> 5, t = lane & 31;
    const int n = rt * 32 + t;
    const int nc = imin(n, N - 1);
    const int tc = t < T ? t : 0;
    const uint16_t* lo = reinterpret_cast<const uint16_t*>(a.x);

    f32x16 acc = {};
    for (int cb = 0; cb < nblk; cb += kUpCB) {
        u32x4 wq[kUpCB];
        uint16_t wd[kUpCB];
        u32x4 xa[kUpCB][2];
#pragma unroll
        for (int b = 0; b < kUpCB; ++b) {
            const int bb = imin(cb + b, nblk - 1);
            wq[b] = ld_nt16(a.q + (size_t)nc * K + 32 * bb + 16 * g);
            wd[b] = a.d[(size_t)nc * nblk + bb];
#pragma unroll
            for (int m = 0; m < 2; ++m)
                xa[b][m] = *reinterpret_cast<const u32x4*>(lo + (size_t)tc * K + 32 * bb + 16 * g + 8 * m);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < kUpCB; ++b) {
            if (cb + b < nblk) {
                const float dsc = h2f(wd[b]);
                const u32x4 z = {0u, 0u, 0u, 0u};
                const bf16x8 a0 = __builtin_bit_cast(bf16x8, t < T ? xa[b][0] : z);
                const bf16x8 a1 = __builtin_bit_cast(bf16x8, t < T ? xa[b][1] : z);
                f32x16 D = {};
                D = mfma_bf16_32x32x16(a0, i8x8_to_bf16x8(wq[b].x, wq[b].y), D);
                D = mfma_bf16_32x32x16(a1, i8x8_to_bf16x8(wq[b].z, wq[b].w), D);
#pragma unroll
                for (int v = 0; v < VMAX; ++v) acc[v] = fmaf(dsc, D[v], acc[v]);
            }
        }
    }
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
    for (int v = 0; v < VMAX; ++v) {
        const int tt = mfma32_row(v, lane);
        if (tt < T && n < N) out[(size_t)tt * N + n] = f2bf_bits(acc[v]);
    }
}

template <int T>
static int launch_up_t(GemvArgs a, hipStream_t st) {
    const int ntile = (a.N + 31) / 32;
    hipLaunchKernelGGL((hc_up_kernel<T>), dim3((ntile + 3) / 4), dim3(256), 0, st, a);
    return launch_status();
}

int launch_hc_up(GemvArgs a, hipStream_t st) { GQ8_T_SWITCH(launch_up_t, a, st) }

}  // namespace gq8
