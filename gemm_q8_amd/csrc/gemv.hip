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

template <int T> constexpr int gemv_rw() { return T <= 4 ? 2 : 1; }

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
constexpr int kDnStride = kDownSlab + 16; // padded LDS row stride of a wave's weight tile (bytes)

// One work-group: slab blockIdx.x (128 columns) x up to 16 waves of 32 rows (two 16-row MFMA
// tiles each). Each wave reads its 32 x 128-byte weight tile with four coalesced 1 KiB loads
// (eight 128-byte row segments per load) into LDS and takes the MFMA operands from there.
template <int T>
__global__ void __launch_bounds__(1024) hc_down_partial_kernel(GemvArgs a) {
    __shared__ u32x4 ua[2][kDnNB][64];                            // u hi / lo, 16x16x32 A layout
    __shared__ float sq[kDnNB][4][16];                            // sums of R^2 per 8-column piece
    __shared__ __attribute__((aligned(16))) uint8_t wt[16][32 * kDnStride];   // weight tiles
    __shared__ uint16_t ws[16][32][kDnNB];                        // their block scales
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int N = a.N, K = a.K, nblk = K >> 5;
    const int s = blockIdx.x;
    const int k0 = s * kDownSlab;
    const int r0 = (blockIdx.y * 16 + wave) * 32;                 // first row of this wave
    const uint16_t* R = reinterpret_cast<const uint16_t*>(a.x);

    // 1. coalesced weight loads: load i covers rows 8i..8i+7 of the tile, 16 bytes per lane
    u32x4 wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = imin(r0 + 8 * i + (lane >> 3), N - 1);
        const int kb = imin(k0 + 16 * (lane & 7), K - 16);
        wv[i] = ld_nt16(a.q + (size_t)row * K + kb);
    }
    uint16_t sc[kDnNB];
    {
        const int row = imin(r0 + (lane & 31), N - 1);
#pragma unroll
        for (int b = 0; b < kDnNB; ++b) sc[b] = a.d[(size_t)row * nblk + imin((k0 >> 5) + b, nblk - 1)];
    }

    // 2. stage u = R * w_norm for the slab as exact bf16 hi + lo (A operand: lane l holds row
    //    t = l % 16, columns 32b + 8(l/16) .. +8), and the R^2 sums
    for (int it = threadIdx.x; it < kDnNB * 64; it += blockDim.x) {
        const int b = it >> 6, l = it & 63;
        const int t = l & 15, gg = l >> 4;
        const int k = k0 + 32 * b + 8 * gg;
        const bool ok = t < T && k < K;
        const int kc = ok ? k : 0, tc = ok ? t : 0;
        const uint4 rv = *reinterpret_cast<const uint4*>(R + (size_t)tc * K + kc);
        const uint4 nv = *reinterpret_cast<const uint4*>(a.wnorm + kc);
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w}, ww[4] = {nv.x, nv.y, nv.z, nv.w};
        uint32_t hi[4], lo[4];
        float r2 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float q0 = __uint_as_float(rw[i] << 16), q1 = __uint_as_float(rw[i] & 0xffff0000u);
            const float w0 = __uint_as_float(ww[i] << 16), w1 = __uint_as_float(ww[i] & 0xffff0000u);
            const float u0 = ok ? q0 * w0 : 0.f, u1 = ok ? q1 * w1 : 0.f;   // exact products
            const uint16_t h0 = f2bf_bits(u0), h1 = f2bf_bits(u1);
            const float l0 = u0 - bf2f(h0), l1 = u1 - bf2f(h1);             // exact residuals
            hi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lo[i] = pack_bf16_trunc(l0, l1);                                // exact in bf16
            r2 = fmaf(q0, q0, r2);
            r2 = fmaf(q1, q1, r2);
        }
        ua[0][b][l] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        ua[1][b][l] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        sq[b][gg][t] = ok ? r2 : 0.f;
    }
    // 3. the wave's weight tile and scales into LDS
    uint8_t* tile = wt[wave];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(tile + (8 * i + (lane >> 3)) * kDnStride + 16 * (lane & 7)) = wv[i];
    if (lane < 32) {
#pragma unroll
        for (int b = 0; b < kDnNB; ++b) ws[wave][lane][b] = sc[b];
    }
    __syncthreads();

    // 4. per block and 16-row half: two exact-product MFMAs (hi, lo), then the block scale
    const int j = lane & 15, g = lane >> 4;
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int b = 0; b < kDnNB; ++b) {
        const bool bok = k0 + 32 * b < K;
        const bf16x8 ahi = __builtin_bit_cast(bf16x8, ua[0][b][lane]);
        const bf16x8 alo = __builtin_bit_cast(bf16x8, ua[1][b][lane]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 16 * h + j;
            const uint2 q = *reinterpret_cast<const uint2*>(tile + row * kDnStride + 32 * b + 8 * g);
            const bf16x8 w = i8x8_to_bf16x8(q.x, q.y);
            f32x4 D = {0.f, 0.f, 0.f, 0.f};
            D = mfma_bf16_16x16x32(ahi, w, D);
            D = mfma_bf16_16x16x32(alo, w, D);
            const float dsc = bok ? h2f(ws[wave][row][b]) : 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[h][v] = fmaf(dsc, D[v], acc[h][v]);
        }
    }

    // 5. partial sums of this slab: part[s][t][n], and the slab's sum of R^2 per row t
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int n = r0 + 16 * h + j;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = 4 * g + v;
            if (t < T && n < N) a.part[((size_t)s * T + t) * N + n] = acc[h][v];
        }
    }
    if (blockIdx.y == 0 && threadIdx.x < T) {
        const int t = threadIdx.x;
        float v = 0.f;
        for (int b = 0; b < kDnNB; ++b)
            for (int gg = 0; gg < 4; ++gg) v += sq[b][gg][t];
        a.ssq[(size_t)s * T + t] = v;
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

constexpr int kUpCW = 320;                  // columns per chunk (the K = 320 read is one chunk)
constexpr int kUpCB = kUpCW / 32;           // Q8_0 blocks per chunk
constexpr int kUpStride = kUpCW + 16;       // padded LDS row stride of a weight tile (bytes)
constexpr int kUpLoStride = 2 * kUpCW + 16; // padded LDS row stride of the bf16 input (bytes)
constexpr int kUpLoads = 16 * kUpCW / 1024; // coalesced 1 KiB loads per 16-row tile chunk

// One wave per 16 output rows (one 16x16x32 MFMA per Q8_0 block); a work-group of 4 waves
// shares the staged input chunk. A wave's 16 rows x 320 bytes are one contiguous 5 KiB range:
// five coalesced 1 KiB loads into LDS, then MFMA operands (row = lane % 16) out of LDS.
// FULL: every chunk is 320 columns wide (K % 320 == 0), so every load, LDS access and MFMA of a
// chunk is unconditional and the three phases (LDS reads, MFMAs, scale FMAs) issue back to back.
template <int T, bool FULL>
__global__ void __launch_bounds__(256) hc_up_kernel(GemvArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t wt[4][16 * kUpStride];
    __shared__ uint16_t wsc[4][16][kUpCB];
    __shared__ __attribute__((aligned(16))) uint8_t xl[kMaxT][kUpLoStride];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int N = a.N, K = a.K, nblk = K >> 5;
    const int r0 = (blockIdx.x * 4 + wave) * 16;
    const int j = lane & 15, g = lane >> 4;
    const uint16_t* lo = reinterpret_cast<const uint16_t*>(a.x);
    const u32x4 z = {0u, 0u, 0u, 0u};

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < K; c0 += kUpCW) {
        const int cw = FULL ? kUpCW : (K - c0 < kUpCW ? K - c0 : kUpCW);   // multiple of 32
        const int np = cw >> 4;                             // 16-byte pieces per weight row
        const int cb = cw >> 5;
        const int npx = cw >> 3;                            // 16-byte pieces per input row
        // weights: piece e = i*64 + lane of the tile -> (row e/np, piece e%np)
        u32x4 wv[kUpLoads];
#pragma unroll
        for (int i = 0; i < kUpLoads; ++i) {
            const int e = imin(i * 64 + lane, 16 * np - 1);
            const int row = e / np, pc = e - row * np;
            wv[i] = ld_nt16(a.q + (size_t)imin(r0 + row, N - 1) * K + c0 + 16 * pc);
        }
        uint16_t sv[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int e = imin(i * 64 + lane, 16 * cb - 1);
            const int row = e / cb, b = e - row * cb;
            sv[i] = a.d[(size_t)imin(r0 + row, N - 1) * nblk + (c0 >> 5) + b];
        }
        // the input chunk, shared by the work-group: T rows x npx pieces of 8 bf16
        u32x4 xv[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int e = imin(i * 256 + (int)threadIdx.x, T * npx - 1);
            const int t = e / npx, pc = e - t * npx;
            xv[i] = *reinterpret_cast<const u32x4*>(lo + (size_t)t * K + c0 + 8 * pc);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kUpLoads; ++i) {
            const int e = i * 64 + lane;
            if (FULL || e < 16 * np) {
                const int row = e / np, pc = e - row * np;
                *reinterpret_cast<u32x4*>(&wt[wave][row * kUpStride + 16 * pc]) = wv[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int e = i * 64 + lane;
            if (e < 16 * cb) wsc[wave][e / cb][e % cb] = sv[i];
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int e = i * 256 + (int)threadIdx.x;
            if (e < T * npx) {
                const int t = e / npx, pc = e - t * npx;
                *reinterpret_cast<u32x4*>(&xl[t][16 * pc]) = xv[i];
            }
        }
        __syncthreads();
        const int tj = j < T ? j : 0;
        if (FULL) {
            uint2 q[kUpCB];
            u32x4 x[kUpCB];
            uint16_t sc[kUpCB];
#pragma unroll
            for (int b = 0; b < kUpCB; ++b) {
                q[b] = *reinterpret_cast<const uint2*>(&wt[wave][j * kUpStride + 32 * b + 8 * g]);
                x[b] = *reinterpret_cast<const u32x4*>(&xl[tj][2 * (32 * b + 8 * g)]);
                sc[b] = wsc[wave][j][b];
            }
            f32x4 D[kUpCB];
#pragma unroll
            for (int b = 0; b < kUpCB; ++b) {
                const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
                D[b] = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, j < T ? x[b] : z),
                                          i8x8_to_bf16x8(q[b].x, q[b].y), zf);
            }
#pragma unroll
            for (int b = 0; b < kUpCB; ++b) {
                const float dsc = h2f(sc[b]);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(dsc, D[b][v], acc[v]);
            }
        } else {
#pragma unroll
            for (int b = 0; b < kUpCB; ++b) {
                if (b < cb) {
                    const uint2 q = *reinterpret_cast<const uint2*>(&wt[wave][j * kUpStride + 32 * b + 8 * g]);
                    const u32x4 x = *reinterpret_cast<const u32x4*>(&xl[tj][2 * (32 * b + 8 * g)]);
                    f32x4 D = {0.f, 0.f, 0.f, 0.f};
                    D = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, j < T ? x : z), i8x8_to_bf16x8(q.x, q.y), D);
                    const float dsc = h2f(wsc[wave][j][b]);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] = fmaf(dsc, D[v], acc[v]);
                }
            }
        }
        if (c0 + kUpCW < K) __syncthreads();                // the next chunk overwrites LDS
    }
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    const int n = r0 + j;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int t = 4 * g + v;
        if (t < T && n < N) out[(size_t)t * N + n] = f2bf_bits(acc[v]);
    }
}

template <int T>
static int launch_up_t(GemvArgs a, hipStream_t st) {
    const int ntile = (a.N + 15) / 16;
    if (a.K % kUpCW == 0)
        hipLaunchKernelGGL((hc_up_kernel<T, true>), dim3((ntile + 3) / 4), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((hc_up_kernel<T, false>), dim3((ntile + 3) / 4), dim3(256), 0, st, a);
    return launch_status();
}

int launch_hc_up(GemvArgs a, hipStream_t st) { GQ8_T_SWITCH(launch_up_t, a, st) }

}  // namespace gq8
