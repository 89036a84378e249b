// Q8_0 reads (HC-Q8 page, "What changed"): the Q8_0 matrix-vector product with fp32 x, the fused
// RMSNorm + Q8_0 hyper-connection down read, the Q8_0 up read, the two as one call, and the same
// pair on BF16 weights (the comparison read the Q8_0 read replaces).
//
// Every weight byte is read once from HBM with 16-byte non-temporal loads. Each wave issues its
// loads (clamped to valid addresses, never behind a branch) before its first arithmetic, in the
// order the work consumes them (a wave's loads complete in issue order), so a wave costs about
// one memory latency; a kernel launch costs more than most of these reads, so each operation is
// one or two kernels.
//
//  * GEMV, T <= 3 and K <= 4096 (gemv_wave_kernel): one wave owns one or two whole rows, lane
//    partials over its chunks, one wave sum, no LDS.
//    Other T <= 4 (gemv_rows_kernel): a work-group owns RW rows and all of K; wave w reads
//    1024-column chunks w, w+NW, ...; lane partials are reduced over the wave (DPP) and the
//    waves' sums are added through LDS in wave order. T >= 5: the down read's slab kernel on
//    256-column slabs with x split into bf16 hi + lo as the MFMA A operand, then the combine
//    kernel without rs.
//  * down read at T = 1 (hc_down_rows_kernel): a work-group owns two whole rows and all of K,
//    VALU dots on u = R * w_norm formed in fp32, its own sum of squares for rs: one kernel, no
//    partial sums; the pair then takes the direct up kernel (two launches), and its launch of
//    the down read carries extra work-groups that fetch the up read's weights ahead.
//  * down read, T >= 2 (hc_down_partial_kernel): a work-group takes a 512-column slab x 64 rows, one
//    16-row 16x16x32 bf16 MFMA tile per wave (from T = 9 two waves per tile, one per column
//    half). u = R * w_norm is exact in fp32 (8-bit x 8-bit
//    significands) and splits exactly into bf16 hi + lo, so the MFMA products are exact; it is
//    staged once per work-group in LDS. The wave's weight tile goes through an LDS transpose in
//    four column quarters. The slab partial sums and sums of R^2 go to the workspace, and a
//    combine (hc_down_combine_kernel, or inside the up kernel for small T) adds them in a fixed
//    order, applies rs = 1/sqrt(mean R^2 + eps) and rounds to bf16.
//  * up read (hc_up_direct_kernel): one wave per 16 output rows over K = 320 columns; the weight
//    loads become MFMA operands directly through v_permlane32_swap (no LDS). hc_pair_up_kernel
//    adds the down read's combine in four extra waves of the same work-group.
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
        // all x rows in registers (TG == T): x first, then the weight rows in order, so that
        // row r's dots wait only for loads up to row r (a wave's loads complete in issue order)
        float xv[TG][16];
        if (TG == T) {
#pragma unroll
            for (int t = 0; t < TG; ++t) load16_f32(x + (size_t)t * K + kc, xv[t]);
        }
        u32x4 wq[RW];
        uint16_t wd[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int row = imin(row0 + r, N - 1);
            wd[r] = a.d[(size_t)row * nblk + (kc >> 5)];
            wq[r] = ld_nt16(a.q + (size_t)row * K + kc);
        }
#pragma unroll
        for (int t0 = 0; t0 < T; t0 += TG) {
            // rows t0 + t >= T exist only when TG does not divide T: those are skipped at
            // compile time (no load, no accumulator)
            if (TG != T) {
#pragma unroll
                for (int t = 0; t < TG; ++t)
                    if (t0 + t < T) load16_f32(x + (size_t)(t0 + t) * K + kc, xv[t]);
            }
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

// T <= 3, K <= 4096: one wave per work-group owns RW whole rows. Lane l takes columns
// 1024c + 16l of every chunk c: x for all of K and the RW rows' weights are loaded up front (x
// first), each lane sums its chunks in order, and one wave sum per (row, token) ends the work:
// no LDS, no barrier (a cross-wave sum through LDS and a barrier cost more than the extra x
// reads of wave-owned rows here).
template <int T, int RW, int NCH>
__global__ void __launch_bounds__(64) gemv_wave_kernel(GemvArgs a) {
    const int lane = threadIdx.x;
    const int N = a.N, K = a.K, nblk = K >> 5;
    const int row0 = blockIdx.x * RW;
    const float* x = reinterpret_cast<const float*>(a.x);
    float xv[T][NCH][16];
    int kc[NCH];
    bool kok[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int k = c * 1024 + lane * 16;
        kok[c] = k < K;                                   // K % 32 == 0: k + 16 <= K
        kc[c] = kok[c] ? k : K - 16;
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int c = 0; c < NCH; ++c) load16_f32(x + (size_t)t * K + kc[c], xv[t][c]);
    u32x4 wq[RW][NCH];
    uint16_t wd[RW][NCH];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int row = imin(row0 + r, N - 1);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            wd[r][c] = a.d[(size_t)row * nblk + (kc[c] >> 5)];
            wq[r][c] = ld_nt16(a.q + (size_t)row * K + kc[c]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)       // a clamped chunk (k >= K) gets scale 0
                acc = fmaf(dot16_i8_f32(wq[r][c], xv[t][c]), kok[c] ? h2f(wd[r][c]) : 0.f, acc);
            const float v = wave_sum(acc);
            if (lane == r * T + t && row0 + r < N) reinterpret_cast<float*>(a.out)[(size_t)t * N + row0 + r] = v;
        }
}

template <int T, int RW>
static void launch_gemv_wave_rw(GemvArgs a, hipStream_t st) {
    const dim3 g((a.N + RW - 1) / RW), b(64);
    switch ((a.K + 1023) / 1024) {
        case 1: hipLaunchKernelGGL((gemv_wave_kernel<T, RW, 1>), g, b, 0, st, a); break;
        case 2: hipLaunchKernelGGL((gemv_wave_kernel<T, RW, 2>), g, b, 0, st, a); break;
        case 3: hipLaunchKernelGGL((gemv_wave_kernel<T, RW, 3>), g, b, 0, st, a); break;
        default: hipLaunchKernelGGL((gemv_wave_kernel<T, RW, 4>), g, b, 0, st, a); break;
    }
}

// wave-owned rows up to this many tokens and this depth (measured at 1024 x 4096: T = 1 / 2 / 3
// 3.16 / 3.73 / 4.58 us against 3.50 / 4.04 / 4.89 with the work-group kernel; T = 4 spills)
constexpr int kGemvWaveMaxT = 3;
constexpr int kGemvWaveMaxK = 4096;

template <int T> constexpr int gemv_rw() { return T == 2 ? 4 : (T <= 4 ? 2 : 1); }

// From this many token rows on, the GEMV runs on MFMA (the down read's slab kernel with x as the
// A operand and 256-column slabs, then its combine): the VALU dot re-reads x from cache for
// every 16 weight bytes, which binds once T grows.
constexpr int kGemvMfmaT = 5;

template <int T>
static int launch_gemv_mfma_t(GemvArgs a, void* ws, hipStream_t st);

template <int T>
static int launch_gemv_t(GemvArgs a, void* ws, hipStream_t st) {
    if constexpr (T >= kGemvMfmaT) {
        if (a.K > 0) return launch_gemv_mfma_t<T>(a, ws, st);
    }
    if constexpr (T <= kGemvWaveMaxT) {
        if (a.K <= kGemvWaveMaxK && !force_general()) {
            launch_gemv_wave_rw<T, (T == 1 ? 1 : 2)>(a, st);
            return launch_status();
        }
    }
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

int launch_q8_0_gemv(GemvArgs a, void* ws, hipStream_t st) { GQ8_T_SWITCH(launch_gemv_t, a, ws, st) }

// ------------------------------------------------------------------------------ down read

constexpr int kDnNB = kDownSlab / 32;      // Q8_0 blocks per slab
constexpr int kDnStride = kDownSlab + 16;  // padded LDS row stride of a wave's weight tile (bytes)
constexpr int kDnRows = 64;                // rows per work-group: four row tiles of 16

// Column parts of a work-group's 512-column slab: from T = 9 on (two A planes, so twice the
// staging and MFMA work per wave) eight waves take the four row tiles x two column halves and add
// the halves through LDS; up to T = 8, and on the GEMV's narrower slabs, four waves take whole
// rows (the split is slower there, measured).
template <int T, bool WB, int SLAB = kDownSlab>
constexpr int dn_parts() { return (WB || T <= 8 || SLAB < kDownSlab) ? 1 : 2; }

// One work-group: a slab of 512 columns x 64 rows, one 16-row MFMA tile per wave (from T = 9, two
// waves per tile, one per 256-column half: see dn_parts). Work-groups
// are dealt round-robin to the 8 XCDs (work-group i to XCD i % 8), each with its own L2; when the
// slab count is a multiple of 8, XCD x gets slabs [x S/8, (x+1) S/8) for every row group, so the
// activation columns and the 128-byte scale lines a slab group shares are fetched into one L2
// only. The A operand is u = R * w_norm for the slab, staged once per work-group as exact bf16
// hi and lo parts; for T <= 8 the two parts share one A operand (rows 0..7 hi, rows 8..15 lo of
// token t), so one MFMA per block does both, and the hi and lo results are added at the end
// (the block scale multiplies both). A wave reads its 16 x 512-byte weight tile in four column
// quarters of two coalesced 1 KiB loads (eight rows x 128 bytes each), in the order the work
// consumes them: activations and block scales first, then quarter 0, 1, 2, 3, so that the LDS
// transpose, int8 -> bf16 conversion and MFMAs of one quarter run while the later quarters are
// still in flight. The weight tile is private to its wave; each lane loads the block scales of
// its own result row directly.
//
// XF (the Q8_0 GEMV at larger T): the A operand is x itself (fp32 [T][K]) instead of R * w_norm;
// hi = bf16(x) and lo = bf16(x - hi), both rounded to nearest, leave |x - hi - lo| <= 2^-17 |x|,
// far inside the read's tolerance; no sums of squares.
//
// WB (the BF16 comparison read): the weights are bf16 [N][K], no block scales. A wave's tile is
// 16 x 1024 bytes, read in four quarters of four 1 KiB loads (four rows x 256 bytes each); the
// MFMA B operand is 8 bf16 straight from the LDS tile and the block results chain in the MFMA
// accumulator (A is zero past the slab end).
//
// LA (the last-arriver combine, one column part only): every work-group also keeps its own copy
// of its slab's sums of squares (per row group), and after its partial sums are stored (every
// wave waiting for its stores, then a work-group barrier), thread 0 adds one to the row group's
// counter with an agent-scope release atomic (the one that sees S - 1 then takes an agent-scope
// acquire fence: the arrivals form a release sequence on the counter). The work-group that sees S - 1 was
// the last: it adds the row group's S partial planes and applies rs exactly as
// hc_down_combine_kernel does (same order: bitwise the same outputs) and resets the counter.
// No work-group waits for another, so nothing assumes that they are resident together.
//
// PW (the pending write, HC-Q8 page "Summary"): the staging reads P beside R and takes
// R' = bf16(R + P) in place of R (the fp32 sum of two bf16 values, rounded to nearest even);
// the work-groups of row group 0 also write R' to R_out for their slab.
template <int T, bool XF = false, bool WB = false, int SLAB = kDownSlab, bool LA = false, bool PW = false>
__global__ void __launch_bounds__((256 * dn_parts<T, WB, SLAB>())) hc_down_partial_kernel(GemvArgs a) {
    static_assert(!PW || !XF, "the pending write belongs to the down read");
    static_assert(!LA || dn_parts<T, WB, SLAB>() == 1, "the last-arriver combine takes one column part");
    static_assert(!WB || SLAB == kDownSlab, "the BF16 read uses 512-column slabs");
    constexpr int NB = SLAB / 32;                                  // Q8_0 blocks per slab
    constexpr int NCP = dn_parts<T, WB, SLAB>();                   // column parts of the slab
    constexpr int NWV = 4 * NCP;                                   // waves: 4 row tiles x NCP parts
    constexpr int NTH = 64 * NWV;
    constexpr int NQ = SLAB / 128 / NCP;                           // 128-column quarters per wave
    constexpr bool PACK = T <= 8;
    constexpr int NPL = PACK ? 1 : 2;                              // A planes (hi, lo)
    constexpr int TR = PACK ? 8 : 16;                              // token rows per plane
    constexpr int NI = NB * 4 * TR / NTH;                          // staging items per thread
    constexpr int WS = WB ? 2 * kDownSlab + 16 : SLAB / NCP + 16;  // LDS tile row stride (bytes)
    constexpr int NW = WB ? 16 : 2 * NQ;                           // weight loads per lane
    constexpr int NSW = NB / 2 / NCP;                              // scale words (2 blocks each) per lane
    __shared__ u32x4 ua[NPL][NB][64];                              // A operands, lane order
    __shared__ float sqw[NWV][TR];                                 // per-wave sums of R^2
    __shared__ __attribute__((aligned(16))) uint8_t wt[NWV][16 * WS];
    __shared__ f32x4 part1[NCP > 1 ? 4 : 1][64];                   // column part 1's sums per row tile
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rt = wave & 3, cp = wave >> 2;                       // row tile, column part
    const int N = a.N, K = a.K, nblk = K >> 5;
    const int S = a.S;
    int s, y;
    if ((S & 7) == 0) {
        const int x = blockIdx.x & 7, k = blockIdx.x >> 3, per = S >> 3;
        s = x * per + k % per;
        y = k / per;
    } else {
        s = blockIdx.x % S;
        y = blockIdx.x / S;
    }
    const int k0 = s * SLAB;
    const int cw = imin(SLAB, K - k0);                             // multiple of 32
    const int cb = cw >> 5;
    const int r0 = y * kDnRows + 16 * rt;                          // first row of this wave
    const uint16_t* R = reinterpret_cast<const uint16_t*>(a.x);

    // 0. activations: item it = NTH j + thread covers token t = it % TR (the same t for every
    //    j), columns 32b + 8g .. +8 with b = it / (4 TR), g = (it / TR) % 4
    const int t = (int)threadIdx.x % TR;
    uint4 rv[NI], nv[NI], pv[PW ? NI : 1];
    bool okv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int it = NTH * i + (int)threadIdx.x;
        const int b = it / (4 * TR), g = (it / TR) & 3;
        const int k = k0 + 32 * b + 8 * g;
        okv[i] = t < T && 32 * b < cw;
        const int kc = okv[i] ? k : 0, tc = okv[i] ? t : 0;
        if (XF) {                                  // eight fp32 x values
            const float* xf = reinterpret_cast<const float*>(a.x) + (size_t)tc * K + kc;
            rv[i] = *reinterpret_cast<const uint4*>(xf);
            nv[i] = *reinterpret_cast<const uint4*>(xf + 4);
        } else {
            rv[i] = *reinterpret_cast<const uint4*>(R + (size_t)tc * K + kc);
            nv[i] = *reinterpret_cast<const uint4*>(a.wnorm + kc);
            if constexpr (PW) pv[PW ? i : 0] = *reinterpret_cast<const uint4*>(a.pw + (size_t)tc * K + kc);
        }
    }
    // block scales in the MFMA result layout: lane l needs the scales of row r0 + l%16 for the
    //    wave's column part (16 contiguous bytes a part when the slab is whole and scale rows are
    //    16-byte aligned)
    const int j = lane & 15, g = lane >> 4;
    const int b0 = (NB / NCP) * cp;                                // first block of the part
    uint32_t sw[NSW];
    if (!WB) {
        const int row = imin(r0 + j, N - 1);
        const uint16_t* dr = a.d + (size_t)row * nblk + (k0 >> 5) + b0;
        if (cb == NB && (nblk & 7) == 0) {
            if constexpr (NSW >= 4) {
#pragma unroll
                for (int h = 0; h < NSW / 4; ++h) {
                    const u32x4 s4 = *reinterpret_cast<const u32x4*>(dr + 8 * h);
                    sw[4 * h] = s4.x; sw[4 * h + 1] = s4.y; sw[4 * h + 2] = s4.z; sw[4 * h + 3] = s4.w;
                }
            } else {
                const uint2 s2 = *reinterpret_cast<const uint2*>(dr);
                sw[0] = s2.x; sw[1] = s2.y;
            }
        } else {
            // a ragged slab: clamped loads, all in flight at once (no branch and wait per load);
            // the MFMA loop gives the blocks past the slab's end scale 0
            const uint16_t* ds = a.d + (size_t)row * nblk + (k0 >> 5);
            uint32_t lo16[NSW], hi16[NSW];
#pragma unroll
            for (int i = 0; i < NSW; ++i) {
                lo16[i] = ds[imin(b0 + 2 * i, cb - 1)];
                hi16[i] = ds[imin(b0 + 2 * i + 1, cb - 1)];
            }
#pragma unroll
            for (int i = 0; i < NSW; ++i) sw[i] = lo16[i] | (hi16[i] << 16);
        }
    }
    // 1. weights: the wave's quarter q = i / 2 (slab quarter NQ cp + q) covers columns
    //    128 (NQ cp + q) .. +128; load i covers rows 8(i%2) .. +8 of it (8 lanes a row)
    u32x4 wv[NW];
    if constexpr (WB) {
        // quarter q = i / 4 covers bytes 256q .. +256 of the slab's 1024-byte rows; load i covers
        // rows 4(i%4) .. +4 of it (16 lanes a row)
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int row = imin(r0 + 4 * (i & 3) + (lane >> 4), N - 1);
            const int col = 2 * k0 + imin(256 * (i >> 2) + 16 * (lane & 15), 2 * cw - 16);
            wv[i] = ld_nt16(a.q + (size_t)row * 2 * K + col);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int row = imin(r0 + 8 * (i & 1) + (lane >> 3), N - 1);
            const int col = k0 + imin(128 * (NQ * cp + (i >> 1)) + 16 * (lane & 7), cw - 16);
            wv[i] = ld_nt16(a.q + (size_t)row * K + col);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. u = R * w_norm, exact in fp32, split exactly into bf16 hi + lo, written as A operands:
    //    lane l of block b holds row l%16, columns 32b + 8(l/16) .. +8
    float r2acc = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int it = NTH * i + (int)threadIdx.x;
        const int b = it / (4 * TR), g = (it / TR) & 3;
        const bool ok = okv[i];
        uint32_t rw[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
        if constexpr (PW) {
            // R' = bf16(R + P) (the fp32 sum, rounded to nearest even), written out by row group 0
            const uint32_t pw4[4] = {pv[PW ? i : 0].x, pv[PW ? i : 0].y, pv[PW ? i : 0].z, pv[PW ? i : 0].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float s0 = __uint_as_float(rw[e] << 16) + __uint_as_float(pw4[e] << 16);
                const float s1 = __uint_as_float(rw[e] & 0xffff0000u) + __uint_as_float(pw4[e] & 0xffff0000u);
                rw[e] = (uint32_t)f2bf_bits(s0) | ((uint32_t)f2bf_bits(s1) << 16);
            }
            if (y == 0 && ok) {
                const int k = k0 + 32 * b + 8 * g;
                *reinterpret_cast<uint4*>(a.r_out + (size_t)t * K + k) = make_uint4(rw[0], rw[1], rw[2], rw[3]);
            }
        }
        const uint32_t ww[4] = {nv[i].x, nv[i].y, nv[i].z, nv[i].w};
        uint32_t hi[4], lo[4];
        float r2 = 0.f;
        if (XF) {
            const uint32_t xw[8] = {rw[0], rw[1], rw[2], rw[3], ww[0], ww[1], ww[2], ww[3]};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float u0 = ok ? __uint_as_float(xw[2 * e]) : 0.f;
                const float u1 = ok ? __uint_as_float(xw[2 * e + 1]) : 0.f;
                const uint16_t h0 = f2bf_bits(u0), h1 = f2bf_bits(u1);
                hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                lo[e] = (uint32_t)f2bf_bits(u0 - bf2f(h0)) | ((uint32_t)f2bf_bits(u1 - bf2f(h1)) << 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float q0 = __uint_as_float(rw[e] << 16), q1 = __uint_as_float(rw[e] & 0xffff0000u);
                const float w0 = __uint_as_float(ww[e] << 16), w1 = __uint_as_float(ww[e] & 0xffff0000u);
                const float u0 = ok ? q0 * w0 : 0.f, u1 = ok ? q1 * w1 : 0.f;   // exact products
                const uint16_t h0 = f2bf_bits(u0), h1 = f2bf_bits(u1);
                const float l0 = u0 - bf2f(h0), l1 = u1 - bf2f(h1);             // exact residuals
                hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                lo[e] = pack_bf16_trunc(l0, l1);                                // exact in bf16
                r2 = fmaf(q0, q0, r2);
                r2 = fmaf(q1, q1, r2);
            }
        }
        if (PACK) {
            ua[0][b][16 * g + t] = u32x4{hi[0], hi[1], hi[2], hi[3]};
            ua[0][b][16 * g + 8 + t] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        } else {
            ua[0][b][16 * g + t] = u32x4{hi[0], hi[1], hi[2], hi[3]};
            ua[NPL - 1][b][16 * g + t] = u32x4{lo[0], lo[1], lo[2], lo[3]};
        }
        r2acc += ok ? r2 : 0.f;
    }
    // sums of R^2 of token t: over the lanes of the wave holding t (lane bits above TR), then
    // over the waves (in the epilogue), in a fixed order
#pragma unroll
    for (int m = TR; m < 64; m <<= 1)
        r2acc += m == 8 ? lane_xor8f(r2acc) : (m == 16 ? lane_xor16f(r2acc) : lane_xor32f(r2acc));
    if (lane < TR) sqw[wave][lane] = r2acc;
    __syncthreads();

    // 3. per quarter: weight tile into LDS (this wave only), then per block one MFMA (two for
    //    T > 8) on the exact operands and the block scale (0 past the slab end)
    uint8_t* tile = wt[wave];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (WB) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4*>(tile + (4 * i + (lane >> 4)) * WS + 256 * qq + 16 * (lane & 15)) =
                    wv[4 * qq + i];
            __builtin_amdgcn_wave_barrier();   // LDS accesses of one wave complete in order
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = 4 * qq + i;
                const u32x4 w = *reinterpret_cast<const u32x4*>(tile + j * WS + 64 * b + 16 * g);
                acc = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, ua[0][b][lane]), __builtin_bit_cast(bf16x8, w), acc);
                if (!PACK) acc = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, ua[NPL - 1][b][lane]), __builtin_bit_cast(bf16x8, w), acc);
            }
        }
    }
    if constexpr (!WB)
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *reinterpret_cast<u32x4*>(tile + (8 * i + (lane >> 3)) * WS + 128 * qq + 16 * (lane & 7)) =
                wv[2 * qq + i];
        __builtin_amdgcn_wave_barrier();       // LDS accesses of one wave complete in order
        uint2 q[4];
        u32x4 x0[4], x1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int bl = 4 * qq + i, b = b0 + bl;             // block in the part, in the slab
            q[i] = *reinterpret_cast<const uint2*>(tile + j * WS + 32 * bl + 8 * g);
            x0[i] = ua[0][b][lane];
            if (!PACK) x1[i] = ua[NPL - 1][b][lane];
        }
        f32x4 D[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8 w = i8x8_to_bf16x8(q[i].x, q[i].y);
            const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
            D[i] = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, x0[i]), w, zf);
            if (!PACK) D[i] = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, x1[i]), w, D[i]);
        }
        __builtin_amdgcn_sched_barrier(0);     // four MFMAs in flight, then their scales
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int bl = 4 * qq + i, b = b0 + bl;
            const uint32_t sp = sw[bl >> 1];
            const float dsc = b < cb ? h2f((uint16_t)((bl & 1) ? (sp >> 16) : (sp & 0xffffu))) : 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = fmaf(dsc, D[i][v], acc[v]);
        }
    }

    // 4. the column parts' sums added in part order (part 1's through LDS), then the partial sums
    //    of this slab, part[s][t][n] (D lane l: column n = r0 + l%16, rows 4(l/16)+v)
    if constexpr (NCP > 1) {
        if (cp == 1) part1[rt][lane] = acc;
        __syncthreads();
        if (cp == 1) return;
        const f32x4 o = part1[rt][lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = acc[v] + o[v];
    }
    const int n = r0 + j;
    if (PACK) {
        // rows 8..15 (lanes 32..63) hold the lo parts of tokens 0..7: add them to rows 0..7
        float tot[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) tot[v] = acc[v] + lane_xor32f(acc[v]);   // lanes < 32: l + 32
        if (lane < 32) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tt = 4 * g + v;
                if (tt < T && n < N) a.part[((size_t)s * T + tt) * N + n] = tot[v];
            }
        }
    } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 4 * g + v;
            if (tt < T && n < N) a.part[((size_t)s * T + tt) * N + n] = acc[v];
        }
    }
    if (!XF && (y == 0 || LA) && threadIdx.x < T) {
        const int tt = threadIdx.x;
        float v = sqw[0][tt];
#pragma unroll
        for (int w = 1; w < NWV; ++w) v += sqw[w][tt];
        a.ssq[((size_t)y * S + s) * T + tt] = v;           // row group 0's copy is [S][T]
    }
    if constexpr (LA) {
        __shared__ int s_last;
        __shared__ float s_rs[16];
        // every wave's partial-sum stores complete in L2 (vmcnt 0) before the barrier, so that
        // thread 0's agent-scope release (an L2 writeback) covers all of them, not only its own
        // wave's (the barrier alone does not wait for other waves' global stores)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            // release: this work-group's partial sums before the arrival; only the last arriver
            // needs the acquire (an L2 invalidate), so the others skip it
            const unsigned old = __hip_atomic_fetch_add(a.cnt + y, 1u, __ATOMIC_RELEASE,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            s_last = old == (unsigned)(S - 1);
            if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        if (!s_last) return;
        // the last work-group of row group y: rs per token (the combine kernel's lane-strided
        // sums and wave sum), then the 64 rows x T outputs over the S planes
        if (!XF && wave == 0) {
            for (int tt = 0; tt < T; ++tt) {
                float ss = 0.f;
                for (int s2 = lane; s2 < S; s2 += 64) ss += a.ssq[((size_t)y * S + s2) * T + tt];
                ss = wave_sum(ss);
                if (lane == 0) {
                    const float rs = 1.0f / sqrtf(ss / (float)a.K + a.eps);
                    s_rs[tt] = rs;
                    if (y == 0 && a.rs_out != nullptr) a.rs_out[tt] = rs;
                }
            }
        }
        __syncthreads();
        const int per = (S + 3) / 4;
        for (int o = threadIdx.x; o < 64 * T; o += NTH) {
            const int nl = o & 63, tt = o >> 6;
            const int nn = y * kDnRows + nl;
            if (nn >= N) continue;
            float gs[4];
#pragma unroll
            for (int sg = 0; sg < 4; ++sg) {
                const int s0 = sg * per, s1 = imin(S, s0 + per);
                float v = 0.f;
                for (int sb = s0; sb < s1; sb += 8) {
                    float p[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) p[i] = a.part[((size_t)imin(sb + i, S - 1) * T + tt) * N + nn];
#pragma unroll
                    for (int i = 0; i < 8; ++i) v += sb + i < s1 ? p[i] : 0.f;
                }
                gs[sg] = v;
            }
            const float tot = ((gs[0] + gs[1]) + gs[2]) + gs[3];
            if (XF)
                reinterpret_cast<float*>(a.out)[(size_t)tt * N + nn] = tot;
            else
                reinterpret_cast<uint16_t*>(a.out)[(size_t)tt * N + nn] = f2bf_bits(s_rs[tt] * tot);
        }
        if (threadIdx.x == 0) __hip_atomic_store(a.cnt + y, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// lo[t][n] = bf16(rs[t] * sum_s part[s][t][n]); one work-group per (64 rows, t). Four slab groups
// of ceil(S/4) consecutive slabs are each added in ascending order, then the groups in order.
// XF: the GEMV's y[t][n] = sum_s part[s][t][n] in fp32, same order, no rs.
template <bool XF = false>
__global__ void __launch_bounds__(256) hc_down_combine_kernel(GemvArgs a) {
    __shared__ float red[4][64];
    __shared__ float s_rs;
    const int t = blockIdx.y;
    const int sg = threadIdx.x >> 6, nl = threadIdx.x & 63;
    const int n = blockIdx.x * 64 + nl;
    const int S = a.S, N = a.N;
    const int per = (S + 3) / 4;
    const int s0 = sg * per, s1 = imin(S, s0 + per);
    const int nc = imin(n, N - 1);
    // the first sum-of-squares term of each rs lane (the only one while S <= 64) is loaded ahead
    // of the partial sums, clamped rather than behind a branch, so it shares their round trip
    const float sq0 = XF ? 0.f : a.ssq[(size_t)imin((int)threadIdx.x & 63, S - 1) * a.T + t];
    float v = 0.f;
    for (int s = s0; s < s1; s += 8) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = a.part[((size_t)imin(s + i, S - 1) * a.T + t) * N + nc];
#pragma unroll
        for (int i = 0; i < 8; ++i) v += s + i < s1 ? p[i] : 0.f;
    }
    if (!XF && threadIdx.x < 64) {     // rs[t]: lane-strided sums, then the wave sum
        float ss = (int)threadIdx.x < S ? 0.f + sq0 : 0.f;
        for (int s = threadIdx.x + 64; s < S; s += 64) ss += a.ssq[(size_t)s * a.T + t];
        ss = wave_sum(ss);
        if (threadIdx.x == 0) {
            const float rs = 1.0f / sqrtf(ss / (float)a.K + a.eps);
            s_rs = rs;
            if (blockIdx.x == 0 && a.rs_out != nullptr) a.rs_out[t] = rs;
        }
    }
    red[sg][nl] = v;
    __syncthreads();
    if (threadIdx.x < 64 && n < N && a.out != nullptr) {
        const float tot = ((red[0][nl] + red[1][nl]) + red[2][nl]) + red[3][nl];
        if (XF)
            reinterpret_cast<float*>(a.out)[(size_t)t * N + n] = tot;
        else
            reinterpret_cast<uint16_t*>(a.out)[(size_t)t * N + n] = f2bf_bits(s_rs * tot);
    }
}

// The up read's weights fetched ahead (the pair at T = 1). The whole-row down read below keeps
// its SIMDs busy with VALU work and leaves HBM bandwidth unused, while the up read that follows
// it starts with its own weights cold. So the pair's down launch carries one extra work-group
// per up work-group (64 rows each): extra work-group i reads up work-group i's quant rows and
// block scales with cache-allocating loads, all issued before the first use (addresses past
// the rows clamp to their first piece), and folds them into a value stored only under an
// impossible condition, so no load can be dropped. Work-groups are dealt to the 8 XCDs in turn,
// so with the extra work-groups starting at a multiple of 8, extra work-group i and up
// work-group i run on the same XCD and the up read finds its rows in that XCD's L2 or the
// memory-side cache. No result depends on it.
constexpr int kUpAheadRows = 64;           // rows of an up work-group (four waves of 16)
constexpr int kUpAheadMaxWG = 1024;        // up reads of more rows than this many work-groups: no fetch

template <int NPT>
GQ8_DEV uint32_t fetch_rows_ahead(const GemvArgs& a, size_t qb, size_t qe, size_t sb, size_t se) {
    const size_t nt = blockDim.x, tid = threadIdx.x;
    u32x4 v[NPT];
    uint32_t w[2];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const size_t o = qb + 16 * (tid + (size_t)j * nt);
        v[j] = *reinterpret_cast<const u32x4*>(a.pfq + (o < qe ? o : qb));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const size_t o = sb + 2 * (tid + (size_t)j * nt);          // two scales a load
        w[j] = *reinterpret_cast<const uint32_t*>(a.pfd + (o + 1 < se ? o : sb));
    }
    uint32_t acc = w[0] ^ w[1];
#pragma unroll
    for (int j = 0; j < NPT; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    // what the batch does not cover (deep rows, small work-groups): further rounds
    for (size_t o = qb + 16 * (tid + (size_t)NPT * nt); o < qe; o += 16 * nt) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(a.pfq + o);
        acc ^= u.x ^ u.y ^ u.z ^ u.w;
    }
    for (size_t o = sb + 2 * (tid + 2 * nt); o + 1 < se; o += 2 * nt)
        acc ^= *reinterpret_cast<const uint32_t*>(a.pfd + o);
    return acc;
}

GQ8_DEV void fetch_up_rows_ahead(const GemvArgs& a, int i) {
    const int rlo = kUpAheadRows * i, rhi = imin(a.pf_n, rlo + kUpAheadRows);
    const size_t qb = (size_t)rlo * a.pf_k, qe = (size_t)rhi * a.pf_k;
    const size_t sb = (size_t)rlo * (a.pf_k / 32), se = (size_t)rhi * (a.pf_k / 32);
    const size_t npt = ((qe - qb) / 16 + blockDim.x - 1) / blockDim.x;
    uint32_t acc;
    switch (npt) {
        case 0: case 1: acc = fetch_rows_ahead<1>(a, qb, qe, sb, se); break;
        case 2: acc = fetch_rows_ahead<2>(a, qb, qe, sb, se); break;
        case 3: acc = fetch_rows_ahead<3>(a, qb, qe, sb, se); break;
        case 4: acc = fetch_rows_ahead<4>(a, qb, qe, sb, se); break;
        case 5: acc = fetch_rows_ahead<5>(a, qb, qe, sb, se); break;
        default: acc = fetch_rows_ahead<6>(a, qb, qe, sb, se); break;
    }
    if (acc == 0x9e3779b9u && a.N < 0) reinterpret_cast<uint16_t*>(a.out)[0] = 0;
}

// Down read on whole rows (small T): a work-group owns RW rows and all of K, so no partial sums
// and no combine. Wave w takes the 1024-column chunks w, w + NW, ... (CPW of them per pass, all
// loaded before the first arithmetic: activations first, then the weights, as the GEMV's
// work-group kernel does with x); lane l takes columns
// 16l .. 16l + 15 of a chunk. u = R * w_norm is formed in fp32 (exact: two 8-bit significands)
// and each lane adds q * u for its 16 columns (each product exact in fp32), times the block
// scale, in chunk order; the sums of R^2 ride along. Each work-group reads all of R and w_norm
// (from L2 after the first), adds the waves' sums through LDS in wave order, forms rs from its
// own sum of squares (the same order in every work-group, so every work-group gets the same rs)
// and rounds lo = bf16(rs * y). PW: the pending write, R' = bf16(R + P) in place of R, written
// to R_out by work-group 0.
template <int T, int RW, int CPW, bool PW = false>
__global__ void __launch_bounds__(1024) hc_down_rows_kernel(GemvArgs a) {
    __shared__ float red[16][RW * T + T];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int NW = blockDim.x >> 6;
    const int N = a.N, K = a.K, nblk = K >> 5;
    {
        const int nrg = (N + RW - 1) / RW;                 // row work-groups; then the fetch-ahead
        if ((int)blockIdx.x >= nrg) {                      // ones from the next multiple of 8
            const int nrg8 = (nrg + 7) & ~7;
            if ((int)blockIdx.x >= nrg8) fetch_up_rows_ahead(a, (int)blockIdx.x - nrg8);
            return;
        }
    }
    const int row0 = blockIdx.x * RW;
    const int nchunk = (K + 1023) >> 10;
    const uint16_t* R = reinterpret_cast<const uint16_t*>(a.x);

    float acc[RW][T], r2[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        r2[t] = 0.f;
#pragma unroll
        for (int r = 0; r < RW; ++r) acc[r][t] = 0.f;
    }
    for (int c0 = wave; c0 < nchunk; c0 += NW * CPW) {
        int kc[CPW];
        bool kok[CPW];
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int k = (c0 + c * NW) * 1024 + lane * 16;
            kok[c] = k < K;                                     // K % 32 == 0: k + 16 <= K
            kc[c] = kok[c] ? k : K - 16;
        }
        uint4 rv[CPW][T][2], nv[CPW][2], pv[CPW][PW ? T : 1][2];
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint4* rp = reinterpret_cast<const uint4*>(R + (size_t)t * K + kc[c]);
                rv[c][t][0] = rp[0];
                rv[c][t][1] = rp[1];
                if constexpr (PW) {
                    const uint4* pp = reinterpret_cast<const uint4*>(a.pw + (size_t)t * K + kc[c]);
                    pv[c][t][0] = pp[0];
                    pv[c][t][1] = pp[1];
                }
            }
            const uint4* np = reinterpret_cast<const uint4*>(a.wnorm + kc[c]);
            nv[c][0] = np[0];
            nv[c][1] = np[1];
        }
        u32x4 wq[CPW][RW];
        uint16_t wd[CPW][RW];
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int row = imin(row0 + r, N - 1);
                wd[c][r] = a.d[(size_t)row * nblk + (kc[c] >> 5)];
                wq[c][r] = ld_nt16(a.q + (size_t)row * K + kc[c]);
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const uint32_t nw[8] = {nv[c][0].x, nv[c][0].y, nv[c][0].z, nv[c][0].w,
                                    nv[c][1].x, nv[c][1].y, nv[c][1].z, nv[c][1].w};
#pragma unroll
            for (int t = 0; t < T; ++t) {
                uint32_t rw[8] = {rv[c][t][0].x, rv[c][t][0].y, rv[c][t][0].z, rv[c][t][0].w,
                                  rv[c][t][1].x, rv[c][t][1].y, rv[c][t][1].z, rv[c][t][1].w};
                if constexpr (PW) {
                    const uint32_t pw8[8] = {pv[c][PW ? t : 0][0].x, pv[c][PW ? t : 0][0].y,
                                             pv[c][PW ? t : 0][0].z, pv[c][PW ? t : 0][0].w,
                                             pv[c][PW ? t : 0][1].x, pv[c][PW ? t : 0][1].y,
                                             pv[c][PW ? t : 0][1].z, pv[c][PW ? t : 0][1].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float s0 = __uint_as_float(rw[e] << 16) + __uint_as_float(pw8[e] << 16);
                        const float s1 = __uint_as_float(rw[e] & 0xffff0000u) + __uint_as_float(pw8[e] & 0xffff0000u);
                        rw[e] = (uint32_t)f2bf_bits(s0) | ((uint32_t)f2bf_bits(s1) << 16);
                    }
                    if (blockIdx.x == 0 && kok[c]) {
                        uint4* op = reinterpret_cast<uint4*>(a.r_out + (size_t)t * K + kc[c]);
                        op[0] = make_uint4(rw[0], rw[1], rw[2], rw[3]);
                        op[1] = make_uint4(rw[4], rw[5], rw[6], rw[7]);
                    }
                }
                float u[16], s2 = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float q0 = __uint_as_float(rw[e] << 16), q1 = __uint_as_float(rw[e] & 0xffff0000u);
                    u[2 * e] = q0 * __uint_as_float(nw[e] << 16);              // exact products
                    u[2 * e + 1] = q1 * __uint_as_float(nw[e] & 0xffff0000u);
                    s2 = fmaf(q0, q0, s2);
                    s2 = fmaf(q1, q1, s2);
                }
                r2[t] += kok[c] ? s2 : 0.f;
#pragma unroll
                for (int r = 0; r < RW; ++r)
                    acc[r][t] = fmaf(dot16_i8_f32(wq[c][r], u), kok[c] ? h2f(wd[c][r]) : 0.f, acc[r][t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const float v = wave_sum(acc[r][t]);
            if (lane == 0) red[wave][r * T + t] = v;
        }
        const float s = wave_sum(r2[t]);
        if (lane == 0) red[wave][RW * T + t] = s;
    }
    __syncthreads();
    if ((int)threadIdx.x < RW * T) {
        const int t = (int)threadIdx.x / RW, r = (int)threadIdx.x - t * RW;
        float y = 0.f, ss = 0.f;
        for (int w = 0; w < NW; ++w) {
            y += red[w][r * T + t];
            ss += red[w][RW * T + t];
        }
        const float rs = 1.0f / sqrtf(ss / (float)K + a.eps);
        if (blockIdx.x == 0 && r == 0 && a.rs_out != nullptr) a.rs_out[t] = rs;
        const int row = row0 + r;
        if (row < N && a.out != nullptr) reinterpret_cast<uint16_t*>(a.out)[(size_t)t * N + row] = f2bf_bits(rs * y);
    }
}

// Whole-row down reads up to this many tokens. At T = 1 this kernel is VALU-bound (its dots, and
// the activation arithmetic that every work-group repeats) but needs no combine: measured on
// MI355X at 320 x 16384, the down call 5.90 -> 4.25 us and the pair (then with the direct up
// kernel) 8.24 -> 8.00 us. At T = 2 and 3 the down call gains too but the pair loses against the
// fused combine, and the pair must stay bitwise the two separate calls.
constexpr int kDownRowsMaxT = 1;
constexpr int kDownRowsRW = 2;     // rows per work-group: 160 work-groups at N = 320 (1 and 4: slower)

template <int T, bool PW>
static int launch_down_rows_t(GemvArgs a, hipStream_t st) {
    constexpr int RW = kDownRowsRW;
    const int nchunk = (a.K + 1023) / 1024;
    const int nw = nchunk > 16 ? 16 : nchunk;
    const int nrg = (a.N + RW - 1) / RW;
    const int grid = a.pfq != nullptr ? ((nrg + 7) & ~7) + (a.pf_n + kUpAheadRows - 1) / kUpAheadRows : nrg;
    hipLaunchKernelGGL((hc_down_rows_kernel<T, RW, 1, PW>), dim3(grid), dim3(64 * nw), 0, st, a);
    return launch_status();
}

// Down-read workspace: one arrival counter per 64-row group first (zero between calls; 256
// bytes for every N <= 4096, so calls of different shapes find their counters at the same
// zeroed bytes), then the partial sums [S][T][N], then the sums of squares [G][S][T] (G = row
// groups; the kernel combine reads row group 0's copy, the last-arriver combine each group's own).
static size_t dn_groups(int N) { return (size_t)(N + kDnRows - 1) / kDnRows; }

size_t hc_down_counter_bytes(int N) { return round_up(dn_groups(N) * sizeof(unsigned), kCounterAlign); }

size_t hc_down_workspace_bytes(int T, int N, int K) {
    const size_t S = hc_down_slabs(K);
    return hc_down_counter_bytes(N) + round_up(S * T * N * sizeof(float), kCounterAlign) +
           round_up(dn_groups(N) * S * T * sizeof(float), kCounterAlign);
}

static void dn_workspace(GemvArgs& a, int T, void* ws) {
    const int S = hc_down_slabs(a.K);
    char* w = static_cast<char*>(ws);
    const size_t cb = hc_down_counter_bytes(a.N);
    const size_t pb = round_up((size_t)S * T * a.N * sizeof(float), kCounterAlign);
    a.S = S;
    a.cnt = reinterpret_cast<unsigned*>(w);
    a.part = reinterpret_cast<float*>(w + cb);
    a.ssq = reinterpret_cast<float*>(w + cb + pb);
}

// the last-arriver combine where the slab kernel has one column part (T <= 8 for 512 columns)
template <int T>
static bool dn_last_arriver() { return dn_parts<T, false>() == 1 && combine_last_arriver(); }

template <int T>
static bool down_rows() { return T <= kDownRowsMaxT && !force_general(); }

template <int T>
static int launch_down_t(GemvArgs a, void* ws, hipStream_t st) {
    if constexpr (T <= kDownRowsMaxT) {
        if (down_rows<T>()) return launch_down_rows_t<T, false>(a, st);
    }
    dn_workspace(a, T, ws);
    const int S = a.S;
    if constexpr (dn_parts<T, false>() == 1) {
        if (combine_last_arriver()) {
            hipLaunchKernelGGL((hc_down_partial_kernel<T, false, false, kDownSlab, true>), dim3(S * ((a.N + kDnRows - 1) / kDnRows)), dim3(256), 0, st, a);
            return launch_status();
        }
    }
    hipLaunchKernelGGL((hc_down_partial_kernel<T>), dim3(S * ((a.N + kDnRows - 1) / kDnRows)), dim3(256 * dn_parts<T, false>()), 0, st, a);
    int rc = launch_status();
    if (rc != GQ8_OK) return rc;
    hipLaunchKernelGGL(hc_down_combine_kernel<false>, dim3((a.N + 63) / 64, T), dim3(256), 0, st, a);
    return launch_status();
}

int launch_hc_down(GemvArgs a, void* ws, hipStream_t st) { GQ8_T_SWITCH(launch_down_t, a, ws, st) }

// the down read with the pending write: the slab kernel with PW, then the combine kernel
template <int T>
static int launch_down_pending_t(GemvArgs a, void* ws, hipStream_t st) {
    if constexpr (T <= kDownRowsMaxT) {
        if (down_rows<T>()) return launch_down_rows_t<T, true>(a, st);
    }
    dn_workspace(a, T, ws);
    hipLaunchKernelGGL((hc_down_partial_kernel<T, false, false, kDownSlab, false, true>), dim3(a.S * ((a.N + kDnRows - 1) / kDnRows)), dim3(256 * dn_parts<T, false>()), 0, st, a);
    const int rc = launch_status();
    if (rc != GQ8_OK) return rc;
    hipLaunchKernelGGL(hc_down_combine_kernel<false>, dim3((a.N + 63) / 64, T), dim3(256), 0, st, a);
    return launch_status();
}

int launch_hc_down_pending(GemvArgs a, void* ws, hipStream_t st) { GQ8_T_SWITCH(launch_down_pending_t, a, ws, st) }

// The GEMV's slabs are 256 columns wide (the down read's are 512): twice the work-groups on the
// weight stream (the 1024 x 4096 read has 16 row groups), for twice the partial planes.
constexpr int kGemvSlab = 256;

static int gemv_slabs(int K) { return (K + kGemvSlab - 1) / kGemvSlab; }

// GEMV workspace (T >= 5): one arrival counter per row group first (as the down read's), then
// the partial sums [S][T][N]
size_t gemv_counter_bytes(int T, int N, int K) {
    if (T < kGemvMfmaT || N == 0 || K == 0) return 0;
    return round_up(dn_groups(N) * sizeof(unsigned), kCounterAlign);
}

size_t gemv_workspace_bytes(int T, int N, int K) {
    if (T < kGemvMfmaT || N == 0 || K == 0) return 0;
    const size_t S = gemv_slabs(K);
    return gemv_counter_bytes(T, N, K) + round_up(S * T * N * sizeof(float), kCounterAlign);
}

template <int T>
static int launch_gemv_mfma_t(GemvArgs a, void* ws, hipStream_t st) {
    const int S = gemv_slabs(a.K);
    a.S = S;
    a.cnt = static_cast<unsigned*>(ws);
    a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + gemv_counter_bytes(T, a.N, a.K));
    a.ssq = nullptr;
    if (combine_last_arriver()) {
        hipLaunchKernelGGL((hc_down_partial_kernel<T, true, false, kGemvSlab, true>), dim3(S * ((a.N + kDnRows - 1) / kDnRows)), dim3(256), 0, st, a);
        return launch_status();
    }
    hipLaunchKernelGGL((hc_down_partial_kernel<T, true, false, kGemvSlab>), dim3(S * ((a.N + kDnRows - 1) / kDnRows)), dim3(256 * dn_parts<T, false, kGemvSlab>()), 0, st, a);
    int rc = launch_status();
    if (rc != GQ8_OK) return rc;
    hipLaunchKernelGGL(hc_down_combine_kernel<true>, dim3((a.N + 63) / 64, T), dim3(256), 0, st, a);
    return launch_status();
}

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
template <int T>
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
        const int cw = K - c0 < kUpCW ? K - c0 : kUpCW;   // multiple of 32
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
            if (e < 16 * np) {
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

// K % 320 == 0: the weight tile goes straight from the loads into MFMA operands. Load i gives lane
// l the 16 bytes of row l%16 at column 64i + 16(l/16) of the chunk: Q8_0 block 2i in lanes 0..31,
// block 2i+1 in lanes 32..63. One v_permlane32_swap per dword pair (lanes l and l+32 trade a dword)
// leaves lane (row j, k-group g) holding, for each of the two blocks, the 8 bytes at block offset
// {0, 16, 8, 24}[g]; the input operand takes its k-groups at the same offsets. Each block's MFMA
// waits only for its own load, so the work of early loads overlaps the arrival of later ones.
GQ8_DEV int up_koff(int g) { return 16 * (g & 1) + 8 * (g >> 1); }

// TL: quants in the tiled layout: the wave's 16 rows x 64 columns of load i are one 1 KiB tile,
// lane l's 16 bytes at byte 16 l of it (the same bytes a lane as the split layout's row pieces).
template <int T, bool TL = false>
__global__ void __launch_bounds__(256) hc_up_direct_kernel(GemvArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t xl[kMaxT][kUpLoStride];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int N = a.N, K = a.K, nblk = K >> 5;
    const int r0 = (blockIdx.x * 4 + wave) * 16;
    const int j = lane & 15, g = lane >> 4;
    const int row = imin(r0 + j, N - 1);
    const uint16_t* lo = reinterpret_cast<const uint16_t*>(a.x);
    constexpr int npx = kUpCW / 8;                                  // 16-byte pieces per input row
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int tj = j < T ? j : 0;
    const int ko = 2 * up_koff(g);                                  // byte offset in a bf16 row

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < K; c0 += kUpCW) {
        // the input chunk (T rows x 40 pieces), the row's 10 block scales, the 5 weight loads
        u32x4 xv[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int e = imin(i * 256 + (int)threadIdx.x, T * npx - 1);
            const int t = e / npx, pc = e - t * npx;
            xv[i] = *reinterpret_cast<const u32x4*>(lo + (size_t)t * K + c0 + 8 * pc);
        }
        uint32_t sc[kUpCB / 2];
        const uint32_t* dp = reinterpret_cast<const uint32_t*>(a.d + (size_t)row * nblk + (c0 >> 5));
#pragma unroll
        for (int i = 0; i < kUpCB / 2; ++i) sc[i] = dp[i];
        u32x4 wv[kUpLoads];
        const int8_t* wp = TL ? a.q + ((size_t)(r0 >> 4) * (K >> 6) + (c0 >> 6)) * 1024 + 16 * lane
                              : a.q + (size_t)row * K + c0 + 16 * g;
#pragma unroll
        for (int i = 0; i < kUpLoads; ++i) wv[i] = ld_nt16(wp + (TL ? 1024 : 64) * i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int e = i * 256 + (int)threadIdx.x;
            if (e < T * npx) {
                const int t = e / npx, pc = e - t * npx;
                *reinterpret_cast<u32x4*>(&xl[t][16 * pc]) = xv[i];
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kUpLoads; ++i) {
            const auto s02 = __builtin_amdgcn_permlane32_swap(wv[i].x, wv[i].z, false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(wv[i].y, wv[i].w, false, false);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int b = 2 * i + h;
                const u32x4 x = *reinterpret_cast<const u32x4*>(&xl[tj][64 * b + ko]);
                const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
                const f32x4 D = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, j < T ? x : z),
                                                   i8x8_to_bf16x8(s02[h], s13[h]), zf);
                const float dsc = h2f((uint16_t)(h ? (sc[i] >> 16) : (sc[i] & 0xffffu)));
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(dsc, D[v], acc[v]);
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

// The BF16 comparison up read (any K % 32 == 0): one wave per 16 output rows, the input staged
// per 320-column chunk in LDS; lane l loads the 16 bytes of row l%16 at column 32b + 8(l/16) of
// block b, the MFMA B operand as it stands, and the blocks chain in the accumulator.
template <int T>
__global__ void __launch_bounds__(256) hc_up_bf16_kernel(GemvArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t xl[kMaxT][kUpLoStride];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int N = a.N, K = a.K;
    const int r0 = (blockIdx.x * 4 + wave) * 16;
    const int j = lane & 15, g = lane >> 4;
    const int row = imin(r0 + j, N - 1);
    const uint16_t* lo = reinterpret_cast<const uint16_t*>(a.x);
    const uint8_t* wr = reinterpret_cast<const uint8_t*>(a.q) + (size_t)row * 2 * K;
    constexpr int npx = kUpCW / 8;                                  // 16-byte pieces per chunk row
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int tj = j < T ? j : 0;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < K; c0 += kUpCW) {
        const int cbn = imin(kUpCB, (K - c0) >> 5);                  // blocks in this chunk
        const int npc = 4 * cbn;                                    // pieces in this chunk row
        u32x4 xv[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int e = imin(i * 256 + (int)threadIdx.x, T * npx - 1);
            const int t = e / npx, pc = imin(e - t * npx, npc - 1);
            xv[i] = *reinterpret_cast<const u32x4*>(lo + (size_t)t * K + c0 + 8 * pc);
        }
        u32x4 wb[kUpCB];
#pragma unroll
        for (int b = 0; b < kUpCB; ++b) wb[b] = ld_nt16(wr + 2 * (c0 + 32 * imin(b, cbn - 1)) + 16 * g);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int e = i * 256 + (int)threadIdx.x;
            if (e < T * npx) {
                const int t = e / npx, pc = e - t * npx;
                if (pc < npc) *reinterpret_cast<u32x4*>(&xl[t][16 * pc]) = xv[i];
            }
        }
        __syncthreads();
#pragma unroll
        for (int b = 0; b < kUpCB; ++b) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(&xl[tj][64 * b + 16 * g]);
            acc = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, (j < T && b < cbn) ? x : z),
                                     __builtin_bit_cast(bf16x8, wb[b]), acc);
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
    if (a.wt) {                            // tiled weights: the direct kernel only
        if (a.K % kUpCW != 0 || a.N % 16 != 0) return GQ8_ESHAPE;
        hipLaunchKernelGGL((hc_up_direct_kernel<T, true>), dim3((ntile + 3) / 4), dim3(256), 0, st, a);
        return launch_status();
    }
    if (a.K % kUpCW == 0 && !force_general()) {
        hipLaunchKernelGGL((hc_up_direct_kernel<T>), dim3((ntile + 3) / 4), dim3(256), 0, st, a);
    } else {
        GQ8_NOTE_GENERAL("up read: general up kernel (LDS staged): depth not a multiple of 320, or forced");
        hipLaunchKernelGGL((hc_up_kernel<T>), dim3((ntile + 3) / 4), dim3(256), 0, st, a);
    }
    return launch_status();
}

int launch_hc_up(GemvArgs a, hipStream_t st) { GQ8_T_SWITCH(launch_up_t, a, st) }

// ------------------------------------------------------------------------------ fused pair

// The up read of the down/up pair for K == 320 and small T with the down's combine folded in:
// waves 4..7 of the work-group add the down's slab partial sums for all T x 320 inputs (the same
// order as hc_down_combine_kernel, so lo is bitwise the down read's output), apply rs and round
// to bf16 into LDS, while waves 0..3 have their weight loads in flight; after the combine's
// barriers waves 0..3 run the up read's MFMAs as hc_up_direct_kernel does. Every work-group
// computes the same lo; work-group 0 also writes lo and rs out. Separate waves keep the
// partial-sum loads from waiting behind the weight loads (a wave's loads complete in issue
// order), and the weight loads start only after the partial-sum loads are issued.
constexpr int kPairQuads = kUpCW / 4;       // float4 quads of a 320-wide row

// WB (the BF16 comparison read): bf16 weights [N][320]; lane l loads the 16 bytes of row l%16 at
// column 32b + 8(l/16) for block b, which is the MFMA B operand as it stands (no scales).
// Waves of the fused kernel: kPairNup up waves (16 rows each) and kPairNcw combine waves.
// Measured on MI355X (pair at T = 2 / 3 / 4): 4 + 4 8.74 / 9.28 / 10.02 us; 8 + 4 9.29 / 9.76 /
// 10.61; 8 + 8 9.71 / 9.96 / 10.81; 12 + 4 10.6 / 12.2 / 16.4. Fewer, larger work-groups halve
// the partial-sum reads in total but not the combine on each work-group's critical path, and put
// the weight stream on fewer CUs.
constexpr int kPairNup = 4;
constexpr int kPairNcw = 4;

template <int T, bool WB = false, bool TL = false>
__global__ void __launch_bounds__(64 * (kPairNup + kPairNcw)) hc_pair_up_kernel(GemvArgs a) {
    constexpr int NQ = T * kPairQuads;                            // float4 quads of lo
    constexpr int NTC = 64 * kPairNcw;                            // combine threads
    constexpr int NIT = (4 * NQ + NTC - 1) / NTC;                 // (quad, slab group) items per thread
    __shared__ __attribute__((aligned(16))) uint8_t xl[kMaxT][kUpLoStride];
    __shared__ float4 red[4][NQ];                                 // slab-group sums
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int N = a.N, K = a.K;                                   // up rows, up depth (== 320)
    const int j = lane & 15, g = lane >> 4;
    if (wave < kPairNup) {
        // weights and scales of this wave's 16 rows, issued once the combine waves have issued
        // their partial-sum loads (those are few and on the critical path; issued behind the
        // weight stream they wait in the same memory queues), then in flight across the combine
        const int r0 = (blockIdx.x * kPairNup + wave) * 16;
        __syncthreads();                                          // partial-sum loads issued
        const int row = imin(r0 + j, N - 1);
        const u32x4 z = {0u, 0u, 0u, 0u};
        const int tj = j < T ? j : 0;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (WB) {
            u32x4 wb[kUpCB];
            const uint8_t* wp = reinterpret_cast<const uint8_t*>(a.q) + (size_t)row * 2 * K + 16 * g;
#pragma unroll
            for (int b = 0; b < kUpCB; ++b) wb[b] = ld_nt16(wp + 64 * b);
            __syncthreads();                                      // slab-group sums in LDS
            __syncthreads();                                      // lo in LDS
#pragma unroll
            for (int b = 0; b < kUpCB; ++b) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(&xl[tj][64 * b + 16 * g]);
                acc = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, j < T ? x : z), __builtin_bit_cast(bf16x8, wb[b]), acc);
            }
        }
        uint32_t sc[kUpCB / 2];
        u32x4 wv[kUpLoads];
        if constexpr (!WB) {
            const uint32_t* dp = reinterpret_cast<const uint32_t*>(a.d + (size_t)row * (K >> 5));
#pragma unroll
            for (int i = 0; i < kUpCB / 2; ++i) sc[i] = dp[i];
            const int8_t* wp = TL ? a.q + (size_t)(r0 >> 4) * (K >> 6) * 1024 + 16 * lane
                                  : a.q + (size_t)row * K + 16 * g;
#pragma unroll
            for (int i = 0; i < kUpLoads; ++i) wv[i] = ld_nt16(wp + (TL ? 1024 : 64) * i);
            __syncthreads();                                      // slab-group sums in LDS
            __syncthreads();                                      // lo in LDS
        }
        const int ko = 2 * up_koff(g);
#pragma unroll
        for (int i = 0; i < (WB ? 0 : kUpLoads); ++i) {
            const auto s02 = __builtin_amdgcn_permlane32_swap(wv[i].x, wv[i].z, false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(wv[i].y, wv[i].w, false, false);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int b = 2 * i + h;
                const u32x4 x = *reinterpret_cast<const u32x4*>(&xl[tj][64 * b + ko]);
                const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
                const f32x4 D = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, j < T ? x : z),
                                                   i8x8_to_bf16x8(s02[h], s13[h]), zf);
                const float dsc = h2f((uint16_t)(h ? (sc[i] >> 16) : (sc[i] & 0xffffu)));
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(dsc, D[v], acc[v]);
            }
        }
        uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
        const int n = r0 + j;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = 4 * g + v;
            if (t < T && n < N) out[(size_t)t * N + n] = f2bf_bits(acc[v]);
        }
        return;
    }
    // combine waves. Item it = ct + NTC m is (quad it % NQ, slab group it / NQ): the group's
    // ceil(S/4) consecutive slabs added in ascending order; every item's loads are issued before
    // the first wait. Then rs[t] from the slab sums of squares (lane-strided, then the wave sum),
    // and lo = bf16(rs * (((g0 + g1) + g2) + g3)) -- hc_down_combine_kernel's order.
    const int S = a.S;
    const int ct = (int)threadIdx.x - 64 * kPairNup;
    const int per = (S + 3) / 4;
    const size_t plane = (size_t)T * K / 4;                       // float4s per slab plane
    float4 gs[NIT];
    float sv[T];                                                  // S == 32: ssq of slab lane % 32
    if (S == 32) {                                                // per == 8: one batch of loads
        float4 pv[NIT][8];
#pragma unroll
        for (int m = 0; m < NIT; ++m) {
            const int it = imin(ct + NTC * m, 4 * NQ - 1);
            const int qd = it % NQ, sg = it / NQ;
            const int t = qd / kPairQuads, n = 4 * (qd - t * kPairQuads);
            const float4* p = reinterpret_cast<const float4*>(a.part + (size_t)t * K + n) + (size_t)8 * sg * plane;
#pragma unroll
            for (int i = 0; i < 8; ++i) pv[m][i] = p[(size_t)i * plane];
        }
#pragma unroll
        for (int t = 0; t < T; ++t) sv[t] = a.ssq[(size_t)(lane & 31) * T + t];
        __builtin_amdgcn_sched_barrier(0);                        // every load issued, then
        __syncthreads();                                          // the weight loads may start
#pragma unroll
        for (int m = 0; m < NIT; ++m) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v.x += pv[m][i].x; v.y += pv[m][i].y; v.z += pv[m][i].z; v.w += pv[m][i].w;
            }
            gs[m] = v;
        }
    } else {
        __syncthreads();
#pragma unroll
        for (int m = 0; m < NIT; ++m) {
            const int it = imin(ct + NTC * m, 4 * NQ - 1);
            const int qd = it % NQ, sg = it / NQ;
            const int t = qd / kPairQuads, n = 4 * (qd - t * kPairQuads);
            const float4* p = reinterpret_cast<const float4*>(a.part + (size_t)t * K + n);
            const int s0 = sg * per, s1 = imin(S, s0 + per);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int s = s0; s < s1; s += 8) {
                float4 pv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) pv[i] = p[(size_t)imin(s + i, S - 1) * plane];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const bool in = s + i < s1;
                    v.x += in ? pv[i].x : 0.f; v.y += in ? pv[i].y : 0.f;
                    v.z += in ? pv[i].z : 0.f; v.w += in ? pv[i].w : 0.f;
                }
            }
            gs[m] = v;
        }
    }
    float rs[T];
    {
        float ss[T];
#pragma unroll
        for (int t = 0; t < T; ++t) ss[t] = (S == 32 && lane < 32) ? 0.f + sv[t] : 0.f;
        for (int s = S == 32 ? S : lane; s < S; s += 64) {
#pragma unroll
            for (int t = 0; t < T; ++t) ss[t] += a.ssq[(size_t)s * T + t];
        }
#pragma unroll
        for (int t = 0; t < T; ++t) rs[t] = 1.0f / sqrtf(wave_sum(ss[t]) / (float)a.kd + a.eps);
    }
#pragma unroll
    for (int m = 0; m < NIT; ++m) {
        const int it = ct + NTC * m;
        if (it < 4 * NQ) red[it / NQ][it % NQ] = gs[m];
    }
    if (blockIdx.x == 0 && ct < T && a.rs_out != nullptr) {
#pragma unroll
        for (int t = 0; t < T; ++t)
            if (t == ct) a.rs_out[t] = rs[t];
    }
    __syncthreads();
    for (int qd = ct; qd < NQ; qd += NTC) {
        const int t = qd / kPairQuads, n = 4 * (qd - t * kPairQuads);
        float r = rs[0];
#pragma unroll
        for (int tt = 1; tt < T; ++tt) r = tt == t ? rs[tt] : r;
        const float4 v0 = red[0][qd], v1 = red[1][qd], v2 = red[2][qd], v3 = red[3][qd];
        const float tx = ((v0.x + v1.x) + v2.x) + v3.x;
        const float ty = ((v0.y + v1.y) + v2.y) + v3.y;
        const float tz = ((v0.z + v1.z) + v2.z) + v3.z;
        const float tw = ((v0.w + v1.w) + v2.w) + v3.w;
        uint2 lv;
        lv.x = (uint32_t)f2bf_bits(r * tx) | ((uint32_t)f2bf_bits(r * ty) << 16);
        lv.y = (uint32_t)f2bf_bits(r * tz) | ((uint32_t)f2bf_bits(r * tw) << 16);
        *reinterpret_cast<uint2*>(&xl[t][2 * n]) = lv;
        if (blockIdx.x == 0 && a.lo_out != nullptr)
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.lo_out) + (size_t)t * K + n) = lv;
    }
    __syncthreads();
}

// The in-kernel combine reads all S x T x 320 partial sums in every up work-group (L2 traffic
// and registers that grow with T), the separate combine kernel costs one more launch: measured on
// MI355X at K = 16384 (S = 32), folding wins up to T = 4 (T = 4: 9.9 us vs 10.8 us).
constexpr int kPairMaxT = 4;

// the pair's whole-row down read fetches the up read's weights ahead (hc_down_rows_kernel)
static void fetch_up_ahead(GemvArgs& dn, const GemvArgs& up) {
    // rows and depth in multiples of 32 (as every pair has them): each extra work-group then has
    // at least 32 block scales, so its two-scale loads never pass its rows
    if (up.N % 32 != 0 || up.K % 32 != 0) return;
    if ((up.N + kUpAheadRows - 1) / kUpAheadRows > kUpAheadMaxWG) return;
    dn.pfq = up.q; dn.pfd = up.d; dn.pf_n = up.N; dn.pf_k = up.K;
}

template <int T>
static int launch_pair_t(GemvArgs dn, GemvArgs up, void* ws, hipStream_t st) {
    if constexpr (T > kPairMaxT) {
        const int rc = launch_down_t<T>(dn, ws, st);
        return rc != GQ8_OK ? rc : launch_up_t<T>(up, st);
    } else {
        if (down_rows<T>() || dn_last_arriver<T>()) {   // the down call, then the up read
            if (down_rows<T>()) fetch_up_ahead(dn, up);
            const int rc = launch_down_t<T>(dn, ws, st);
            return rc != GQ8_OK ? rc : launch_up_t<T>(up, st);
        }
        dn_workspace(dn, T, ws);
        const int S = dn.S;
        hipLaunchKernelGGL((hc_down_partial_kernel<T>), dim3(S * ((dn.N + kDnRows - 1) / kDnRows)), dim3(256 * dn_parts<T, false>()), 0, st, dn);
        int rc = launch_status();
        if (rc != GQ8_OK) return rc;
        up.S = S; up.part = dn.part; up.ssq = dn.ssq; up.eps = dn.eps; up.kd = dn.K;
        up.rs_out = dn.rs_out; up.lo_out = dn.out;
        const int ntile = (up.N + 15) / 16;
        if (up.wt) {
            if (up.N % 16 != 0) return GQ8_ESHAPE;
            hipLaunchKernelGGL((hc_pair_up_kernel<T, false, true>), dim3((ntile + kPairNup - 1) / kPairNup), dim3(64 * (kPairNup + kPairNcw)), 0, st, up);
        } else {
            hipLaunchKernelGGL((hc_pair_up_kernel<T>), dim3((ntile + kPairNup - 1) / kPairNup), dim3(64 * (kPairNup + kPairNcw)), 0, st, up);
        }
        return launch_status();
    }
}

// the pair with the pending write: as launch_pair_t, the down read's slab kernel with PW
template <int T>
static int launch_pair_pending_t(GemvArgs dn, GemvArgs up, void* ws, hipStream_t st) {
    if constexpr (T > kPairMaxT) {
        const int rc = launch_down_pending_t<T>(dn, ws, st);
        return rc != GQ8_OK ? rc : launch_up_t<T>(up, st);
    } else {
        if (up.K != kUpCW || force_general() || down_rows<T>()) {
            if (down_rows<T>()) fetch_up_ahead(dn, up);
            const int rc = launch_down_pending_t<T>(dn, ws, st);
            return rc != GQ8_OK ? rc : launch_up_t<T>(up, st);
        }
        dn_workspace(dn, T, ws);
        const int S = dn.S;
        hipLaunchKernelGGL((hc_down_partial_kernel<T, false, false, kDownSlab, false, true>), dim3(S * ((dn.N + kDnRows - 1) / kDnRows)), dim3(256 * dn_parts<T, false>()), 0, st, dn);
        int rc = launch_status();
        if (rc != GQ8_OK) return rc;
        up.S = S; up.part = dn.part; up.ssq = dn.ssq; up.eps = dn.eps; up.kd = dn.K;
        up.rs_out = dn.rs_out; up.lo_out = dn.out;
        const int ntile = (up.N + 15) / 16;
        hipLaunchKernelGGL((hc_pair_up_kernel<T>), dim3((ntile + kPairNup - 1) / kPairNup), dim3(64 * (kPairNup + kPairNcw)), 0, st, up);
        return launch_status();
    }
}

int launch_hc_pair_pending(GemvArgs dn, GemvArgs up, void* ws, hipStream_t st) {
    GemvArgs& a = dn;
    GQ8_T_SWITCH(launch_pair_pending_t, dn, up, ws, st)
}

int launch_hc_pair(GemvArgs dn, GemvArgs up, void* ws, hipStream_t st) {
    if (up.K != kUpCW || force_general()) {   // no fused variant: the down read, then the up read
        const int rc = launch_hc_down(dn, ws, st);
        return rc != GQ8_OK ? rc : launch_hc_up(up, st);
    }
    GemvArgs& a = dn;
    GQ8_T_SWITCH(launch_pair_t, dn, up, ws, st)
}

// ------------------------------------------------------------------------------ BF16 pair

template <int T>
static int launch_bf16_pair_t(GemvArgs dn, GemvArgs up, void* ws, hipStream_t st) {
    dn_workspace(dn, T, ws);
    const int S = dn.S;
    hipLaunchKernelGGL((hc_down_partial_kernel<T, false, true>), dim3(S * ((dn.N + kDnRows - 1) / kDnRows)), dim3(256), 0, st, dn);
    int rc = launch_status();
    if (rc != GQ8_OK) return rc;
    const int ntile = (up.N + 15) / 16;
    if constexpr (T <= kPairMaxT) {
        if (up.K == kUpCW) {               // the combine inside the up kernel
            up.S = S; up.part = dn.part; up.ssq = dn.ssq; up.eps = dn.eps; up.kd = dn.K;
            up.rs_out = dn.rs_out; up.lo_out = dn.out;
            hipLaunchKernelGGL((hc_pair_up_kernel<T, true>), dim3((ntile + kPairNup - 1) / kPairNup), dim3(64 * (kPairNup + kPairNcw)), 0, st, up);
            return launch_status();
        }
    }
    hipLaunchKernelGGL(hc_down_combine_kernel<false>, dim3((dn.N + 63) / 64, T), dim3(256), 0, st, dn);
    if ((rc = launch_status()) != GQ8_OK) return rc;
    hipLaunchKernelGGL((hc_up_bf16_kernel<T>), dim3((ntile + 3) / 4), dim3(256), 0, st, up);
    return launch_status();
}

int launch_hc_bf16_pair(GemvArgs dn, GemvArgs up, void* ws, hipStream_t st) {
    GemvArgs& a = dn;
    GQ8_T_SWITCH(launch_bf16_pair_t, dn, up, ws, st)
}

}  // namespace gq8
