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
//   M >= 2:  v_mfma_i32_16x16x64_i8 (rows past M are zero), one MFMA row tile for M <= 16 and
//            two (sharing the weight fragment) for M <= 32. One x load per k-step per lane;
//            the VALU dot needs M of them, which bound it from M = 4 on (measured).
//   M == 1:  v_dot4_i32_i8 on the VALU over the same fragments.
// int32 sums are exact, so every order gives the one correct accumulator; the epilogue is
// bf16( (fp32(acc) * x_scale[m]) * w_scale[n] ), two rounded fp32 products.
#include "gq8_device.h"
#include "gq8_internal.h"

namespace gq8 {

typedef int v4i __attribute__((ext_vector_type(4)));

struct W8Args {
    const int8_t* xq;
    const float* xs;
    const int8_t* wp;
    const float* wsc;
    void* out;
    int i32_out;
    int M, N, K;
    int ksteps;
};

GQ8_DEV int imin8(int a, int b) { return a < b ? a : b; }

// x_scale[m] * ... of the thread's first output (i = thread of the M x 16 tile), loaded at kernel
// start so that the epilogue does not wait for a global load after the reduction.
struct W8Scales {
    float xs, ws;
};

GQ8_DEV W8Scales w8a8_prefetch_scales(const W8Args& a, int nt) {
    const int i = (int)threadIdx.x;
    const int m = imin8(i >> 4, a.M - 1), n = imin8(nt * 16 + (i & 15), a.N - 1);
    W8Scales sc;
    sc.xs = a.i32_out ? 0.f : a.xs[m];
    sc.ws = a.i32_out ? 0.f : a.wsc[n];
    return sc;
}

// The WG's int32 tiles [NW][32][16] -> sum over waves (in wave order) -> epilogue.
GQ8_DEV void w8a8_finish(const W8Args& a, int nt, int nw, int (*tile)[32][16], W8Scales sc) {
    __syncthreads();
    for (int i = threadIdx.x; i < a.M * 16; i += blockDim.x) {
        const int m = i >> 4, nl = i & 15;
        const int n = nt * 16 + nl;
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
                f = f * (first ? sc.xs : a.xs[m]);
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

template <int MT, int KPW>
__global__ void __launch_bounds__(1024) w8a8_mfma_kernel(W8Args a) {
    __shared__ int tile[16][32][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int nt = blockIdx.x;
    v4i b[KPW];
    bool ok[KPW];
    load_frags<KPW>(a, nt, wave, nw, lane, b, ok);
    const W8Scales sc = w8a8_prefetch_scales(a, nt);
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
    w8a8_finish(a, nt, nw, tile, sc);
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
    const W8Scales sc = w8a8_prefetch_scales(a, nt);
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
        t += __shfl_xor(t, 16, 64);
        t += __shfl_xor(t, 32, 64);
        if (lane < 16 && m < a.M) tile[wave][m][lane] = t;
    }
    w8a8_finish(a, nt, nw, tile, sc);
}

// ------------------------------------------------------------------------------------ planning

W8Plan plan_w8a8(int M, int N, int K) {
    W8Plan p{};
    p.mfma = M >= 2;
    p.ntiles = (N + 15) / 16;
    p.ksteps = (K + 63) / 64;
    p.nw = p.ksteps < 16 ? p.ksteps : 16;
    p.kpw = (p.ksteps + p.nw - 1) / p.nw;
    return p;
}

template <int KPW>
static int launch_w8a8_kpw(const W8Plan& p, W8Args a, hipStream_t st) {
    const dim3 g(p.ntiles), b(64 * p.nw);
    if (p.mfma) {
        if (a.M <= 16) hipLaunchKernelGGL((w8a8_mfma_kernel<1, KPW>), g, b, 0, st, a);
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
                const float* ws_scale, void* out, bool i32_out, int M, int N, int K, hipStream_t st) {
    W8Args a{};
    a.xq = xq; a.xs = xs; a.wp = wp; a.wsc = ws_scale; a.out = out; a.i32_out = i32_out ? 1 : 0;
    a.M = M; a.N = N; a.K = K; a.ksteps = p.ksteps;
    switch (p.kpw) {
        case 1: return launch_w8a8_kpw<1>(p, a, st);
        case 2: return launch_w8a8_kpw<2>(p, a, st);
        case 3: return launch_w8a8_kpw<3>(p, a, st);
        case 4: return launch_w8a8_kpw<4>(p, a, st);
        default: {
            // K > 4096: more k-steps per wave than the unrolled variants hold
            if (p.kpw <= 8) return launch_w8a8_kpw<8>(p, a, st);
            return GQ8_ESHAPE;
        }
    }
}

}  // namespace gq8
