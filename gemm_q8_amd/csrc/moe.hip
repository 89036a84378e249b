// Routed experts with Q8_0 weights and a q8_1 input (EP page, "What changed": the q8_1 MoE input,
// the routed entries grouped by expert so each expert is computed once, then the single-card
// combine; defer page, "What it changes": rows combined weighted by their routing weight).
//
// Kernels, in stream order (D <= 4096 and F in {256, 512, 1024}):
//   gate/up  grid (row pairs, entries): the work-group of entry i works only when i is the first
//            entry routed to its expert (a wave ballot over the ids, no plan kernel) and then
//            serves all of that expert's entries, so each routed expert's weights are read once;
//            per 32-block integer dots (v_dot4_i32_i8) of weight quants with the q8_1 quants,
//            scaled by both block scales; h = SiLU(gate) * up -> h[entry][F] fp32
//   down     grid (16-row tiles, tokens): the token's entries on MFMA, then the combine
//            out[t] = bf16( sum_j w[t][j] * r_{t,j} ), j in order, in the same kernel
// Other shapes: a one-work-group plan kernel (entries sorted by expert) feeds the general gate/up
// kernel (D > 4096) and a VALU down kernel that writes rows[entry][D], then a combine kernel.
// Experts that no token routes to are never read.
#include "gq8_device.h"
#include "gq8_internal.h"

namespace gq8 {

typedef int v4i __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------ routing

GQ8_DEV float block_sum_256(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return ((red[0] + red[1]) + red[2]) + red[3];
}

GQ8_DEV float block_max_256(float v, float* red) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// better = larger value, then lower index
GQ8_DEV bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

__global__ void __launch_bounds__(256) moe_route_kernel(const float* __restrict__ logits, int E,
                                                        int topk, int32_t* __restrict__ ids,
                                                        float* __restrict__ wout) {
    extern __shared__ float sl[];                       // E logits, then E selection flags
    int* sel = reinterpret_cast<int*>(sl + E);
    __shared__ float red[4];
    __shared__ float rv[4];
    __shared__ int ri[4];
    const int t = blockIdx.x;
    const float* l = logits + (size_t)t * E;
    for (int i = threadIdx.x; i < E; i += 256) {
        sl[i] = l[i];
        sel[i] = 0;
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int i = threadIdx.x; i < E; i += 256) mx = fmaxf(mx, sl[i]);
    mx = block_max_256(mx, red);
    float sum = 0.f;
    for (int i = threadIdx.x; i < E; i += 256) sum += expf(sl[i] - mx);
    sum = block_sum_256(sum, red);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int j = 0; j < topk; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int i = threadIdx.x; i < E; i += 256)
            if (!sel[i] && better(sl[i], i, bv, bi)) { bv = sl[i]; bi = i; }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        if (lane == 0) { rv[wave] = bv; ri[wave] = bi; }
        __syncthreads();
        if (threadIdx.x == 0) {
            float b = rv[0];
            int bidx = ri[0];
            for (int w = 1; w < 4; ++w)
                if (better(rv[w], ri[w], b, bidx)) { b = rv[w]; bidx = ri[w]; }
            const bool ok = bidx >= 0 && bidx < E;          // false only for NaN logits
            ids[(size_t)t * topk + j] = ok ? bidx : -1;
            wout[(size_t)t * topk + j] = ok ? expf(b - mx) / sum : 0.f;
            if (ok) sel[bidx] = 1;
        }
        __syncthreads();
    }
}

int launch_moe_route(const float* logits, int T, int E, int topk, int32_t* ids, float* w,
                     hipStream_t st) {
    const size_t lds = (size_t)E * (sizeof(float) + sizeof(int));
    hipLaunchKernelGGL(moe_route_kernel, dim3(T), dim3(256), lds, st, logits, E, topk, ids, w);
    return launch_status();
}

// ------------------------------------------------------------------------------------ plan

// Device plan (layout documented with gq8_moe_plan). P = T*topk <= 256 entries.
GQ8_DEV void build_plan(const int32_t* ids, int P, int E, int32_t* plan) {
    __shared__ int sid[256];
    __shared__ int sorted[256];
    __shared__ int first[256];
    __shared__ int s_bad, s_u;
    const int tid = threadIdx.x;
    if (tid == 0) { s_bad = 0; s_u = 0; }
    __syncthreads();
    if (tid < P) {
        const int e = ids[tid];
        sid[tid] = e;
        if (e < 0 || e >= E) atomicOr(&s_bad, 1);
    }
    __syncthreads();
    if (s_bad) {
        if (tid == 0) plan[0] = -1;
        if (tid < P) {
            plan[1 + tid] = -1;
            plan[1 + P + tid] = 0;
            plan[1 + 2 * P + tid] = P;
            plan[1 + 3 * P + tid] = -1;
        }
        return;
    }
    if (tid < P) {
        const int key = sid[tid];
        int rank = 0;
        for (int j = 0; j < P; ++j) rank += (sid[j] < key) || (sid[j] == key && j < tid);
        sorted[rank] = tid;
    }
    __syncthreads();
    if (tid < P) {
        first[tid] = (tid == 0) || (sid[sorted[tid]] != sid[sorted[tid - 1]]);
        if (first[tid]) atomicAdd(&s_u, 1);
    }
    __syncthreads();
    const int U = s_u;
    if (tid == 0) plan[0] = U;
    if (tid < P) {
        int u = -1;
        for (int j = 0; j <= tid; ++j) u += first[j];
        plan[1 + 3 * P + tid] = sorted[tid];
        if (first[tid]) {
            int c = 1;
            while (tid + c < P && !first[tid + c]) ++c;
            plan[1 + u] = sid[sorted[tid]];
            plan[1 + P + u] = c;
            plan[1 + 2 * P + u] = tid;
        }
        if (tid >= U) {
            plan[1 + tid] = -1;
            plan[1 + P + tid] = 0;
            plan[1 + 2 * P + tid] = P;
        }
    }
}

// The plan (1 + 4P words) copied into LDS with one round of vector loads: the slot's expert,
// count, start and entries are then LDS reads instead of a chain of dependent global loads.
constexpr int kPlanWords = 1 + 4 * 256;

GQ8_DEV void plan_to_lds(const int32_t* plan, int P, int32_t* lplan) {
    const int n = 1 + 4 * P;
#pragma unroll
    for (int k = 0; k < kPlanWords / 256 + 1; ++k) {
        const int i = (int)threadIdx.x + 256 * k;
        if (i < n) lplan[i] = plan[i];
    }
    __syncthreads();
}

__global__ void __launch_bounds__(256) moe_plan_kernel(const int32_t* ids, int P, int E, int32_t* plan) {
    build_plan(ids, P, E, plan);
}

int launch_moe_plan(const int32_t* ids, int T, int topk, int E, int32_t* plan, hipStream_t st) {
    hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(256), 0, st, ids, T * topk, E, plan);
    return launch_status();
}

// ------------------------------------------------------------------------------------ experts

struct MoeArgs {
    const int8_t* xq;       // [T][D]
    const uint16_t* xd;     // [T][D/32]
    const uint16_t* xb;     // bf16 [T][D] (the gate/up kernel that quantizes its input itself)
    const float* w;         // routing weights [T][topk]
    const int8_t* wgu;      // gate/up arena
    const int8_t* wdn;      // down arena
    size_t gu_bytes, dn_bytes;
    uint16_t* out;          // [T][D]
    int T, topk, P, E, D, F;
    const int32_t* ids;     // [T][topk] (the kernels that take no plan)
    const int32_t* plan;
    float* h;               // [P][F]
    float* rows;            // [P][D]
};

// The entries routed to entry i's expert, straight from the ids (no plan): lane l of the wave
// holds ids[l], ids[64 + l], ... (P <= 256) and one ballot per word marks the entries whose id
// equals ids[i]; bit k of m[w] is entry 64 w + k. Every lane gets the same (wave-uniform) masks.
// ok is false when any id lies outside [0, E) (the call then writes zeros, as a plan error does).
struct EntrySet {
    uint64_t m[4];
    int e;
    bool ok;
};

GQ8_DEV EntrySet entry_set(const int32_t* ids, int P, int E, int i) {
    const int lane = threadIdx.x & 63;
    int v[4];
    bool bad = false;
    // four loads in flight at once (clamped, no branches: P >= 1), one wait; entry i's own id
    // is lane i % 64 of word i / 64, read across lanes rather than loaded again
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = ids[64 * w + lane < P ? 64 * w + lane : P - 1];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int k = 64 * w + lane;
        if (k >= P) v[w] = -1;
        bad = bad || (k < P && (v[w] < 0 || v[w] >= E));
    }
    EntrySet r;
    const int iw = i >> 6;
    r.e = __builtin_amdgcn_readlane(iw == 0 ? v[0] : iw == 1 ? v[1] : iw == 2 ? v[2] : v[3], i & 63);
    r.ok = __ballot(bad) == 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) r.m[w] = __ballot(64 * w + lane < P && v[w] == r.e);
    return r;
}

// first entry of the set (P if empty)
GQ8_DEV int entry_first(const EntrySet& s) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
        if (s.m[w] != 0) return 64 * w + __builtin_ctzll(s.m[w]);
    return 1 << 30;
}

constexpr int kGuRpw = 2;    // gate/up row pairs per wave

// Gate/up: each wave owns kGuRpw row pairs (gate row n, up row F + n) of one routed expert and
// all of D; a lane reads 16 columns per 1024-column chunk. Loads of a chunk batch (weights,
// scales and the entries' q8_1 quants) are issued together, clamped, before any arithmetic.
template <int CMAX>
__global__ void __launch_bounds__(256) moe_gate_up_kernel(MoeArgs a) {
    constexpr int KB = 1;                          // 1024-column chunks per load batch
    __shared__ int32_t lplan[kPlanWords];
    plan_to_lds(a.plan, a.P, lplan);
    const int slot = blockIdx.y;
    const int U = lplan[0];
    if (slot >= U) return;
    const int P = a.P, D = a.D, F = a.F;
    const int e = lplan[1 + slot];
    const int c = lplan[1 + P + slot];
    const int st = lplan[1 + 2 * P + slot];
    const int8_t* q = a.wgu + (size_t)e * a.gu_bytes;
    const uint16_t* d = reinterpret_cast<const uint16_t*>(q + (size_t)2 * F * D);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pr0 = (blockIdx.x * 4 + wave) * kGuRpw;
    const int nblk = D >> 5;

    // entries in chunks of CMAX (an expert has at most T entries when each token routes to
    // distinct experts, so one chunk in practice; more chunks re-read the weights)
    for (int cb = 0; cb < c; cb += CMAX) {
        const int cn = c - cb < CMAX ? c - cb : CMAX;
        int ent[CMAX], tok[CMAX];
#pragma unroll
        for (int ci = 0; ci < CMAX; ++ci) {
            ent[ci] = lplan[1 + 3 * P + st + cb + (ci < cn ? ci : 0)];
            tok[ci] = ent[ci] / a.topk;
        }
        float ag[kGuRpw][CMAX], au[kGuRpw][CMAX];
#pragma unroll
        for (int r = 0; r < kGuRpw; ++r)
#pragma unroll
            for (int ci = 0; ci < CMAX; ++ci) { ag[r][ci] = 0.f; au[r][ci] = 0.f; }

        for (int k0 = 0; k0 < D; k0 += 1024 * KB) {
            v4i qg[kGuRpw][KB], qu[kGuRpw][KB], xv[CMAX][KB];
            uint16_t dg[kGuRpw][KB], du[kGuRpw][KB], dx[CMAX][KB];
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int k = k0 + j * 1024 + lane * 16;
                const int kc = k < D ? k : D - 16;
#pragma unroll
                for (int r = 0; r < kGuRpw; ++r) {
                    const int n = pr0 + r < F ? pr0 + r : F - 1;
                    qg[r][j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(q + (size_t)n * D + kc));
                    qu[r][j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(q + (size_t)(F + n) * D + kc));
                    dg[r][j] = d[(size_t)n * nblk + (kc >> 5)];
                    du[r][j] = d[(size_t)(F + n) * nblk + (kc >> 5)];
                }
#pragma unroll
                for (int ci = 0; ci < CMAX; ++ci) {
                    xv[ci][j] = *reinterpret_cast<const v4i*>(a.xq + (size_t)tok[ci] * D + kc);
                    dx[ci][j] = a.xd[(size_t)tok[ci] * nblk + (kc >> 5)];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                if (k0 + j * 1024 + lane * 16 >= D) continue;
#pragma unroll
                for (int ci = 0; ci < CMAX; ++ci) {
                    if (ci >= cn) continue;
                    const v4i x = xv[ci][j];
                    const float dxf = h2f(dx[ci][j]);
#pragma unroll
                    for (int r = 0; r < kGuRpw; ++r) {
                        int sg = 0, su = 0;
                        sg = __builtin_amdgcn_sdot4(qg[r][j].x, x.x, sg, false);
                        sg = __builtin_amdgcn_sdot4(qg[r][j].y, x.y, sg, false);
                        sg = __builtin_amdgcn_sdot4(qg[r][j].z, x.z, sg, false);
                        sg = __builtin_amdgcn_sdot4(qg[r][j].w, x.w, sg, false);
                        su = __builtin_amdgcn_sdot4(qu[r][j].x, x.x, su, false);
                        su = __builtin_amdgcn_sdot4(qu[r][j].y, x.y, su, false);
                        su = __builtin_amdgcn_sdot4(qu[r][j].z, x.z, su, false);
                        su = __builtin_amdgcn_sdot4(qu[r][j].w, x.w, su, false);
                        // d_w * d_x is exact in fp32 (11-bit x 11-bit significands)
                        ag[r][ci] = fmaf((float)sg, h2f(dg[r][j]) * dxf, ag[r][ci]);
                        au[r][ci] = fmaf((float)su, h2f(du[r][j]) * dxf, au[r][ci]);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kGuRpw; ++r) {
#pragma unroll
            for (int ci = 0; ci < CMAX; ++ci) {
                if (ci < cn) {
                    const float g = wave_sum(ag[r][ci]);
                    const float u = wave_sum(au[r][ci]);
                    const int n = pr0 + r;
                    if (lane == 0 && n < F) a.h[(size_t)ent[ci] * F + n] = g / (1.0f + expf(-g)) * u;
                }
            }
        }
    }
}

// Gate/up with the wave's weight rows for all of D in registers (D <= 1024 NCH), with no plan:
// the work-group of grid row i works only if entry i is the first entry routed to its expert,
// and then serves every entry of that expert (entry_set), so each routed expert's weights are
// read once. The weight loads of the whole row pairs are issued at once, then the entries are
// taken one at a time in ascending order (x loads per entry, L2-resident), so the registers do
// not grow with the entry count and more work-groups stay resident per CU.
//
// XB: the input is bf16 x itself; the work-group quantizes each entry's row to q8_1 once, into
// LDS (8 values a thread; a block's four threads share its amax through two cross-lane maxes),
// with the q8_1 quantize kernel's rounding (q8_quant_bf16 is q8_quant bit for bit on bf16
// values), so the quants and scales are bitwise those that kernel writes.
template <int NCH, bool XB>
__global__ void __launch_bounds__(256) moe_gate_up_rows_kernel(MoeArgs a) {
    __shared__ __attribute__((aligned(16))) int8_t xq_s[XB ? 1024 * NCH : 16];   // q8_1 of the row
    __shared__ uint16_t xd_s[XB ? 32 * NCH : 1];
    __shared__ uint32_t scs[4][64 * NCH];      // per wave: its gate rows' scales, then its up rows'
    const int i0 = blockIdx.y;
    const EntrySet es = entry_set(a.ids, a.P, a.E, i0);
    if (!es.ok || entry_first(es) != i0) return;
    const int D = a.D, F = a.F;
    const int8_t* q = a.wgu + (size_t)es.e * a.gu_bytes;
    const uint16_t* d = reinterpret_cast<const uint16_t*>(q + (size_t)2 * F * D);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pr0 = (blockIdx.x * 4 + wave) * kGuRpw;
    const int nblk = D >> 5;

    // block scales: the wave's two gate rows (pr0, pr0 + 1, even pr0 < F - 1 since F % 8 == 0)
    // are one run of nblk dwords, its two up rows another; lane l loads dwords l, l + 64, ... of
    // the two runs (NCH loads a lane instead of one 2-byte load per row and chunk: the weight
    // loads wait behind far fewer instructions), ahead of the weights
    static_assert(kGuRpw == 2, "two rows a wave: one dword run per gate or up row pair");
    const uint32_t* d32 = reinterpret_cast<const uint32_t*>(d);
    const size_t g0 = (size_t)pr0 * nblk / 2, u0 = (size_t)(F + pr0) * nblk / 2;
    uint32_t sv[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int idx = lane + 64 * i;
        const int ic = idx < 2 * nblk ? idx : 2 * nblk - 1;
        sv[i] = __builtin_nontemporal_load(d32 + (ic < nblk ? g0 + ic : u0 + (ic - nblk)));
    }
    v4i qg[kGuRpw][NCH], qu[kGuRpw][NCH];
    uint16_t dg[kGuRpw][NCH], du[kGuRpw][NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int k = j * 1024 + lane * 16;
        const int kc = k < D ? k : D - 16;
#pragma unroll
        for (int r = 0; r < kGuRpw; ++r) {
            const int n = pr0 + r;
            qg[r][j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(q + (size_t)n * D + kc));
            qu[r][j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(q + (size_t)(F + n) * D + kc));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NCH; ++i)
        if (lane + 64 * i < 2 * nblk) scs[wave][lane + 64 * i] = sv[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
        const uint16_t* sc16 = reinterpret_cast<const uint16_t*>(scs[wave]);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int k = j * 1024 + lane * 16;
            const int b = (k < D ? k : D - 16) >> 5;
#pragma unroll
            for (int r = 0; r < kGuRpw; ++r) {
                dg[r][j] = sc16[r * nblk + b];
                du[r][j] = sc16[(2 + r) * nblk + b];
            }
        }
    }
    int first_w = 0;                                    // the word holding the first entry
    while (first_w < 3 && es.m[first_w] == 0) ++first_w;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        for (uint64_t mm = es.m[w]; mm != 0; mm &= mm - 1) {
            const int ent = 64 * w + __builtin_ctzll(mm);
            const int tok = ent / a.topk;
            v4i xv[NCH];
            uint16_t dx[NCH];
            if constexpr (XB) {
                // the work-group quantizes the token's row once: thread i takes 8 values (4
                // threads a block, amax over them by two cross-lane maxes) into LDS
                if (mm != es.m[w] || w != first_w) __syncthreads();   // the previous entry's reads
                for (int k8 = 8 * (int)threadIdx.x; k8 < D; k8 += 8 * 256) {
                    const u32x4 xr = *reinterpret_cast<const u32x4*>(a.xb + (size_t)tok * D + k8);
                    const uint32_t w4[4] = {xr.x, xr.y, xr.z, xr.w};
                    float v[8];
                    float am = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[2 * e] = __uint_as_float(w4[e] << 16);
                        v[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
                        am = fmaxf(am, fabsf(v[2 * e]));
                        am = fmaxf(am, fabsf(v[2 * e + 1]));
                    }
                    am = fmaxf(am, lane_xor1f(am));
                    am = fmaxf(am, lane_xor2f(am));
                    const uint16_t db = q8_scale_bits(am);
                    const float dd = h2f(db);
                    uint32_t q2[2] = {0u, 0u};
                    if (dd < __builtin_inff()) {
                        const float rd = __builtin_amdgcn_rcpf(dd);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            q2[e >> 2] |= ((uint32_t)q8_quant_bf16(v[e], dd, rd) & 0xffu) << (8 * (e & 3));
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            q2[e >> 2] |= ((uint32_t)q8_quant(v[e], dd) & 0xffu) << (8 * (e & 3));
                    }
                    *reinterpret_cast<uint2*>(&xq_s[k8]) = make_uint2(q2[0], q2[1]);
                    if ((k8 & 31) == 0) xd_s[k8 >> 5] = db;
                }
                __syncthreads();
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    const int k = j * 1024 + lane * 16;
                    const int kc = k < D ? k : D - 16;
                    xv[j] = *reinterpret_cast<const v4i*>(&xq_s[kc]);
                    dx[j] = xd_s[kc >> 5];
                }
            } else {
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    const int k = j * 1024 + lane * 16;
                    const int kc = k < D ? k : D - 16;
                    xv[j] = *reinterpret_cast<const v4i*>(a.xq + (size_t)tok * D + kc);
                    dx[j] = a.xd[(size_t)tok * nblk + (kc >> 5)];
                }
            }
            float ag[kGuRpw], au[kGuRpw];
#pragma unroll
            for (int r = 0; r < kGuRpw; ++r) { ag[r] = 0.f; au[r] = 0.f; }
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                if (j * 1024 + lane * 16 >= D) continue;
                const v4i x = xv[j];
                const float dxf = h2f(dx[j]);
#pragma unroll
                for (int r = 0; r < kGuRpw; ++r) {
                    int sg = 0, su = 0;
                    sg = __builtin_amdgcn_sdot4(qg[r][j].x, x.x, sg, false);
                    sg = __builtin_amdgcn_sdot4(qg[r][j].y, x.y, sg, false);
                    sg = __builtin_amdgcn_sdot4(qg[r][j].z, x.z, sg, false);
                    sg = __builtin_amdgcn_sdot4(qg[r][j].w, x.w, sg, false);
                    su = __builtin_amdgcn_sdot4(qu[r][j].x, x.x, su, false);
                    su = __builtin_amdgcn_sdot4(qu[r][j].y, x.y, su, false);
                    su = __builtin_amdgcn_sdot4(qu[r][j].z, x.z, su, false);
                    su = __builtin_amdgcn_sdot4(qu[r][j].w, x.w, su, false);
                    // d_w * d_x is exact in fp32 (11-bit x 11-bit significands)
                    ag[r] = fmaf((float)sg, h2f(dg[r][j]) * dxf, ag[r]);
                    au[r] = fmaf((float)su, h2f(du[r][j]) * dxf, au[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < kGuRpw; ++r) {
                const float g = wave_sum(ag[r]);
                const float u = wave_sum(au[r]);
                const int n = pr0 + r;
                if (lane == 0 && n < F) a.h[(size_t)ent * F + n] = g / (1.0f + expf(-g)) * u;
            }
        }
    }
}

// Down projection: rows of F quants, F/16 lanes per row (F <= 1024), h in registers; each row's
// lane partials are summed in a fixed order through LDS.
constexpr int kDnNrs = 2;

template <int CMAX>
__global__ void __launch_bounds__(256) moe_down_kernel(MoeArgs a) {
    extern __shared__ float smem[];
    const int slot = blockIdx.y;
    const int U = a.plan[0];
    if (slot >= U) return;
    const int P = a.P, D = a.D, F = a.F;
    const int e = a.plan[1 + slot];
    const int c = a.plan[1 + P + slot];
    const int st = a.plan[1 + 2 * P + slot];
    const int8_t* q = a.wdn + (size_t)e * a.dn_bytes;
    const uint16_t* d = reinterpret_cast<const uint16_t*>(q + (size_t)D * F);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int LPR = F >> 4, RPS = 64 / LPR;
    const int rsub = lane / LPR, cl = lane - rsub * LPR;
    const bool lane_ok = rsub < RPS;
    const int k = lane_ok ? cl * 16 : 0;
    const int nblk = F >> 5;
    const int base = (blockIdx.x * 4 + wave) * kDnNrs * RPS;

    v4i wq[kDnNrs];
    uint16_t wd[kDnNrs];
#pragma unroll
    for (int i = 0; i < kDnNrs; ++i) {
        int row = base + i * RPS + (lane_ok ? rsub : 0);
        row = row < D ? row : D - 1;
        wq[i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(q + (size_t)row * F + k));
        wd[i] = d[(size_t)row * nblk + (k >> 5)];
    }
    float* red = smem + wave * (kDnNrs * 64 * CMAX);
    const int rows_w = kDnNrs * RPS;

    for (int cb = 0; cb < c; cb += CMAX) {
        const int cn = c - cb < CMAX ? c - cb : CMAX;
        int ent[CMAX];
        float hv[CMAX][16];
#pragma unroll
        for (int ci = 0; ci < CMAX; ++ci) {
            ent[ci] = a.plan[1 + 3 * P + st + cb + (ci < cn ? ci : 0)];
            const float* hp = a.h + (size_t)ent[ci] * F + k;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 f = reinterpret_cast<const float4*>(hp)[i];
                hv[ci][4 * i] = f.x; hv[ci][4 * i + 1] = f.y; hv[ci][4 * i + 2] = f.z; hv[ci][4 * i + 3] = f.w;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ci = 0; ci < CMAX; ++ci) {
            if (ci >= cn) continue;
#pragma unroll
            for (int i = 0; i < kDnNrs; ++i) {
                const float v = h2f(wd[i]) * dot16_i8_f32(__builtin_bit_cast(u32x4, wq[i]), hv[ci]);
                if (lane_ok) red[((i * RPS + rsub) * CMAX + ci) * LPR + cl] = v;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        for (int o = lane; o < rows_w * cn; o += 64) {
            const int ci = o / rows_w;
            const int rl = o - ci * rows_w;
            const int row = base + rl;
            if (row >= D) continue;
            const float* p = red + (rl * CMAX + ci) * LPR;
            float v = 0.f;
            for (int c2 = 0; c2 < LPR; ++c2) v += p[c2];
            int en = 0;
#pragma unroll
            for (int cc = 0; cc < CMAX; ++cc) if (cc == ci) en = ent[cc];
            a.rows[(size_t)en * D + row] = v;
        }
        // the next chunk overwrites red: every lane's reads of this chunk come first
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// Down projection with the combine folded in (F = 64 NL): one work-group per (16 output rows,
// token t), eight waves. Wave w takes the token's entries j = w, w + 8, ..., one at a time (eight
// waves of one entry each measured faster than four waves of two: the q8_1(h) option's per-entry
// quantization spreads over twice the waves, 23.16 -> 22.46 us per call; the default 23.11 ->
// 23.02 us):
// the entry's expert tile of 16 rows x F bytes is read straight into MFMA operands -- load i
// gives lane l the 16 bytes of row l%16 at column 64i + 16(l/16) (Q8_0 block 2i in lanes 0..31,
// 2i+1 in lanes 32..63), and v_permlane32_swap makes both blocks' operands, so lane (row j,
// k-group g) holds block offset {0, 16, 8, 24}[g]. The entry's h (fp32) is staged through LDS
// as bf16 hi and lo (|h - hi - lo| <= 2^-17 |h|); A rows 0..7 take hi and rows 8..15 lo, so
// result rows 0 and 8 hold the two parts. The per-entry results r_j go to LDS and one wave
// forms out[t] = bf16( sum_j w[t][j] r_j ), j in order (the combine's order). An expert that
// two tokens route to is read by both tokens' work-groups. The expert ids are loaded once per
// lane (they are validated and give each entry's expert by a cross-lane read), so the weight
// loads start after one round trip to the ids.
GQ8_DEV int dn_koff(int g) { return 16 * (g & 1) + 8 * (g >> 1); }
GQ8_DEV int imin_m(int x, int y) { return x < y ? x : y; }

constexpr int kMoeMaxTopk = 16;

//
// HQ (the variant whose down read takes q8_1(h)): the staging quantizes the entry's h per
// 32-block (four lanes a block, the input's q8_1 rule) into int8 codes and fp16 scales in LDS,
// and each block is one v_mfma_i32_16x16x32_i8 of those codes with the weight quants as the
// loads give them (no conversion); its int32 result times d_w * d_h (exact in fp32) accumulates
// in fp32.
constexpr int kMoeDnWaves = 8;

template <int NL, bool HQ, bool TL = false>
__global__ void __launch_bounds__(64 * kMoeDnWaves) moe_down_token_kernel(MoeArgs a) {
    constexpr int NWV = kMoeDnWaves;
    constexpr int NB = 2 * NL;                     // Q8_0 blocks per row
    constexpr int F = 64 * NL;
    constexpr int EG = 1;                          // entries in flight per wave
    constexpr int HC = (F / 8 + 63) / 64;          // 8-float pieces of h per lane
    __shared__ __attribute__((aligned(16))) uint16_t hs[HQ ? 1 : NWV][EG][2][HQ ? 8 : F];
    __shared__ __attribute__((aligned(16))) int8_t hq[HQ ? NWV : 1][EG][HQ ? F : 16];
    __shared__ uint16_t hdq[HQ ? NWV : 1][EG][HQ ? NB : 1];
    __shared__ float rr[kMoeMaxTopk][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int t = blockIdx.y, topk = a.topk, D = a.D;
    const int r0 = blockIdx.x * 16;
    const int row = r0 + j < D ? r0 + j : D - 1;

    // every entry's expert id, one load per lane per 64 entries (P <= 256): they validate the
    // ids and give each entry's expert by a cross-lane read, so the weight loads wait for one
    // round trip only (the h loads of the first round are issued before that wait)
    int idv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) idv[c] = a.ids[imin_m(64 * c + lane, a.P - 1)];   // clamped: P >= 1
    bool ok = true;                                // wave-uniform; the same in every wave
    bool checked = false;
    const int ko = 2 * dn_koff(g);                 // byte offset of the lane's k-group in a bf16 row
    const int hl = j < 8 ? 0 : 1;                  // A rows 0..7 hi, 8..15 lo

    for (int j0 = wave; j0 < topk; j0 += NWV * EG) {
        int ent[EG];
        bool on[EG];
        float4 hv[EG][HC][2];
        uint32_t sc[EG][NL];
        v4i wv[EG][NL];
#pragma unroll
        for (int u = 0; u < EG; ++u) {
            const int jj = j0 + NWV * u;
            on[u] = jj < topk;
            ent[u] = __builtin_amdgcn_readfirstlane(t * topk + (on[u] ? jj : j0));
            const float4* hp = reinterpret_cast<const float4*>(a.h + (size_t)ent[u] * F);
#pragma unroll
            for (int c = 0; c < HC; ++c) {
                const int pc = imin_m(lane + 64 * c, F / 8 - 1);
                hv[u][c][0] = hp[2 * pc];
                hv[u][c][1] = hp[2 * pc + 1];
            }
        }
        if (!checked) {
            // the ids are used only from here on, after the h loads are issued (an empty
            // statement that the compiler may not move across memory accesses)
            __asm__ volatile("" : "+v"(idv[0]), "+v"(idv[1]), "+v"(idv[2]), "+v"(idv[3]) :: "memory");
            bool bad = false;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                bad = bad || (64 * c + lane < a.P && (idv[c] < 0 || idv[c] >= a.E));
            ok = __ballot(bad) == 0;
            checked = true;
        }
        if (!ok) break;
#pragma unroll
        for (int u = 0; u < EG; ++u) {
            const int cw = ent[u] >> 6;
            const int sel = cw == 0 ? idv[0] : cw == 1 ? idv[1] : cw == 2 ? idv[2] : idv[3];
            const int eid = __builtin_amdgcn_readlane(sel, ent[u] & 63);
            const int8_t* q = a.wdn + (size_t)eid * a.dn_bytes;
            const uint32_t* dp = reinterpret_cast<const uint32_t*>(q + (size_t)D * F) + (size_t)row * (NB / 2);
#pragma unroll
            for (int i = 0; i < NL; i += 4) {
                const u32x4 s4 = *reinterpret_cast<const u32x4*>(dp + i);
                sc[u][i] = s4.x; sc[u][i + 1] = s4.y; sc[u][i + 2] = s4.z; sc[u][i + 3] = s4.w;
            }
            // split layout: 64-byte pieces of 16 rows; tiled layout: the same 16 bytes a lane,
            // stored as one contiguous 1 KiB tile per load (row group blockIdx.x, column group i)
            const int8_t* wp = TL ? q + (size_t)blockIdx.x * (NL * 1024) + 16 * lane
                                  : q + (size_t)row * F + 16 * g;
#pragma unroll
            for (int i = 0; i < NL; ++i)
                wv[u][i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp + (TL ? 1024 : 64) * i));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < EG && HQ; ++u) {
            // h -> q8_1 codes and block scales in this wave's LDS slot
#pragma unroll
            for (int c = 0; c < HC; ++c) {
                const int pc = lane + 64 * c;
                if (pc < F / 8) {
                    const float f[8] = {hv[u][c][0].x, hv[u][c][0].y, hv[u][c][0].z, hv[u][c][0].w,
                                        hv[u][c][1].x, hv[u][c][1].y, hv[u][c][1].z, hv[u][c][1].w};
                    float am = 0.f;
#pragma unroll
                    for (int e2 = 0; e2 < 8; ++e2) am = fmaxf(am, fabsf(f[e2]));
                    am = fmaxf(am, lane_xor1f(am));
                    am = fmaxf(am, lane_xor2f(am));
                    const uint16_t db = q8_scale_bits(am);
                    const float dd = h2f(db);
                    uint32_t q2[2] = {0u, 0u};
#pragma unroll
                    for (int e2 = 0; e2 < 8; ++e2)
                        q2[e2 >> 2] |= ((uint32_t)q8_quant(f[e2], dd) & 0xffu) << (8 * (e2 & 3));
                    *reinterpret_cast<uint2*>(&hq[HQ ? wave : 0][u][HQ ? 8 * pc : 0]) = make_uint2(q2[0], q2[1]);
                    if ((pc & 3) == 0) hdq[HQ ? wave : 0][u][HQ ? pc >> 2 : 0] = db;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < EG && !HQ; ++u) {
            // h -> bf16 hi, lo in this wave's LDS slot
#pragma unroll
            for (int c = 0; c < HC; ++c) {
                const int pc = lane + 64 * c;
                if (pc < F / 8) {
                    const float f[8] = {hv[u][c][0].x, hv[u][c][0].y, hv[u][c][0].z, hv[u][c][0].w,
                                        hv[u][c][1].x, hv[u][c][1].y, hv[u][c][1].z, hv[u][c][1].w};
                    uint32_t h4[4], l4[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const uint16_t h0 = f2bf_bits(f[2 * e2]), h1 = f2bf_bits(f[2 * e2 + 1]);
                        h4[e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                        l4[e2] = (uint32_t)f2bf_bits(f[2 * e2] - bf2f(h0)) |
                                 ((uint32_t)f2bf_bits(f[2 * e2 + 1] - bf2f(h1)) << 16);
                    }
                    *reinterpret_cast<u32x4*>(&hs[HQ ? 0 : wave][u][0][HQ ? 0 : 8 * pc]) = u32x4{h4[0], h4[1], h4[2], h4[3]};
                    *reinterpret_cast<u32x4*>(&hs[HQ ? 0 : wave][u][1][HQ ? 0 : 8 * pc]) = u32x4{l4[0], l4[1], l4[2], l4[3]};
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int u = 0; u < EG && HQ; ++u) {
            const int8_t* qb = &hq[HQ ? wave : 0][u][0];
            float acc0 = 0.f;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const auto s02 = __builtin_amdgcn_permlane32_swap((uint32_t)wv[u][i].x, (uint32_t)wv[u][i].z, false, false);
                const auto s13 = __builtin_amdgcn_permlane32_swap((uint32_t)wv[u][i].y, (uint32_t)wv[u][i].w, false, false);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int b = 2 * i + h;
                    const uint2 xa = *reinterpret_cast<const uint2*>(qb + (HQ ? 32 * b + dn_koff(g) : 0));
                    const long av = (long)(((unsigned long)xa.y << 32) | xa.x);
                    const long bv = (long)(((unsigned long)s13[h] << 32) | s02[h]);
                    const v4i zi = {0, 0, 0, 0};
                    const v4i Di = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, bv, zi, 0, 0, 0);
                    const float dwh = h2f((uint16_t)(h ? (sc[u][i] >> 16) : (sc[u][i] & 0xffffu))) *
                                      h2f(hdq[HQ ? wave : 0][u][HQ ? b : 0]);     // exact in fp32
                    acc0 = fmaf((float)Di[0], dwh, acc0);
                }
            }
            // result row 0 (lanes 0..15, v = 0): every A row holds the same codes
            if (on[u] && lane < 16) rr[j0 + NWV * u][j] = acc0;
        }
#pragma unroll
        for (int u = 0; u < EG && !HQ; ++u) {
            const uint8_t* hb = reinterpret_cast<const uint8_t*>(&hs[HQ ? 0 : wave][u][hl][0]);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const auto s02 = __builtin_amdgcn_permlane32_swap((uint32_t)wv[u][i].x, (uint32_t)wv[u][i].z, false, false);
                const auto s13 = __builtin_amdgcn_permlane32_swap((uint32_t)wv[u][i].y, (uint32_t)wv[u][i].w, false, false);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int b = 2 * i + h;
                    const u32x4 x = *reinterpret_cast<const u32x4*>(hb + 64 * b + ko);
                    const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 D4 = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8, x),
                                                        i8x8_to_bf16x8(s02[h], s13[h]), zf);
                    const float dsc = h2f((uint16_t)(h ? (sc[u][i] >> 16) : (sc[u][i] & 0xffffu)));
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] = fmaf(dsc, D4[v], acc[v]);
                }
            }
            // result row 8 (lanes 32..47, v = 0) holds the lo part: add it to row 0 (lanes 0..15)
            const float tot = acc[0] + lane_xor32f(acc[0]);     // lanes < 32: l + 32
            if (on[u] && lane < 16) rr[j0 + NWV * u][j] = tot;
        }
        // the next round overwrites this wave's hs slot: every lane's reads come first
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();
    if (wave == 0 && lane < 16 && r0 + lane < D) {
        float v = 0.f;
        if (ok) {
            for (int jj = 0; jj < topk; ++jj) v = fmaf(a.w[t * topk + jj], rr[jj][lane], v);
        }
        a.out[(size_t)t * D + r0 + lane] = f2bf_bits(v);
    }
}

__global__ void __launch_bounds__(256) moe_combine_kernel(MoeArgs a) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= a.T * a.D) return;
    const int t = i / a.D, m = i - t * a.D;
    float v = 0.f;
    if (a.plan[0] >= 0) {
        for (int j = 0; j < a.topk; ++j)
            v = fmaf(a.w[t * a.topk + j], a.rows[(size_t)(t * a.topk + j) * a.D + m], v);
    }
    a.out[i] = f2bf_bits(v);
}

// plan | h [P][F] | rows [P][D] | q8_1 of a bf16 input: quants [T][D], scales [T][D/32]
size_t moe_workspace_bytes(int T, int topk, int D, int F) {
    const size_t P = (size_t)T * topk;
    return round_up((1 + 4 * P) * sizeof(int32_t), kCounterAlign) +
           round_up(P * F * sizeof(float), kCounterAlign) + round_up(P * D * sizeof(float), kCounterAlign) +
           round_up((size_t)T * D, kCounterAlign) + round_up((size_t)T * (D / 32) * sizeof(uint16_t), kCounterAlign);
}

template <int NL, bool HQ>
static void launch_down_token(const MoeArgs& a, bool tl, hipStream_t st) {
    const dim3 gt((a.D + 15) / 16, a.T);
    if (tl) hipLaunchKernelGGL((moe_down_token_kernel<NL, HQ, true>), gt, dim3(64 * kMoeDnWaves), 0, st, a);
    else hipLaunchKernelGGL((moe_down_token_kernel<NL, HQ, false>), gt, dim3(64 * kMoeDnWaves), 0, st, a);
}

int launch_moe_routed(const int8_t* xq, const uint16_t* xd, const uint16_t* xb, const int32_t* ids,
                      const float* w, const void* wgu, const void* wdn, uint16_t* out, int T,
                      int topk, int E, int D, int F, bool hq, bool tl, void* ws, hipStream_t st) {
    if ((hq || tl) && ((F != 256 && F != 512 && F != 1024) || topk > kMoeMaxTopk)) return GQ8_ESHAPE;
    if (tl && D % 16 != 0) return GQ8_ESHAPE;
    if (F % 8 != 0) return GQ8_ESHAPE;     // the gate/up rows kernel's waves take whole row pairs
    MoeArgs a{};
    a.xq = xq; a.xd = xd; a.xb = xb; a.w = w;
    a.wgu = static_cast<const int8_t*>(wgu);
    a.wdn = static_cast<const int8_t*>(wdn);
    a.gu_bytes = (size_t)2 * F * D + (size_t)2 * F * (D / 32) * 2;
    a.dn_bytes = (size_t)D * F + (size_t)D * (F / 32) * 2;
    a.out = out; a.T = T; a.topk = topk; a.P = T * topk; a.E = E; a.D = D; a.F = F;
    const size_t P = (size_t)a.P;
    char* p = static_cast<char*>(ws);
    int32_t* plan = reinterpret_cast<int32_t*>(p);
    a.plan = plan;
    p += round_up((1 + 4 * P) * sizeof(int32_t), kCounterAlign);
    a.h = reinterpret_cast<float*>(p);
    p += round_up(P * F * sizeof(float), kCounterAlign);
    a.rows = reinterpret_cast<float*>(p);
    p += round_up(P * D * sizeof(float), kCounterAlign);
    a.ids = ids;
    int rc = GQ8_OK;
    const bool general = force_general();
    const bool rows_gu = D <= 4096 && !general;
    if (xb != nullptr && !rows_gu) {       // bf16 input, general gate/up kernel: quantize first
        int8_t* wq = reinterpret_cast<int8_t*>(p);
        uint16_t* wd = reinterpret_cast<uint16_t*>(p + round_up((size_t)T * D, kCounterAlign));
        if ((rc = launch_q8_1_quantize(xb, T, D, wq, wd, nullptr, st)) != GQ8_OK) return rc;
        a.xq = wq; a.xd = wd; a.xb = nullptr;
    }
    // the plan is needed only by the fallback kernels (D > 4096 gate/up; F outside
    // {256, 512, 1024} down)
    // (the q8_1(h) down read and the tiled down weights exist only as the token kernel: the switch
    // leaves them there)
    // (the token kernel keeps one result row per slot in LDS: at most kMoeMaxTopk slots)
    const bool token_dn = (F == 256 || F == 512 || F == 1024) && topk <= kMoeMaxTopk && (!general || hq || tl);
    if (!rows_gu || !token_dn) {
        GQ8_NOTE_GENERAL("routed experts: plan-based general kernels: D > 4096, F not in {256, 512, 1024}, or forced");
        hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(256), 0, st, ids, a.P, E, plan);
        if ((rc = launch_status()) != GQ8_OK) return rc;
    }
    const dim3 ggu((F + 4 * kGuRpw - 1) / (4 * kGuRpw), a.P);
    if (!rows_gu) {                        // the general gate/up kernel (a.xb is q8_1 by now)
        if (T <= 4) hipLaunchKernelGGL((moe_gate_up_kernel<4>), ggu, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((moe_gate_up_kernel<16>), ggu, dim3(256), 0, st, a);
    } else if (a.xb != nullptr) {
        if (D <= 1024) hipLaunchKernelGGL((moe_gate_up_rows_kernel<1, true>), ggu, dim3(256), 0, st, a);
        else if (D <= 2048) hipLaunchKernelGGL((moe_gate_up_rows_kernel<2, true>), ggu, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((moe_gate_up_rows_kernel<4, true>), ggu, dim3(256), 0, st, a);
    }
    else if (D <= 1024) hipLaunchKernelGGL((moe_gate_up_rows_kernel<1, false>), ggu, dim3(256), 0, st, a);
    else if (D <= 2048) hipLaunchKernelGGL((moe_gate_up_rows_kernel<2, false>), ggu, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((moe_gate_up_rows_kernel<4, false>), ggu, dim3(256), 0, st, a);
    if ((rc = launch_status()) != GQ8_OK) return rc;
    if (token_dn) {                        // down + combine in one kernel
        if (hq) {
            if (F == 256) launch_down_token<4, true>(a, tl, st);
            else if (F == 512) launch_down_token<8, true>(a, tl, st);
            else launch_down_token<16, true>(a, tl, st);
        } else {
            if (F == 256) launch_down_token<4, false>(a, tl, st);
            else if (F == 512) launch_down_token<8, false>(a, tl, st);
            else launch_down_token<16, false>(a, tl, st);
        }
        return launch_status();
    }
    const int rps = 64 / (F / 16);
    const dim3 gdn((D + 4 * kDnNrs * rps - 1) / (4 * kDnNrs * rps), a.P);
    hipLaunchKernelGGL((moe_down_kernel<4>), gdn, dim3(256), (size_t)4 * kDnNrs * 64 * 4 * sizeof(float), st, a);
    if ((rc = launch_status()) != GQ8_OK) return rc;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((T * D + 255) / 256), dim3(256), 0, st, a);
    return launch_status();
}

}  // namespace gq8
