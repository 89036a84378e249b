// Host-side internals shared by the gq8 translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdio.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gq8.h"

#define GQ8_EXPORT extern "C" __attribute__((visibility("default")))

// A shape outside the tuned set runs the general kernels of the same family (correct, slower):
// said once per process and call site on stderr.
#define GQ8_NOTE_GENERAL(msg)                                                                   \
    do {                                                                                        \
        static std::atomic<bool> said_{false};                                                  \
        if (!said_.exchange(true)) fprintf(stderr, "gq8: %s\n", msg);                            \
    } while (0)

namespace gq8 {

// Debug switch GQ8_FORCE_GENERIC: "1" sends every call to the general kernels of its family (the
// paths a shape outside the tuned set takes), so that tests can check them at the tuned shapes;
// unset or "0": off; any other value: off, said once on stderr. Read on every call.
bool force_general();

constexpr int kMaxT = 16;        // token rows of the Q8_0 reads
constexpr int kMaxM = 32;        // rows of the W8A8 product
constexpr int kW8MaxK = 8192;    // W8A8 depth: 16 waves x 8 k-steps of 64
constexpr size_t kCounterAlign = 256;

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch status -> gq8 status (clears the sticky launch error).
inline int launch_status() { return hipGetLastError() == hipSuccess ? GQ8_OK : GQ8_EHIP; }

// CU count of the current device (cached per device id). 0 when there is no device.
int device_cus();

// ---------------------------------------------------------------- Q8_0 read family

struct GemvArgs {
    const int8_t* q;        // split layout: quants [N][K]
    const uint16_t* d;      //               scales [N][K/32] (fp16 bits)
    const void* x;          // fp32 [T][K] (GEMV), bf16 R [T][K] (down), bf16 lo [T][K] (up)
    const uint16_t* wnorm;  // bf16 [K] (down)
    int T, N, K;
    int S;                  // down: K slabs
    float* part;            // down: [S][T][N] fp32 partial sums
    float* ssq;             // down: [S][T] partial sums of squares
    void* out;              // fp32 y [T][N] or bf16 [T][N]
    float* rs_out;          // fp32 [T] (down, nullable)
    float eps;
    void* lo_out;           // fused pair: bf16 [T][K] down output written by work-group 0
    int kd;                 // fused pair: depth of the down read (the RMS mean's divisor)
    unsigned* cnt;          // last-arriver combine: one arrival counter per 64-row group
    const uint16_t* pw;     // down read with the pending write: bf16 P [T][K] ...
    uint16_t* r_out;        //   ... and R_out = bf16(R + P) [T][K], the stream the read takes
    const int8_t* pfq;      // pair, whole-row down read: the up read's quants and scales, pf_n
    const uint16_t* pfd;    //   rows of pf_k columns, which extra work-groups of the down read
    int pf_n, pf_k;         //   fetch ahead into the caches (hc_down_rows_kernel)
    bool wt;                // up read: quants in the tiled layout (launch_q8_0_tile16; N % 16 == 0,
                            //   K % 320 == 0: the direct and fused up kernels only)
};

// Combine of split partial sums: a kernel of its own (default), or the last-arriving work-group
// of each row group (GQ8_COMBINE=last, read on every call; other values: default, said once).
bool combine_last_arriver();

// Q8_0 GEMV (fp32 x): T < 5 one work-group per RW rows and all of K on the VALU, no workspace;
// T >= 5 MFMA over 512-column slabs into S partial planes [S][T][N] (the workspace), then a
// combine kernel.
int launch_q8_0_gemv(GemvArgs a, void* ws, hipStream_t st);
size_t gemv_workspace_bytes(int T, int N, int K);

// fused RMSNorm + Q8_0 down read: MFMA partial kernel over K slabs, then a combine kernel.
constexpr int kDownSlab = 512;                 // columns per slab (16 Q8_0 blocks)
inline int hc_down_slabs(int K) { return (K + kDownSlab - 1) / kDownSlab; }
size_t hc_down_workspace_bytes(int T, int N, int K);
size_t hc_down_counter_bytes(int N);                 // counters at the workspace's start (down, pair)
size_t gemv_counter_bytes(int T, int N, int K);      // the GEMV's (T >= 5), 0 otherwise
int launch_hc_down(GemvArgs a, void* ws, hipStream_t st);
// the down read (a.pw, a.r_out set) and the pair with the pending write folded into the staging
int launch_hc_down_pending(GemvArgs a, void* ws, hipStream_t st);
int launch_hc_pair_pending(GemvArgs dn, GemvArgs up, void* ws, hipStream_t st);

// Q8_0 up read (bf16 x, K <= 1024): MFMA, one wave per 16 output rows, no workspace.
int launch_hc_up(GemvArgs a, hipStream_t st);

// the down read then the up read on its output; for an up depth of 320 and T <= 4 the down's
// combine runs inside the up kernel (two launches instead of three). dn.out = lo (bf16 [T][dn.N]).
int launch_hc_pair(GemvArgs dn, GemvArgs up, void* ws, hipStream_t st);

// the same pair on BF16 weights (q = the bf16 weight bytes, d unused): the comparison read
int launch_hc_bf16_pair(GemvArgs dn, GemvArgs up, void* ws, hipStream_t st);

// ---------------------------------------------------------------- W8A8

// The W8A8 kernel: int8 MFMA at every M by default; GQ8_W8A8_KERNEL=dot forces the VALU dot4
// kernel where it exists (M <= 15), "mfma" the default (read on every call; other values: the
// default, said once). int32 sums are exact, so both give bitwise the same results. Returns 0
// default, 1 dot, 2 mfma.
int w8a8_kernel_choice();

struct W8Plan {
    bool mfma;         // int8 MFMA path (the default) or VALU dot4 path (forced, M <= 15)
    int ntiles;        // N rounded up to 16, / 16: one work-group each
    int ksteps;        // K rounded up to 64, / 64
    int nw;            // waves per work-group (<= 16)
    int kpw;           // k-steps per wave
    bool half;         // MFMA path, M <= 16, few tiles: two work-groups of 8 columns per tile
};
W8Plan plan_w8a8(int M, int N, int K);
// xb != nullptr: bf16 x quantized per token inside the kernel (xq, xs unused; bf16x_fused(M, K));
// xq_out / xs_out (nullable) receive the quantized x from work-group 0. Each work-group
// re-quantizes all of x, which pays while x is small (measured: up to 16384 values).
constexpr int kFusedBf16xM = 8;
constexpr int kFusedBf16xElems = 16384;
inline bool bf16x_fused(int M, int K) { return M <= kFusedBf16xM && M * K <= kFusedBf16xElems; }
int launch_w8a8(const W8Plan& p, const int8_t* xq, const float* xs, const int8_t* wp,
                const float* ws_scale, void* out, bool i32_out, int M, int N, int K, hipStream_t st,
                const uint16_t* xb = nullptr, int8_t* xq_out = nullptr, float* xs_out = nullptr);
int launch_per_token_quantize(const uint16_t* x, int M, int K, int8_t* xq, float* xs, hipStream_t st);

// ---------------------------------------------------------------- small kernels

int launch_fill_zero(void* p, size_t bytes, hipStream_t st);
int launch_q8_0_quantize(const float* w, int rows, int K, void* w_split, hipStream_t st);
int launch_q8_0_split_from_blocks(const void* b34, int rows, int K, void* w_split, hipStream_t st);
int launch_q8_1_quantize(const uint16_t* x, int rows, int K, int8_t* q, uint16_t* d, uint16_t* s,
                         hipStream_t st);
int launch_w8a8_pack(const int8_t* W, int K, int N, int8_t* Wp, hipStream_t st);
int launch_q8_0_tile16(const void* w_split, int rows, int K, int count, void* w_tiled, hipStream_t st);
int launch_read_probe(const void* src, size_t bytes, float* sink, hipStream_t st);
int launch_read_probe_ex(const void* src, size_t bytes, float* sink, int lpt, int threads,
                         int work_groups, bool nt, hipStream_t st);
size_t read_probe_blocks(size_t bytes);

// ---------------------------------------------------------------- MoE

int launch_moe_route(const float* logits, int T, int E, int topk, int32_t* ids, float* w,
                     hipStream_t st);
int launch_moe_plan(const int32_t* ids, int T, int topk, int E, int32_t* plan, hipStream_t st);
size_t moe_workspace_bytes(int T, int topk, int D, int F);
// xb != nullptr: bf16 input quantized to q8_1 on the device (xq, xd unused); hq: the down read
// takes q8_1(h) (F in {256, 512, 1024}, else GQ8_ESHAPE)
// tl: the down weights are in the tiled layout (launch_q8_0_tile16; D % 16 == 0, F in {256, 512,
// 1024}, topk <= 16: the token kernel reads them, whatever GQ8_FORCE_GENERIC says)
int launch_moe_routed(const int8_t* xq, const uint16_t* xd, const uint16_t* xb, const int32_t* ids,
                      const float* w, const void* wgu, const void* wdn, uint16_t* out, int T,
                      int topk, int E, int D, int F, bool hq, bool tl, void* ws, hipStream_t st);

}  // namespace gq8
