/*
 * gq8 -- decode-time skinny quantized matrix products on MI355X (gfx950).
 *
 * C ABI of libgq8.so. Plain pointers and sizes only. Unless a parameter says
 * otherwise, every pointer is DEVICE memory owned by the caller (for example
 * a torch tensor's data_ptr()); the library never keeps a pointer past the
 * call, never allocates, and never synchronizes. `stream` is a hipStream_t
 * (0 = the legacy null stream); every call only enqueues work on it, so the
 * compute entry points can be captured into a hipGraph.
 *
 * Return value: GQ8_OK (0) or a negative gq8_status. Arguments are checked
 * before anything is enqueued; on an error nothing has been launched and the
 * outputs are untouched. A HIP launch failure is reported as GQ8_EHIP.
 *
 * Buffers: an output may not overlap any input, another output or the
 * workspace (the kernels assume no aliasing). Threads: every entry point may
 * be called from several host threads at once; the only state the library
 * keeps is a per-device cache of the compute-unit count and once-per-process
 * notes on stderr. Calls that can run at the same time (other streams) need
 * workspaces of their own.
 *
 * Size limits, far above decode-time shapes, beyond which a call returns
 * GQ8_ESHAPE (they keep every launch under 2^32 work-items and the index
 * arithmetic in range): Q8_0 reads N <= 2^21 output rows, K <= 2^24 and
 * N*K <= 2^36; W8A8 N <= 2^24; routed experts D <= 2^20; the top-k and the
 * per-token quantizer at most 2^23 rows (per-token K <= 2^24); the
 * quantizers and the packer at most 2^32 - 256 blocks, slots or 16-byte
 * pieces; the read probe at most that many 16-byte pieces.
 *
 * Pages cited (by title and section):
 *   HC-Q8 page  "sycl: STRATA_HC_Q8=1 reads the Q8_0 hyper-connection projections" (PR #2810)
 *   EP page     "sycl: --expert-parallel-device N, two Arc cards compute each layer's experts together" (PR #1798)
 *   defer page  "verify: STRATA_VERIFY_DEFER_CPU_BELOW=<w>" (PR #2690)
 *   W8A8 page   "INT8 W8A8 GEMM -- Decode (M <= 32) -- gfx928 / SGLang TP4"
 */
#ifndef GQ8_H
#define GQ8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQ8_ABI_VERSION 3

enum gq8_status {
    GQ8_OK = 0,
    GQ8_EINVAL = -1,     /* null pointer, negative size, unknown op                     */
    GQ8_ESHAPE = -2,     /* a size outside what the operation supports                   */
    GQ8_EALIGN = -3,     /* a pointer not aligned as the operation requires (16 bytes)   */
    GQ8_EWORKSPACE = -4, /* workspace null or smaller than gq8_workspace_bytes()         */
    GQ8_ECAPTURE = -5,   /* gq8_workspace_init() called on a capturing stream            */
    GQ8_EHIP = -6,       /* a HIP call or kernel launch failed                           */
    GQ8_ENODEV = -7      /* no usable gfx950 device is current                           */
};

/* Operations that take a workspace (the `op` argument of the workspace functions). */
enum gq8_op {
    GQ8_OP_Q8_0_GEMV = 1,
    GQ8_OP_HC_DOWN = 2,
    GQ8_OP_HC_UP = 3,
    GQ8_OP_W8A8 = 4,
    GQ8_OP_HC_PAIR = 5,    /* rows = T, N = Nlr, K = Khc of gq8_hc_q8_pair */
    GQ8_OP_W8A8_BF16X = 6  /* rows = M of gq8_w8a8_gemm_bf16x */
};

/* Static string for a status code. Host only. */
const char* gq8_status_str(int status);

/* GQ8_ABI_VERSION of the built library. Host only. */
int gq8_abi_version(void);

/* Compute units of the current device (the split-K sizing uses it); GQ8_ENODEV without one. */
int gq8_device_cus(int* cus_out);

/* ------------------------------------------------------------------------------------------
 * Q8_0 weights (HC-Q8 page, "What changed": blocks of 32 int8 quants with one fp16 scale,
 * ggml's 34-byte blocks, and the "split" order the read uses).
 *
 * Split layout of a [rows, K] Q8_0 matrix (K % 32 == 0), gq8_q8_0_bytes(rows, K) bytes:
 *   int8 q[rows][K]            every row's quants, row-major
 *   fp16 d[rows][K/32]         then every row's block scales, row-major
 * The scales start at byte offset rows*K. The buffer must be 16-byte aligned.
 * ------------------------------------------------------------------------------------------ */
size_t gq8_q8_0_bytes(int64_t rows, int64_t K);

/* Quantize fp32 rows w[rows][K] into the split layout (HC-Q8 page, "What changed": ggml's
 * rounding). Per block: d = fp16(amax / 127) (fp32 quotient, round to nearest even);
 * q = round(w / d) with the fp32 quotient by the stored fp16 d, ties away from zero, clamped to
 * [-127, 127]; a block whose fp16 d is 0 gets zero quants. Weight preparation, not a hot-path
 * call. w: 16-byte aligned, finite (a block holding an infinity or a NaN gets unspecified
 * quants); K % 32 == 0. */
int gq8_q8_0_quantize(const float* w, int rows, int K, void* w_split, void* stream);

/* Reorder ggml 34-byte blocks {fp16 d; int8 q[32]} (row-major blocks, [rows][K/32]) into the
 * split layout: the same bytes, reordered (HC-Q8 page, "What changed"). */
int gq8_q8_0_split_from_blocks(const void* blocks34, int rows, int K, void* w_split, void* stream);

/* Tiled layout, for the routed down weights (gq8_moe_q8_0_routed_flags, GQ8_MOE_DOWN_TILED) and
 * the up read's weights:
 * `count` split-layout matrices [rows][K] stored back to back (each gq8_q8_0_bytes(rows, K)
 * bytes, e.g. an expert arena) are copied to w_tiled, each matrix at the same offset and of the
 * same size, with its scales unchanged and its quants reordered into 1 KiB tiles: tile (G, c)
 * of row group G (16 rows) and column group c (64 columns) sits at byte (G * K/64 + c) * 1024,
 * and its 16-byte piece l (l < 64) is row 16G + l%16, columns 64c + 16(l/16) .. +16. These are
 * the 16 bytes that lane l of the routed down read's MFMA tile takes for that row and column
 * group, so a tile is one contiguous 1 KiB load instead of sixteen 64-byte row pieces. Weight
 * preparation, not a hot-path call (the layout is a choice for MI355X; the pages' blocks hold
 * the same bytes). rows % 16 == 0, K % 64 == 0 (else GQ8_ESHAPE); both buffers 16-byte
 * aligned (GQ8_EALIGN) and not overlapping (GQ8_EINVAL); count == 0, rows == 0 or K == 0: no
 * work. The up read takes the same layout (gq8_hc_q8_up_tiled, gq8_hc_q8_pair_tiled). */
int gq8_q8_0_tile16(const void* w_split, int rows, int K, int count, void* w_tiled, void* stream);

/* q8_1 quantization of bf16 rows x[rows][K] (EP page, "What changed": the q8_1 MoE input).
 * Per 32-block, the Q8_0 rule above plus s = fp16(d * sum(q)).
 * Outputs: q int8 [rows][K], d fp16 [rows][K/32], s fp16 [rows][K/32] (s may be null). */
int gq8_q8_1_quantize(const uint16_t* x_bf16, int rows, int K, int8_t* q, uint16_t* d,
                      uint16_t* s, void* stream);

/* Host-side preparation: the same three operations on host memory in plain C++ (no device,
 * stream or HIP call), for loaders that prepare weights before upload (HC-Q8 page, "What
 * changed": the loader quantizes a BF16 tensor to Q8_0 at load and uploads the split layout).
 * Byte-identical to gq8_q8_0_quantize, gq8_q8_0_split_from_blocks and gq8_q8_1_quantize.
 * Errors: GQ8_EINVAL (negative size, null pointer), GQ8_ESHAPE (K % 32 != 0). */
int gq8_q8_0_quantize_host(const float* w, int rows, int K, void* split_out);
int gq8_q8_0_split_from_blocks_host(const void* blocks34, int rows, int K, void* split_out);
int gq8_q8_1_quantize_host(const uint16_t* x_bf16, int rows, int K, int8_t* q, uint16_t* d,
                           uint16_t* s);
/* The W8A8 weight packer on the host: byte-identical to gq8_w8a8_pack (W int8 [K][N] row-major,
 * W_packed gq8_w8a8_packed_bytes(K, N) bytes). K % 16 == 0. */
int gq8_w8a8_pack_host(const int8_t* W, int K, int N, int8_t* W_packed);

/* ------------------------------------------------------------------------------------------
 * Workspace: device scratch that a compute call needs beyond its inputs and outputs.
 *   - size it with gq8_workspace_bytes() for the exact (op, rows, N, K) of the call; 0 means the
 *     call needs none (pass NULL, 0). The down read and the down/up pair use one (one 32-bit
 *     arrival counter per 64-row group first, then the fp32 partial sums of the K slabs
 *     [S][T][N], then the slabs' sums of squares per row group [G][S][T]), and so does the GEMV
 *     at T >= 5 (the counters, then the partial sums) (HC-Q8 page, "What changed": one scratch
 *     per queue, allocated and zeroed outside any capture);
 *   - the partial sums are combined in a fixed order either by a kernel of their own (the
 *     default) or by the last-arriving work-group of each row group (environment variable
 *     GQ8_COMBINE=last, read on every call; "kernel" or unset: the default; other values: the
 *     default, said once on stderr). The results are bitwise the same. The last-arriver combine
 *     (HC-Q8 page, "What changed"; W8A8 page, "Split-K requirements") counts arrivals in the
 *     counters, which must be zero before a call and which every complete call leaves at zero:
 *     zero a new workspace once with gq8_workspace_init(); the partial sums themselves are always
 *     rewritten before they are read (W8A8 page, "Split-K requirements": planes fully rewritten,
 *     no memset in the timed region). The counters open the workspace and take
 *     gq8_workspace_counter_bytes() bytes, 256 for every N <= 4096, so one zeroed workspace
 *     serves calls of any shapes it is large enough for; only a call whose counter region is
 *     larger than every earlier call's since the zeroing (N > 4096 growing) needs it zeroed again;
 *   - calls that may run concurrently (different streams, or a graph replayed concurrently with
 *     itself) need separate workspaces;
 *   - gq8_workspace_counter_bytes() is the size of the counter region at the start of the
 *     workspace (0 when the operation has none).
 * rows = T for the Q8_0 calls, M for W8A8.
 * ------------------------------------------------------------------------------------------ */
size_t gq8_workspace_bytes(int op, int rows, int N, int K);
size_t gq8_workspace_counter_bytes(int op, int rows, int N, int K);
int gq8_workspace_init(void* ws, size_t bytes, void* stream);
/* Debug check of a workspace's arrival counters: *nonzero_counters = the number of non-zero 32-bit
 * words in the counter region of a workspace sized for (op, rows, N, K) (0 after any complete
 * call; non-zero means a call was interrupted or the workspace was not zeroed). Copies the region
 * to the host and synchronizes the stream; 0 without a read when the operation has no counters.
 * Errors: GQ8_EINVAL (null nonzero_counters), GQ8_EWORKSPACE (ws null or smaller than
 * gq8_workspace_bytes), GQ8_ECAPTURE (capturing stream), GQ8_EHIP. */
int gq8_workspace_check(int op, int rows, int N, int K, const void* ws, size_t bytes, void* stream,
                        int* nonzero_counters);

/* Q8_0 matrix-vector product for T = 1..16 token rows (HC-Q8 page, "What changed": w = d*q,
 * exact in fp32):
 *   y[t][n] = sum_k d[n][k/32] * q[n][k] * x[t][k]
 * w_split: split-layout Q8_0 [N][K]; x fp32 [T][K]; y fp32 [T][N] (written, not accumulated).
 * K % 32 == 0. Accumulation is fp32 in a fixed order: the result is deterministic for a given
 * device and shape (replays are bitwise identical). T == 0 or N == 0: nothing to do.
 * K == 0: y is zero-filled. T <= 4: VALU dots, one kernel, no workspace. T >= 5: bf16 MFMA on
 * x split into bf16 hi + lo (|x - hi - lo| <= 2^-17 |x|) over 256-column slabs, then a combine
 * of the slab sums in a fixed order (a kernel, or the last-arriving work-group: see Workspace);
 * workspace gq8_workspace_bytes(GQ8_OP_Q8_0_GEMV, T, N, K), its counters zeroed once. */
int gq8_q8_0_gemv(const void* w_split, const float* x, float* y, int T, int N, int K,
                  void* ws, size_t ws_bytes, void* stream);

/* Fused RMSNorm + Q8_0 hyper-connection down read (HC-Q8 page, "What changed": the down kernel
 * works on R * w_norm unscaled plus the slab's sums of squares, and the RMSNorm factor is applied
 * when the slabs' partial sums are combined, in a fixed order):
 *   rs[t]    = 1 / sqrt(mean_k R[t][k]^2 + eps)
 *   lo[t][n] = bf16( rs[t] * sum_k d[n][k/32] * q[n][k] * (R[t][k] * w_norm[k]) )
 * w_split: Q8_0 [N][K]; R bf16 [T][K]; w_norm bf16 [K]; lo bf16 [T][N]; rs_out fp32 [T]
 * (nullable). T = 1..16, K % 32 == 0, K > 0; T == 0 or N == 0: nothing to do (rs_out is not
 * written either). Workspace: gq8_workspace_bytes(GQ8_OP_HC_DOWN, T, N, K), its counters zeroed
 * once. T = 1: one kernel, each work-group owning two whole rows over all of K (fp32 VALU dots,
 * rs from the work-group's own sum of squares, the same in every work-group); the workspace is
 * passed but not touched. T >= 2: two kernels, per 512-column slab partial sums (bf16 MFMA on
 * exact hi/lo operands), then the combine (slab groups in ascending order) with rs and the bf16
 * rounding; with GQ8_COMBINE=last and T <= 8 one kernel, whose last-arriving work-group per row
 * group combines in the same order. */
int gq8_hc_q8_down(const void* w_split, const uint16_t* R, const uint16_t* w_norm, float eps,
                   uint16_t* lo, float* rs_out, int T, int N, int K,
                   void* ws, size_t ws_bytes, void* stream);

/* Q8_0 hyper-connection up read (HC-Q8 page, "What changed": rows of K = 320, the fifths of each
 * row summed in a fixed order). The page's own epilogue (pending write, gate, stream mean) is
 * not defined there and is not part of this call:
 *   out[t][n] = bf16( sum_k d[n][k/32] * q[n][k] * lo[t][k] )
 * w_split: Q8_0 [N][K]; lo bf16 [T][K]; out bf16 [T][N]. T = 1..16, K % 32 == 0, K <= 1024. */
int gq8_hc_q8_up(const void* w_split, const uint16_t* lo, uint16_t* out, int T, int N, int K,
                 void* ws, size_t ws_bytes, void* stream);

/* The down read followed by the up read on its output (HC-Q8 page, "What changed": the down and
 * up projections of one hyper-connection read), in one call:
 *   lo  = gq8_hc_q8_down(w_down [Nlr][Khc], R [T][Khc], w_norm [Khc])     bf16 [T][Nlr]
 *   out = gq8_hc_q8_up(w_up [Khc][Nlr], lo)                                bf16 [T][Khc]
 * lo, rs_out and out are bitwise what the two separate calls produce. For Nlr == 320 and
 * 2 <= T <= 4 the down read's combine of its split partial sums runs inside the up kernel (two
 * kernel launches instead of three); otherwise (T = 1: the whole-row down kernel, no combine)
 * the two calls' kernels run in sequence. For Nlr == 320 and T = 1 the down kernel's launch
 * also reads w_up once into the caches ahead of the up read (up to 65536 rows of w_up); no
 * result depends on it. lo is written (bf16
 * [T][Nlr], 16-byte aligned, required); rs_out fp32 [T] is nullable. T = 1..16, Khc % 32 == 0,
 * Nlr % 32 == 0, 0 < Nlr <= 1024. Workspace: gq8_workspace_bytes(GQ8_OP_HC_PAIR, T, Nlr, Khc). */
int gq8_hc_q8_pair(const void* w_down, const uint16_t* R, const uint16_t* w_norm, float eps,
                   const void* w_up, uint16_t* lo, float* rs_out, uint16_t* out,
                   int T, int Nlr, int Khc, void* ws, size_t ws_bytes, void* stream);

/* gq8_hc_q8_up and gq8_hc_q8_pair with the up weights in the tiled layout (gq8_q8_0_tile16 with
 * rows = N (Khc for the pair), K = the up depth (Nlr), count = 1): the up read's 16-row tiles are
 * then contiguous 1 KiB loads instead of sixteen 64-byte row pieces each. The results are bitwise
 * those of the calls on the split layout. Needs N % 16 == 0 and an up depth that is a multiple
 * of 320 (the up kernels that read whole 320-column chunks), else GQ8_ESHAPE; everything else
 * (shapes, workspace, errors) as the split-layout calls. Weight preparation (the tiling) is
 * outside the hot path; the layout is a choice for MI355X. */
int gq8_hc_q8_up_tiled(const void* w_tiled, const uint16_t* lo, uint16_t* out, int T, int N, int K,
                       void* ws, size_t ws_bytes, void* stream);
int gq8_hc_q8_pair_tiled(const void* w_down, const uint16_t* R, const uint16_t* w_norm, float eps,
                         const void* w_up_tiled, uint16_t* lo, float* rs_out, uint16_t* out,
                         int T, int Nlr, int Khc, void* ws, size_t ws_bytes, void* stream);

/* The down read and the pair with the pending write folded in (HC-Q8 page, "Summary": R_out, the
 * pending write between the two reads, bitwise the default read's; the page does not define it
 * further, and this is a reading of it): a pending residual update P is added to the stream
 * before the down read,
 *   R_out[t][k] = bf16( R[t][k] + P[t][k] )    (fp32 sum of the two bf16 values, round to nearest even)
 * and the RMSNorm and the down read take R_out in place of R; lo, rs_out and out are then what
 * gq8_hc_q8_down / gq8_hc_q8_pair give on R_out (bitwise). P and R_out bf16 [T][K] (K = Khc),
 * 16-byte aligned; R_out may not overlap R or P. The up read's own epilogue on the page (gate,
 * stream mean) is not defined there and not part of these calls. Shapes, workspace and errors as
 * the calls without the pending write, except that N == 0 returns GQ8_ESHAPE (the write is done
 * by the down read's work-groups); at T >= 2 the partial sums are combined by the combine kernel. */
int gq8_hc_q8_down_pending(const void* w_split, const uint16_t* R, const uint16_t* P,
                           const uint16_t* w_norm, float eps, uint16_t* R_out, uint16_t* lo,
                           float* rs_out, int T, int N, int K, void* ws, size_t ws_bytes,
                           void* stream);
int gq8_hc_q8_pair_pending(const void* w_down, const uint16_t* R, const uint16_t* P,
                           const uint16_t* w_norm, float eps, const void* w_up, uint16_t* R_out,
                           uint16_t* lo, float* rs_out, uint16_t* out, int T, int Nlr, int Khc,
                           void* ws, size_t ws_bytes, void* stream);

/* gq8_hc_q8_pair without a workspace argument, for callers that cannot allocate memory (code
 * under hipGraph capture that may not call hipMalloc, allocation-free serving loops, harnesses
 * that forbid allocation): the workspace is a fixed device array inside the library, of
 * GQ8_NOALLOC_SCRATCH_BYTES, one per device, held until the process ends. The call itself
 * allocates nothing. Inputs, outputs, shapes and results are those of gq8_hc_q8_pair (bitwise);
 * a shape whose workspace, gq8_workspace_bytes(GQ8_OP_HC_PAIR, T, Nlr, Khc), exceeds the array
 * returns GQ8_ESHAPE (T = 16, Nlr = 320, Khc = 16384 needs 642 KiB; at T = 16 and Nlr = 1024,
 * Khc up to 32256 fits). Every call on one device shares that device's array, which keeps the
 * last call's contents. Nothing needs clearing: the array starts zeroed, every call writes the
 * partial sums before it reads them, and the one part that must be zero before a call, the
 * 256-byte block of arrival counters at its start (read only with GQ8_COMBINE=last; 256 bytes
 * for every pair shape), is left at zero by every complete call. Calls that may run at the same
 * time on one device (several streams, host threads or concurrent graph replays) race and must
 * not overlap. GQ8_EHIP if the array's device address cannot be obtained. */
#define GQ8_NOALLOC_SCRATCH_BYTES (4u << 20)
int gq8_hc_q8_pair_noalloc(const void* w_down, const uint16_t* R, const uint16_t* w_norm, float eps,
                           const void* w_up, uint16_t* lo, float* rs_out, uint16_t* out, int T,
                           int Nlr, int Khc, void* stream);

/* The same pair on BF16 weights: the read the Q8_0 pair replaces (HC-Q8 page, "Summary": the
 * kernel-level BF16 -> Q8_0 read times), kept as an in-library comparison read measured with the
 * same harness. w_down bf16 [Nlr][Khc] and w_up bf16 [Khc][Nlr], row-major, 16-byte aligned; every
 * other argument, the shapes, the workspace (gq8_workspace_bytes(GQ8_OP_HC_PAIR, T, Nlr, Khc)),
 * lo, rs_out and the errors are as in gq8_hc_q8_pair; lo and out are within the same pass rule
 * of the BF16 oracle reads. */
int gq8_hc_bf16_pair(const uint16_t* w_down, const uint16_t* R, const uint16_t* w_norm, float eps,
                     const uint16_t* w_up, uint16_t* lo, float* rs_out, uint16_t* out, int T,
                     int Nlr, int Khc, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * W8A8 (W8A8 page, operator statement): int8 x_q[M][K] @ int8 W[K][N] -> int32, then
 * * x_scale[M] * w_scale[N] -> bf16[M][N], M = 1..32.
 * The weight is packed once, outside the timed path (W8A8 page, "Cross-shape rules": pack the
 * cold weight into the fragment layout): gq8_w8a8_pack() turns the logical row-major W[K][N]
 * into an opaque layout of gq8_w8a8_packed_bytes(K, N) bytes (N rounded up to 16 and K to 64,
 * padding zero-filled). K % 16 == 0; x_q rows are K bytes, 16-byte aligned.
 * ------------------------------------------------------------------------------------------ */
size_t gq8_w8a8_packed_bytes(int K, int N);
int gq8_w8a8_pack(const int8_t* W, int K, int N, int8_t* W_packed, void* stream);

/* out[m][n] = bf16( (fp32(acc[m][n]) * x_scale[m]) * w_scale[n] ), acc = exact int32 sum,
 * two separately rounded fp32 products, round to nearest even. Exactly one correct output.
 * Every M runs on int8 MFMA; the environment variable GQ8_W8A8_KERNEL=dot (read on every call)
 * forces a VALU dot4 kernel where it exists (M <= 15), for comparison: the output is the same
 * either way. */
int gq8_w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* W_packed,
                  const float* w_scale, uint16_t* out, int M, int N, int K,
                  void* ws, size_t ws_bytes, void* stream);

/* Same kernels, int32 accumulators written instead of the bf16 epilogue (acc int32 [M][N]).
 * Both W8A8 calls: M = 0..32, K % 16 == 0, K <= 8192 (GQ8_ESHAPE above), no workspace. */
int gq8_w8a8_gemm_i32(const int8_t* xq, const int8_t* W_packed, int32_t* acc, int M, int N,
                      int K, void* ws, size_t ws_bytes, void* stream);

/* Per-token int8 of a bf16 activation: the x_q and x_scale the W8A8 product takes (W8A8 page,
 * operator statement: int8 activation rows with one fp32 scale per row; the page does not say
 * how they are made, and the reading here is symmetric in each row's largest magnitude):
 *   amax = max_k |x[m][k]|, xs[m] = amax / 127, inv = 127 / amax (both 0 when amax == 0),
 *   xq[m][k] = clamp(round_half_away(x[m][k] * inv), -127, 127),
 * each quotient and product rounded to nearest-even fp32 (no fused multiply-add).
 * x bf16 [M][K], xq int8 [M][K] (both 16-byte aligned), xs fp32 [M]. M >= 0, K % 16 == 0;
 * K == 0 writes xs = 0. Errors: GQ8_EINVAL (negative size, null pointer), GQ8_ESHAPE,
 * GQ8_EALIGN, GQ8_ENODEV. */
int gq8_quantize_per_token(const uint16_t* x, int M, int K, int8_t* xq, float* xs, void* stream);

/* W8A8 on a bf16 activation: gq8_quantize_per_token(x), then gq8_w8a8_gemm on its x_q / x_scale.
 * out is bit-identical to that pair of calls. M <= 8 and M * K <= 16384: ONE kernel, in which
 * every work-group quantizes x into LDS while its weight tile streams in (no x_q round trip
 * through memory). Otherwise the two kernels, x_q / x_scale staged in xq_out / xs_out when both
 * are given, else in the workspace (gq8_workspace_bytes(GQ8_OP_W8A8_BF16X, M, N, K) bytes,
 * 16-byte aligned; 0 for the one-kernel shapes). x bf16 [M][K] (16-byte aligned, finite); W_packed, w_scale, out, shapes and errors as
 * gq8_w8a8_gemm (M = 0..32, K % 16 == 0, K <= 8192; K == 0 writes zeros and xs_out = 0), plus
 * GQ8_EWORKSPACE. xq_out int8 [M][K] (16-byte aligned) and xs_out fp32 [M] are nullable: when
 * given they receive that x_q and x_scale. */
int gq8_w8a8_gemm_bf16x(const uint16_t* x, const int8_t* W_packed, const float* w_scale,
                        uint16_t* out, int8_t* xq_out, float* xs_out, int M, int N, int K,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Routed experts (EP page, "What changed": q8_1 MoE input, the routed entries grouped by expert
 * so each expert's weights are read once, then the single-card combine; defer page, "What it
 * changes": rows combined by routing weight).
 * ------------------------------------------------------------------------------------------ */

/* Softmax over E router logits per token, then the top-k experts by probability, descending
 * (ties to the lower id); weights are those probabilities (not renormalised).
 * logits fp32 [T][E]; ids int32 [T][topk]; weights fp32 [T][topk]. T >= 1, 1 <= topk <= 16,
 * topk <= E <= 4096. */
int gq8_moe_route(const float* logits, int T, int E, int topk, int32_t* ids, float* weights,
                  void* stream);

/* Device plan (EP page, "What changed" and "How it was checked": every routed entry exactly
 * once). With P = T*topk entries, entry i = t*topk + j, the plan is int32 [gq8_moe_plan_words]:
 *   plan[0]               U, the number of distinct experts routed
 *   plan[1 + u]           expert of slot u (u < U), ascending
 *   plan[1 + P + u]       number of entries of slot u
 *   plan[1 + 2P + u]      index of slot u's first entry in the entry list
 *   plan[1 + 3P + i]      entry list: the entries grouped by slot, ascending within a slot
 * Slots u >= U are written as -1 / 0 / P. An id outside [0, E) makes U = -1 (plan error). */
size_t gq8_moe_plan_words(int T, int topk);
int gq8_moe_plan(const int32_t* ids, int T, int topk, int E, int32_t* plan, void* stream);

/* Routed Q8_0 experts on a q8_1 input. Expert e's gate/up weight, Q8_0 [2F][D] in split
 * layout (rows 0..F-1 gate, F..2F-1 up), starts at w_gate_up + e * gq8_q8_0_bytes(2F, D);
 * its down weight, Q8_0 [D][F], at w_down + e * gq8_q8_0_bytes(D, F). For each entry (t, j):
 *   g, u = gate/up rows . x[t]   (per 32-block: d_w * d_x * sum q_w q_x)
 *   h    = SiLU(g) * u            (fp32, not re-quantized)
 *   r    = down . h
 * and out[t] = bf16( sum_{j=0..topk-1} weights[t][j] * r_{t,j} ), in slot order.
 * xq int8 [T][D], xd fp16 [T][D/32] (the q8_1 quants and scales); ids int32 [T][topk];
 * weights fp32 [T][topk]; out bf16 [T][D]. D % 32 == 0, F % 32 == 0, F <= 1024,
 * T*topk <= 256. Only the routed experts' bytes are read. An id outside [0, E) anywhere in
 * ids (gq8_moe_route writes -1 for a row of NaN logits) makes the call write zeros to out and
 * read no expert. */
size_t gq8_moe_workspace_bytes(int T, int topk, int D, int F);
int gq8_moe_q8_0_routed(const int8_t* xq, const uint16_t* xd, const int32_t* ids,
                        const float* weights, const void* w_gate_up, const void* w_down,
                        uint16_t* out, int T, int topk, int E, int D, int F,
                        void* ws, size_t ws_bytes, void* stream);

/* The routed call on the bf16 MoE input itself (EP page, "What changed": the experts take the
 * q8_1 form of the input; here that quantization runs on the device, inside the gate/up kernel
 * when D <= 4096, else as a quantize step into the workspace). x bf16 [T][D] is quantized per
 * 32-block exactly as gq8_q8_1_quantize does, so out is bitwise the out of gq8_q8_1_quantize
 * followed by gq8_moe_q8_0_routed. x must be 16-byte aligned; shapes, weights, workspace
 * (gq8_moe_workspace_bytes) and errors as gq8_moe_q8_0_routed. */
int gq8_moe_q8_0_routed_bf16(const uint16_t* x, const int32_t* ids, const float* weights,
                             const void* w_gate_up, const void* w_down, uint16_t* out, int T,
                             int topk, int E, int D, int F, void* ws, size_t ws_bytes,
                             void* stream);

/* The routed call with options (flags, a bitwise or):
 *   GQ8_MOE_X_BF16  x is the bf16 input [T][D] (xd unused), quantized to q8_1 as in
 *                   gq8_moe_q8_0_routed_bf16; else x is the int8 q8_1 quants with scales xd.
 *   GQ8_MOE_H_Q8_1  the variant whose down read takes h in q8_1 form (the form the EP page
 *                   gives the MoE input, "What changed", applied to h): h rounded to fp32, then
 *                   quantized per 32-block with the input's rule, and the down read's blocks are
 *                   integer dots of those codes with the weight quants, scaled by both scales.
 *                   A different, slightly less exact read than the default (h in fp32), within
 *                   the same pass rule of the oracle's variant. Needs F in {256, 512, 1024} and
 *                   topk <= 16, else GQ8_ESHAPE.
 *   GQ8_MOE_DOWN_TILED  w_down holds the experts' down weights in the tiled layout
 *                   (gq8_q8_0_tile16 with rows = D, K = F, count = E; same size and expert
 *                   stride as the split layout). The results are bitwise those on the split
 *                   layout; the read is faster (contiguous 1 KiB loads). Needs F in
 *                   {256, 512, 1024}, topk <= 16 and D % 16 == 0, else GQ8_ESHAPE.
 * Other flag bits: GQ8_EINVAL. Shapes, weights, workspace and errors otherwise as
 * gq8_moe_q8_0_routed; flags = 0 is gq8_moe_q8_0_routed and GQ8_MOE_X_BF16 alone is
 * gq8_moe_q8_0_routed_bf16, bit for bit. */
enum { GQ8_MOE_X_BF16 = 1, GQ8_MOE_H_Q8_1 = 2, GQ8_MOE_DOWN_TILED = 4 };
int gq8_moe_q8_0_routed_flags(const void* x, const uint16_t* xd, const int32_t* ids,
                              const float* weights, const void* w_gate_up, const void* w_down,
                              uint16_t* out, int T, int topk, int E, int D, int F, int flags,
                              void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Diagnostics
 * ------------------------------------------------------------------------------------------ */

/* Streaming read of `bytes` (multiple of 16) from src, one 16-byte non-temporal load per lane,
 * 256 threads per work-group, eight work-groups per compute unit over 4 KiB chunks (the fastest
 * shape of a sweep of gq8_read_probe_ex at 4.5 to 34 MB); sink holds
 * gq8_read_probe_sink_floats(bytes) floats, written only for a bit pattern that keeps the loads
 * from being elided (its contents are unspecified). Measures the read bandwidth reachable for a
 * given byte count in one launch. */
size_t gq8_read_probe_sink_floats(size_t bytes);
int gq8_read_probe(const void* src, size_t bytes, float* sink, void* stream);

/* The same stream with its launch shape chosen: loads_per_lane 16-byte loads per lane per chunk
 * (1, 2, 4 or 8), threads per work-group (256, 512 or 1024), work_groups = 0 for one work-group per
 * chunk of threads * loads_per_lane * 16 bytes, else at most that many work-groups striding over
 * the chunks; nontemporal 1 for non-temporal loads, 0 for plain ones. The sink is as above (its
 * size covers every shape). Other values: GQ8_ESHAPE. For sweeping the shapes that bound how fast
 * a read of a given size can be. */
int gq8_read_probe_ex(const void* src, size_t bytes, float* sink, int loads_per_lane, int threads,
                      int work_groups, int nontemporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQ8_H */
