// C ABI of libgq8.so: argument checks, dispatch to the kernel launchers, workspace sizing.
// Every entry point validates before enqueueing anything and never allocates or synchronizes.
#include <stdlib.h>
#include <string.h>

#include "gq8_internal.h"

using namespace gq8;

namespace gq8 {

int device_cus() {
    static std::atomic<int> cached[64];     // zero-initialised (static storage); 0 = not yet known
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return 0;
    if (dev < 64) cached[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    return prop.multiProcessorCount;
}

bool force_general() {
    const char* v = getenv("GQ8_FORCE_GENERIC");
    if (v == nullptr || strcmp(v, "0") == 0 || v[0] == '\0') return false;
    if (strcmp(v, "1") == 0) return true;
    static std::atomic<bool> said{false};
    if (!said.exchange(true)) fprintf(stderr, "gq8: GQ8_FORCE_GENERIC=%s not understood (0 or 1); ignored\n", v);
    return false;
}

bool combine_last_arriver() {
    const char* v = getenv("GQ8_COMBINE");
    if (v == nullptr || v[0] == '\0' || strcmp(v, "kernel") == 0) return false;
    if (strcmp(v, "last") == 0) return true;
    static std::atomic<bool> said{false};
    if (!said.exchange(true)) fprintf(stderr, "gq8: GQ8_COMBINE=%s not understood (kernel or last); ignored\n", v);
    return false;
}

int w8a8_kernel_choice() {
    const char* v = getenv("GQ8_W8A8_KERNEL");
    if (v == nullptr || v[0] == '\0') return 0;
    if (strcmp(v, "dot") == 0) return 1;
    if (strcmp(v, "mfma") == 0) return 2;
    static std::atomic<bool> said{false};
    if (!said.exchange(true)) fprintf(stderr, "gq8: GQ8_W8A8_KERNEL=%s not understood (dot or mfma); ignored\n", v);
    return 0;
}

}  // namespace gq8

static inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

// Size limits, far above any decode-time shape, that keep every launch below 2^32 work-items and
// the kernels' int index arithmetic in range; a call beyond them returns GQ8_ESHAPE.
constexpr int64_t kMaxQ8Rows = int64_t(1) << 21;     // output rows of a Q8_0 read
constexpr int64_t kMaxQ8Depth = int64_t(1) << 24;    // depth of a Q8_0 read
constexpr int64_t kMaxQ8Elems = int64_t(1) << 36;    // rows x depth of a Q8_0 read
constexpr int64_t kMaxW8N = int64_t(1) << 24;        // W8A8 output columns
constexpr int64_t kMaxMoeD = int64_t(1) << 20;       // routed-expert model width
constexpr int64_t kMaxRouteT = int64_t(1) << 23;     // token rows of the top-k and the per-token quantizer
constexpr uint64_t kMaxItems = (uint64_t(1) << 32) - 256;   // one-work-item-per-element launches

// The largest grids these limits allow, in work-items (each must stay below 2^32):
constexpr uint64_t kItemCap = uint64_t(1) << 32;
// GEMV work-group kernel: up to 16 waves per output row
static_assert(uint64_t(kMaxQ8Rows) * 16 * 64 < kItemCap, "GEMV grid");
// slab kernels (down read: 512 columns; GEMV from T = 5: 256): ceil(K/256) x ceil(N/64) groups
// of up to 512
static_assert((uint64_t(kMaxQ8Elems) / (256 * 64) + uint64_t(kMaxQ8Rows) / 64 +
               uint64_t(kMaxQ8Depth) / 256 + 1) * 512 < kItemCap, "slab grid");
// up reads (N output rows = the pair's depth): ceil(N/64) groups of up to 512
static_assert((uint64_t(kMaxQ8Depth) / 64 + 1) * 512 < kItemCap, "up-read grid");
// W8A8: one group of up to 1024 per 16 columns
static_assert((uint64_t(kMaxW8N) / 16 + 1) * 1024 < kItemCap, "W8A8 grid");
// routed experts: 16 rows of D per group of 256 per token; the combine's T * D stays an int
static_assert((uint64_t(kMaxMoeD) / 16 + 1) * 256 * kMaxT < kItemCap, "routed-expert grid");
static_assert(uint64_t(kMaxMoeD) * kMaxT < (uint64_t(1) << 31), "routed-expert combine index");
// top-k and per-token quantizer: one group of 256 per row
static_assert(uint64_t(kMaxRouteT) * 256 < kItemCap, "per-row grids");

static int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return GQ8_OK;
    if (ws == nullptr || ws_bytes < need) return GQ8_EWORKSPACE;
    if (!aligned16(ws)) return GQ8_EALIGN;
    return GQ8_OK;
}

GQ8_EXPORT const char* gq8_status_str(int st) {
    switch (st) {
        case GQ8_OK: return "ok";
        case GQ8_EINVAL: return "invalid argument";
        case GQ8_ESHAPE: return "unsupported shape";
        case GQ8_EALIGN: return "misaligned pointer";
        case GQ8_EWORKSPACE: return "workspace missing or too small";
        case GQ8_ECAPTURE: return "stream is capturing";
        case GQ8_EHIP: return "HIP error";
        case GQ8_ENODEV: return "no gfx950 device";
        default: return "unknown status";
    }
}

GQ8_EXPORT int gq8_abi_version(void) { return GQ8_ABI_VERSION; }

GQ8_EXPORT int gq8_device_cus(int* cus_out) {
    if (cus_out == nullptr) return GQ8_EINVAL;
    const int c = device_cus();
    *cus_out = c;
    return c > 0 ? GQ8_OK : GQ8_ENODEV;
}

// ---------------------------------------------------------------------------------- Q8_0 layout

GQ8_EXPORT size_t gq8_q8_0_bytes(int64_t rows, int64_t K) {
    if (rows < 0 || K < 0 || K % 32 != 0) return 0;
    return (size_t)rows * (size_t)K + (size_t)rows * (size_t)(K / 32) * 2;
}

GQ8_EXPORT int gq8_q8_0_quantize(const float* w, int rows, int K, void* w_split, void* stream) {
    if (rows < 0 || K < 0) return GQ8_EINVAL;
    if (K % 32 != 0 || (uint64_t)rows * (uint64_t)(K / 32) > kMaxItems) return GQ8_ESHAPE;
    if (rows == 0 || K == 0) return GQ8_OK;
    if (w == nullptr || w_split == nullptr) return GQ8_EINVAL;
    if (!aligned16(w) || !aligned16(w_split)) return GQ8_EALIGN;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_q8_0_quantize(w, rows, K, w_split, S(stream));
}

GQ8_EXPORT int gq8_q8_0_split_from_blocks(const void* blocks34, int rows, int K, void* w_split,
                                          void* stream) {
    if (rows < 0 || K < 0) return GQ8_EINVAL;
    if (K % 32 != 0 || (uint64_t)rows * (uint64_t)(K / 32) > kMaxItems) return GQ8_ESHAPE;
    if (rows == 0 || K == 0) return GQ8_OK;
    if (blocks34 == nullptr || w_split == nullptr) return GQ8_EINVAL;
    if (!aligned16(w_split)) return GQ8_EALIGN;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_q8_0_split_from_blocks(blocks34, rows, K, w_split, S(stream));
}

GQ8_EXPORT int gq8_q8_0_tile16(const void* w_split, int rows, int K, int count, void* w_tiled,
                               void* stream) {
    if (rows < 0 || K < 0 || count < 0) return GQ8_EINVAL;
    if (rows % 16 != 0 || K % 64 != 0) return GQ8_ESHAPE;
    const uint64_t bytes = (uint64_t)rows * (uint64_t)K / 16 * 17;         // one matrix
    if (rows != 0 && K != 0 && (uint64_t)count > kMaxItems / (bytes / 16)) return GQ8_ESHAPE;
    if (rows == 0 || K == 0 || count == 0) return GQ8_OK;
    if (w_split == nullptr || w_tiled == nullptr) return GQ8_EINVAL;
    if (!aligned16(w_split) || !aligned16(w_tiled)) return GQ8_EALIGN;
    const uintptr_t a = reinterpret_cast<uintptr_t>(w_split), b = reinterpret_cast<uintptr_t>(w_tiled);
    const uint64_t n = bytes * (uint64_t)count;
    if (a < b + n && b < a + n) return GQ8_EINVAL;                         // overlapping buffers
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_q8_0_tile16(w_split, rows, K, count, w_tiled, S(stream));
}

GQ8_EXPORT int gq8_q8_1_quantize(const uint16_t* x_bf16, int rows, int K, int8_t* q, uint16_t* d,
                                 uint16_t* s, void* stream) {
    if (rows < 0 || K < 0) return GQ8_EINVAL;
    if (K % 32 != 0 || (uint64_t)rows * (uint64_t)(K / 32) > kMaxItems) return GQ8_ESHAPE;
    if (rows == 0 || K == 0) return GQ8_OK;
    if (x_bf16 == nullptr || q == nullptr || d == nullptr) return GQ8_EINVAL;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_q8_1_quantize(x_bf16, rows, K, q, d, s, S(stream));
}

// ---------------------------------------------------------------------------------- workspace

static bool q8_shape_ok(int T, int N, int K) {
    return T >= 0 && T <= kMaxT && N >= 0 && K >= 0 && K % 32 == 0 && N <= kMaxQ8Rows &&
           K <= kMaxQ8Depth && (int64_t)N * K <= kMaxQ8Elems;
}

// x_q staging of the bf16-activation product when it runs as two kernels: x_q [M][K] at 0, then
// x_scale [M] at the next 256-byte boundary
static size_t bf16x_stage_bytes(int M, int K) {
    return (((size_t)M * K + 255) & ~(size_t)255) + (size_t)M * sizeof(float);
}

GQ8_EXPORT size_t gq8_workspace_counter_bytes(int op, int rows, int N, int K) {
    switch (op) {
        case GQ8_OP_HC_DOWN:
        case GQ8_OP_HC_PAIR:
            if (!q8_shape_ok(rows, N, K) || rows == 0 || N == 0 || K == 0) return 0;
            return hc_down_counter_bytes(N);
        case GQ8_OP_Q8_0_GEMV:
            if (!q8_shape_ok(rows, N, K)) return 0;
            return gemv_counter_bytes(rows, N, K);
        default:
            return 0;
    }
}

GQ8_EXPORT size_t gq8_workspace_bytes(int op, int rows, int N, int K) {
    switch (op) {
        case GQ8_OP_HC_DOWN:
        case GQ8_OP_HC_PAIR:
            if (!q8_shape_ok(rows, N, K) || rows == 0 || N == 0 || K == 0) return 0;
            return hc_down_workspace_bytes(rows, N, K);
        case GQ8_OP_Q8_0_GEMV:
            if (!q8_shape_ok(rows, N, K)) return 0;
            return gemv_workspace_bytes(rows, N, K);
        case GQ8_OP_W8A8_BF16X:
            if (rows <= 0 || N <= 0 || K <= 0 || rows > kMaxM || K % 16 != 0 || bf16x_fused(rows, K))
                return 0;
            return bf16x_stage_bytes(rows, K);
        case GQ8_OP_HC_UP:
        case GQ8_OP_W8A8:
        default:
            return 0;
    }
}

GQ8_EXPORT int gq8_workspace_init(void* ws, size_t bytes, void* stream) {
    if (bytes == 0) return GQ8_OK;
    if (ws == nullptr) return GQ8_EINVAL;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(S(stream), &cs) != hipSuccess) return GQ8_EHIP;
    if (cs != hipStreamCaptureStatusNone) return GQ8_ECAPTURE;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_fill_zero(ws, bytes, S(stream));
}

GQ8_EXPORT int gq8_workspace_check(int op, int rows, int N, int K, const void* ws, size_t bytes,
                                   void* stream, int* nonzero_counters) {
    if (nonzero_counters == nullptr) return GQ8_EINVAL;
    const size_t need = gq8_workspace_bytes(op, rows, N, K);
    const size_t cb = gq8_workspace_counter_bytes(op, rows, N, K);
    *nonzero_counters = 0;
    if (cb == 0) return GQ8_OK;
    if (ws == nullptr || bytes < need) return GQ8_EWORKSPACE;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(S(stream), &cs) != hipSuccess) return GQ8_EHIP;
    if (cs != hipStreamCaptureStatusNone) return GQ8_ECAPTURE;
    unsigned host[1024];
    const size_t words = cb / sizeof(unsigned);
    const char* src = static_cast<const char*>(ws);         // the counters open the workspace
    int nz = 0;
    for (size_t w0 = 0; w0 < words; w0 += 1024) {
        const size_t nw = words - w0 < 1024 ? words - w0 : 1024;
        if (hipMemcpyAsync(host, src + w0 * sizeof(unsigned), nw * sizeof(unsigned),
                           hipMemcpyDeviceToHost, S(stream)) != hipSuccess ||
            hipStreamSynchronize(S(stream)) != hipSuccess)
            return GQ8_EHIP;
        for (size_t i = 0; i < nw; ++i) nz += host[i] != 0u;
    }
    *nonzero_counters = nz;
    return GQ8_OK;
}

// ---------------------------------------------------------------------------------- Q8_0 reads

GQ8_EXPORT int gq8_q8_0_gemv(const void* w_split, const float* x, float* y, int T, int N, int K,
                             void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || N < 0 || K < 0) return GQ8_EINVAL;
    if (!q8_shape_ok(T, N, K)) return GQ8_ESHAPE;
    if (T == 0 || N == 0) return GQ8_OK;
    if (y == nullptr) return GQ8_EINVAL;
    if (K == 0) {
        if (device_cus() == 0) return GQ8_ENODEV;
        return launch_fill_zero(y, (size_t)T * N * sizeof(float), S(stream));
    }
    if (w_split == nullptr || x == nullptr) return GQ8_EINVAL;
    if (!aligned16(w_split) || !aligned16(x)) return GQ8_EALIGN;
    const int rc = check_ws(ws, ws_bytes, gemv_workspace_bytes(T, N, K));
    if (rc != GQ8_OK) return rc;
    if (device_cus() == 0) return GQ8_ENODEV;
    GemvArgs a{};
    a.q = static_cast<const int8_t*>(w_split);
    a.d = reinterpret_cast<const uint16_t*>(a.q + (size_t)N * K);
    a.x = x; a.T = T; a.N = N; a.K = K; a.out = y;
    return launch_q8_0_gemv(a, ws, S(stream));
}

GQ8_EXPORT int gq8_hc_q8_down(const void* w_split, const uint16_t* R, const uint16_t* w_norm,
                              float eps, uint16_t* lo, float* rs_out, int T, int N, int K,
                              void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || N < 0 || K < 0) return GQ8_EINVAL;
    if (!q8_shape_ok(T, N, K) || K == 0) return GQ8_ESHAPE;
    if (T == 0 || N == 0) return GQ8_OK;
    if (w_split == nullptr || R == nullptr || w_norm == nullptr || lo == nullptr) return GQ8_EINVAL;
    if (!aligned16(R) || !aligned16(w_norm) || !aligned16(w_split)) return GQ8_EALIGN;
    if (!(eps >= 0.f)) return GQ8_EINVAL;
    int rc = check_ws(ws, ws_bytes, hc_down_workspace_bytes(T, N, K));
    if (rc != GQ8_OK) return rc;
    if (device_cus() == 0) return GQ8_ENODEV;
    GemvArgs a{};
    a.q = static_cast<const int8_t*>(w_split);
    a.d = reinterpret_cast<const uint16_t*>(a.q + (size_t)N * K);
    a.x = R; a.wnorm = w_norm; a.T = T; a.N = N; a.K = K; a.out = lo; a.rs_out = rs_out; a.eps = eps;
    return launch_hc_down(a, ws, S(stream));
}

// tiled: the up weights in the tiled layout (gq8_q8_0_tile16), N % 16 == 0 and K % 320 == 0
static int hc_up_common(const void* w, const uint16_t* lo, uint16_t* out, int T, int N, int K,
                        bool tiled, void* stream) {
    if (T < 0 || N < 0 || K < 0) return GQ8_EINVAL;
    if (!q8_shape_ok(T, N, K) || K > 1024) return GQ8_ESHAPE;
    if (tiled && (N % 16 != 0 || K % 320 != 0)) return GQ8_ESHAPE;
    if (T == 0 || N == 0) return GQ8_OK;
    if (out == nullptr) return GQ8_EINVAL;
    if (K == 0) {
        if (device_cus() == 0) return GQ8_ENODEV;
        return launch_fill_zero(out, (size_t)T * N * sizeof(uint16_t), S(stream));
    }
    if (w == nullptr || lo == nullptr) return GQ8_EINVAL;
    if (!aligned16(w) || !aligned16(lo)) return GQ8_EALIGN;
    if (device_cus() == 0) return GQ8_ENODEV;
    GemvArgs a{};
    a.q = static_cast<const int8_t*>(w);
    a.d = reinterpret_cast<const uint16_t*>(a.q + (size_t)N * K);
    a.x = lo; a.T = T; a.N = N; a.K = K; a.out = out; a.wt = tiled;
    return launch_hc_up(a, S(stream));
}

GQ8_EXPORT int gq8_hc_q8_up(const void* w_split, const uint16_t* lo, uint16_t* out, int T, int N,
                            int K, void* ws, size_t ws_bytes, void* stream) {
    (void)ws; (void)ws_bytes;
    return hc_up_common(w_split, lo, out, T, N, K, false, stream);
}

GQ8_EXPORT int gq8_hc_q8_up_tiled(const void* w_tiled, const uint16_t* lo, uint16_t* out, int T,
                                  int N, int K, void* ws, size_t ws_bytes, void* stream) {
    (void)ws; (void)ws_bytes;
    return hc_up_common(w_tiled, lo, out, T, N, K, true, stream);
}

static int hc_pair_common(const void* w_down, const uint16_t* R, const uint16_t* w_norm, float eps,
                          const void* w_up, uint16_t* lo, float* rs_out, uint16_t* out, int T,
                          int Nlr, int Khc, bool tiled, void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || Nlr < 0 || Khc < 0) return GQ8_EINVAL;
    if (!q8_shape_ok(T, Nlr, Khc) || Nlr % 32 != 0 || Nlr > 1024 || Khc == 0 || Nlr == 0)
        return GQ8_ESHAPE;
    if (tiled && (Khc % 16 != 0 || Nlr % 320 != 0)) return GQ8_ESHAPE;
    if (T == 0) return GQ8_OK;
    if (w_down == nullptr || R == nullptr || w_norm == nullptr || w_up == nullptr ||
        lo == nullptr || out == nullptr)
        return GQ8_EINVAL;
    if (!aligned16(w_down) || !aligned16(R) || !aligned16(w_norm) || !aligned16(w_up) ||
        !aligned16(lo))
        return GQ8_EALIGN;
    if (!(eps >= 0.f)) return GQ8_EINVAL;
    int rc = check_ws(ws, ws_bytes, hc_down_workspace_bytes(T, Nlr, Khc));
    if (rc != GQ8_OK) return rc;
    if (device_cus() == 0) return GQ8_ENODEV;
    GemvArgs dn{};
    dn.q = static_cast<const int8_t*>(w_down);
    dn.d = reinterpret_cast<const uint16_t*>(dn.q + (size_t)Nlr * Khc);
    dn.x = R; dn.wnorm = w_norm; dn.T = T; dn.N = Nlr; dn.K = Khc; dn.out = lo;
    dn.rs_out = rs_out; dn.eps = eps;
    GemvArgs up{};
    up.q = static_cast<const int8_t*>(w_up);
    up.d = reinterpret_cast<const uint16_t*>(up.q + (size_t)Khc * Nlr);
    up.x = lo; up.T = T; up.N = Khc; up.K = Nlr; up.out = out; up.wt = tiled;
    return launch_hc_pair(dn, up, ws, S(stream));
}

GQ8_EXPORT int gq8_hc_q8_pair(const void* w_down, const uint16_t* R, const uint16_t* w_norm,
                              float eps, const void* w_up, uint16_t* lo, float* rs_out,
                              uint16_t* out, int T, int Nlr, int Khc, void* ws, size_t ws_bytes,
                              void* stream) {
    return hc_pair_common(w_down, R, w_norm, eps, w_up, lo, rs_out, out, T, Nlr, Khc, false, ws,
                          ws_bytes, stream);
}

GQ8_EXPORT int gq8_hc_q8_pair_tiled(const void* w_down, const uint16_t* R, const uint16_t* w_norm,
                                    float eps, const void* w_up_tiled, uint16_t* lo, float* rs_out,
                                    uint16_t* out, int T, int Nlr, int Khc, void* ws,
                                    size_t ws_bytes, void* stream) {
    return hc_pair_common(w_down, R, w_norm, eps, w_up_tiled, lo, rs_out, out, T, Nlr, Khc, true,
                          ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------------- pending write

GQ8_EXPORT int gq8_hc_q8_down_pending(const void* w_split, const uint16_t* R, const uint16_t* P,
                                      const uint16_t* w_norm, float eps, uint16_t* R_out,
                                      uint16_t* lo, float* rs_out, int T, int N, int K, void* ws,
                                      size_t ws_bytes, void* stream) {
    if (T < 0 || N < 0 || K < 0) return GQ8_EINVAL;
    // the down read's row group 0 performs the pending write: N = 0 would leave R_out unwritten
    if (!q8_shape_ok(T, N, K) || K == 0 || N == 0) return GQ8_ESHAPE;
    if (T == 0) return GQ8_OK;
    if (w_split == nullptr || R == nullptr || P == nullptr || w_norm == nullptr || R_out == nullptr ||
        lo == nullptr)
        return GQ8_EINVAL;
    if (!aligned16(R) || !aligned16(P) || !aligned16(R_out) || !aligned16(w_norm) || !aligned16(w_split))
        return GQ8_EALIGN;
    if (!(eps >= 0.f)) return GQ8_EINVAL;
    int rc = check_ws(ws, ws_bytes, hc_down_workspace_bytes(T, N, K));
    if (rc != GQ8_OK) return rc;
    if (device_cus() == 0) return GQ8_ENODEV;
    GemvArgs a{};
    a.q = static_cast<const int8_t*>(w_split);
    a.d = reinterpret_cast<const uint16_t*>(a.q + (size_t)N * K);
    a.x = R; a.wnorm = w_norm; a.T = T; a.N = N; a.K = K; a.out = lo; a.rs_out = rs_out; a.eps = eps;
    a.pw = P; a.r_out = R_out;
    return launch_hc_down_pending(a, ws, S(stream));
}

GQ8_EXPORT int gq8_hc_q8_pair_pending(const void* w_down, const uint16_t* R, const uint16_t* P,
                                      const uint16_t* w_norm, float eps, const void* w_up,
                                      uint16_t* R_out, uint16_t* lo, float* rs_out, uint16_t* out,
                                      int T, int Nlr, int Khc, void* ws, size_t ws_bytes,
                                      void* stream) {
    if (T < 0 || Nlr < 0 || Khc < 0) return GQ8_EINVAL;
    if (!q8_shape_ok(T, Nlr, Khc) || Nlr % 32 != 0 || Nlr > 1024 || Khc == 0 || Nlr == 0)
        return GQ8_ESHAPE;
    if (T == 0) return GQ8_OK;
    if (w_down == nullptr || R == nullptr || P == nullptr || w_norm == nullptr || w_up == nullptr ||
        R_out == nullptr || lo == nullptr || out == nullptr)
        return GQ8_EINVAL;
    if (!aligned16(w_down) || !aligned16(R) || !aligned16(P) || !aligned16(R_out) ||
        !aligned16(w_norm) || !aligned16(w_up) || !aligned16(lo))
        return GQ8_EALIGN;
    if (!(eps >= 0.f)) return GQ8_EINVAL;
    int rc = check_ws(ws, ws_bytes, hc_down_workspace_bytes(T, Nlr, Khc));
    if (rc != GQ8_OK) return rc;
    if (device_cus() == 0) return GQ8_ENODEV;
    GemvArgs dn{};
    dn.q = static_cast<const int8_t*>(w_down);
    dn.d = reinterpret_cast<const uint16_t*>(dn.q + (size_t)Nlr * Khc);
    dn.x = R; dn.wnorm = w_norm; dn.T = T; dn.N = Nlr; dn.K = Khc; dn.out = lo;
    dn.rs_out = rs_out; dn.eps = eps; dn.pw = P; dn.r_out = R_out;
    GemvArgs up{};
    up.q = static_cast<const int8_t*>(w_up);
    up.d = reinterpret_cast<const uint16_t*>(up.q + (size_t)Khc * Nlr);
    up.x = lo; up.T = T; up.N = Khc; up.K = Nlr; up.out = out;
    return launch_hc_pair_pending(dn, up, ws, S(stream));
}

// ---------------------------------------------------------------------------------- no allocation
// The pair's workspace in a file-scope device array, for callers that cannot allocate (code
// under graph capture, allocation-free serving loops). Each device the library runs on holds
// its own copy of the array until the process ends; host code never uses the array's name (on
// the host it is only a stand-in), only the device address that hipGetSymbolAddress returns,
// fetched once per device with that device current and kept per device.

static __device__ __align__(256) unsigned char scratch[GQ8_NOALLOC_SCRATCH_BYTES];

static void* scratch_address() {
    static std::atomic<void*> addr[64];     // per device id; null = not yet fetched
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    addr[dev].store(p, std::memory_order_release);   // every thread that races here gets the same address
    return p;
}

GQ8_EXPORT int gq8_hc_q8_pair_noalloc(const void* w_down, const uint16_t* R, const uint16_t* w_norm,
                                      float eps, const void* w_up, uint16_t* lo, float* rs_out,
                                      uint16_t* out, int T, int Nlr, int Khc, void* stream) {
    if (T < 0 || Nlr < 0 || Khc < 0) return GQ8_EINVAL;
    if (!q8_shape_ok(T, Nlr, Khc) || Nlr % 32 != 0 || Nlr > 1024 || Khc == 0 || Nlr == 0)
        return GQ8_ESHAPE;
    if (T == 0) return GQ8_OK;
    if (hc_down_workspace_bytes(T, Nlr, Khc) > (size_t)GQ8_NOALLOC_SCRATCH_BYTES) return GQ8_ESHAPE;
    if (w_down == nullptr || R == nullptr || w_norm == nullptr || w_up == nullptr ||
        lo == nullptr || out == nullptr)
        return GQ8_EINVAL;
    if (!aligned16(w_down) || !aligned16(R) || !aligned16(w_norm) || !aligned16(w_up) ||
        !aligned16(lo))
        return GQ8_EALIGN;
    if (!(eps >= 0.f)) return GQ8_EINVAL;
    if (device_cus() == 0) return GQ8_ENODEV;
    void* ws = scratch_address();
    if (ws == nullptr) return GQ8_EHIP;
    GemvArgs dn{};
    dn.q = static_cast<const int8_t*>(w_down);
    dn.d = reinterpret_cast<const uint16_t*>(dn.q + (size_t)Nlr * Khc);
    dn.x = R; dn.wnorm = w_norm; dn.T = T; dn.N = Nlr; dn.K = Khc; dn.out = lo;
    dn.rs_out = rs_out; dn.eps = eps;
    GemvArgs up{};
    up.q = static_cast<const int8_t*>(w_up);
    up.d = reinterpret_cast<const uint16_t*>(up.q + (size_t)Khc * Nlr);
    up.x = lo; up.T = T; up.N = Khc; up.K = Nlr; up.out = out;
    return launch_hc_pair(dn, up, ws, S(stream));
}

GQ8_EXPORT int gq8_hc_bf16_pair(const uint16_t* w_down, const uint16_t* R, const uint16_t* w_norm,
                                float eps, const uint16_t* w_up, uint16_t* lo, float* rs_out,
                                uint16_t* out, int T, int Nlr, int Khc, void* ws, size_t ws_bytes,
                                void* stream) {
    if (T < 0 || Nlr < 0 || Khc < 0) return GQ8_EINVAL;
    if (!q8_shape_ok(T, Nlr, Khc) || Nlr % 32 != 0 || Nlr > 1024 || Khc == 0 || Nlr == 0)
        return GQ8_ESHAPE;
    if (T == 0) return GQ8_OK;
    if (w_down == nullptr || R == nullptr || w_norm == nullptr || w_up == nullptr ||
        lo == nullptr || out == nullptr)
        return GQ8_EINVAL;
    if (!aligned16(w_down) || !aligned16(R) || !aligned16(w_norm) || !aligned16(w_up) ||
        !aligned16(lo))
        return GQ8_EALIGN;
    if (!(eps >= 0.f)) return GQ8_EINVAL;
    int rc = check_ws(ws, ws_bytes, hc_down_workspace_bytes(T, Nlr, Khc));
    if (rc != GQ8_OK) return rc;
    if (device_cus() == 0) return GQ8_ENODEV;
    GemvArgs dn{};
    dn.q = reinterpret_cast<const int8_t*>(w_down);
    dn.x = R; dn.wnorm = w_norm; dn.T = T; dn.N = Nlr; dn.K = Khc; dn.out = lo;
    dn.rs_out = rs_out; dn.eps = eps;
    GemvArgs up{};
    up.q = reinterpret_cast<const int8_t*>(w_up);
    up.x = lo; up.T = T; up.N = Khc; up.K = Nlr; up.out = out;
    return launch_hc_bf16_pair(dn, up, ws, S(stream));
}

// ---------------------------------------------------------------------------------- W8A8

GQ8_EXPORT size_t gq8_w8a8_packed_bytes(int K, int N) {
    if (K < 0 || N < 0 || N > kMaxW8N) return 0;
    return (size_t)((N + 15) / 16) * 16 * (size_t)(((int64_t)K + 63) / 64) * 64;
}

GQ8_EXPORT int gq8_w8a8_pack(const int8_t* W, int K, int N, int8_t* W_packed, void* stream) {
    if (K < 0 || N < 0) return GQ8_EINVAL;
    if (K % 16 != 0 || N > kMaxW8N || gq8_w8a8_packed_bytes(K, N) / 16 > kMaxItems) return GQ8_ESHAPE;
    if (K == 0 || N == 0) return GQ8_OK;
    if (W == nullptr || W_packed == nullptr) return GQ8_EINVAL;
    if (!aligned16(W_packed)) return GQ8_EALIGN;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_w8a8_pack(W, K, N, W_packed, S(stream));
}

static int w8a8_common(const int8_t* xq, const float* xs, const int8_t* wp, const float* wsc,
                       void* out, bool i32, int M, int N, int K, void* stream) {
    if (M < 0 || N < 0 || K < 0) return GQ8_EINVAL;
    if (M > kMaxM || K % 16 != 0 || K > kW8MaxK || N > kMaxW8N) return GQ8_ESHAPE;
    if (M == 0 || N == 0) return GQ8_OK;
    if (out == nullptr) return GQ8_EINVAL;
    if (K == 0) {
        if (device_cus() == 0) return GQ8_ENODEV;
        return launch_fill_zero(out, (size_t)M * N * (i32 ? 4 : 2), S(stream));
    }
    if (xq == nullptr || wp == nullptr || (!i32 && (xs == nullptr || wsc == nullptr))) return GQ8_EINVAL;
    if (!aligned16(xq) || !aligned16(wp)) return GQ8_EALIGN;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_w8a8(plan_w8a8(M, N, K), xq, xs, wp, wsc, out, i32, M, N, K, S(stream));
}

GQ8_EXPORT int gq8_quantize_per_token(const uint16_t* x, int M, int K, int8_t* xq, float* xs,
                                      void* stream) {
    if (M < 0 || K < 0) return GQ8_EINVAL;
    if (K % 16 != 0 || M > kMaxRouteT || K > kMaxQ8Depth) return GQ8_ESHAPE;
    if (M == 0) return GQ8_OK;
    if (xs == nullptr || (K > 0 && (x == nullptr || xq == nullptr))) return GQ8_EINVAL;
    if (K > 0 && (!aligned16(x) || !aligned16(xq))) return GQ8_EALIGN;
    if (device_cus() == 0) return GQ8_ENODEV;
    if (K == 0) return launch_fill_zero(xs, (size_t)M * sizeof(float), S(stream));
    return launch_per_token_quantize(x, M, K, xq, xs, S(stream));
}

GQ8_EXPORT int gq8_w8a8_gemm_bf16x(const uint16_t* x, const int8_t* W_packed, const float* w_scale,
                                   uint16_t* out, int8_t* xq_out, float* xs_out, int M, int N,
                                   int K, void* ws, size_t ws_bytes, void* stream) {
    if (M < 0 || N < 0 || K < 0) return GQ8_EINVAL;
    if (M > kMaxM || K % 16 != 0 || K > kW8MaxK || N > kMaxW8N) return GQ8_ESHAPE;
    if (M == 0 || N == 0) return GQ8_OK;
    if (out == nullptr) return GQ8_EINVAL;
    if (K == 0) {
        if (device_cus() == 0) return GQ8_ENODEV;
        if (xs_out != nullptr) {
            const int rc = launch_fill_zero(xs_out, (size_t)M * sizeof(float), S(stream));
            if (rc != GQ8_OK) return rc;
        }
        return launch_fill_zero(out, (size_t)M * N * 2, S(stream));
    }
    if (x == nullptr || W_packed == nullptr || w_scale == nullptr) return GQ8_EINVAL;
    if (!aligned16(x) || !aligned16(W_packed) || (xq_out != nullptr && !aligned16(xq_out)))
        return GQ8_EALIGN;
    const bool fused = bf16x_fused(M, K);
    if (!fused && (xq_out == nullptr || xs_out == nullptr)) {
        const int rc = check_ws(ws, ws_bytes, bf16x_stage_bytes(M, K));
        if (rc != GQ8_OK) return rc;
    }
    if (device_cus() == 0) return GQ8_ENODEV;
    const W8Plan plan = plan_w8a8(M, N, K);
    if (fused)
        return launch_w8a8(plan, nullptr, nullptr, W_packed, w_scale, out, false, M, N, K,
                           S(stream), x, xq_out, xs_out);
    // larger x: the per-token quantize kernel, then the int8 product on its output
    int8_t* xq = xq_out != nullptr ? xq_out : static_cast<int8_t*>(ws);
    float* xs = xs_out != nullptr
                    ? xs_out
                    : reinterpret_cast<float*>(static_cast<char*>(ws) + bf16x_stage_bytes(M, K) -
                                               (size_t)M * sizeof(float));
    const int rc = launch_per_token_quantize(x, M, K, xq, xs, S(stream));
    if (rc != GQ8_OK) return rc;
    return launch_w8a8(plan, xq, xs, W_packed, w_scale, out, false, M, N, K, S(stream));
}

GQ8_EXPORT int gq8_w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* W_packed,
                             const float* w_scale, uint16_t* out, int M, int N, int K, void* ws,
                             size_t ws_bytes, void* stream) {
    (void)ws; (void)ws_bytes;
    return w8a8_common(xq, x_scale, W_packed, w_scale, out, false, M, N, K, stream);
}

GQ8_EXPORT int gq8_w8a8_gemm_i32(const int8_t* xq, const int8_t* W_packed, int32_t* acc, int M,
                                 int N, int K, void* ws, size_t ws_bytes, void* stream) {
    (void)ws; (void)ws_bytes;
    return w8a8_common(xq, nullptr, W_packed, nullptr, acc, true, M, N, K, stream);
}

// ---------------------------------------------------------------------------------- MoE

GQ8_EXPORT int gq8_moe_route(const float* logits, int T, int E, int topk, int32_t* ids,
                             float* weights, void* stream) {
    if (T < 0 || E < 0 || topk < 0) return GQ8_EINVAL;
    if (T == 0) return GQ8_OK;
    if (topk < 1 || topk > 16 || E < topk || E > 4096 || T > kMaxRouteT) return GQ8_ESHAPE;
    if (logits == nullptr || ids == nullptr || weights == nullptr) return GQ8_EINVAL;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_moe_route(logits, T, E, topk, ids, weights, S(stream));
}

GQ8_EXPORT size_t gq8_moe_plan_words(int T, int topk) {
    if (T < 0 || topk < 0) return 0;
    return 1 + 4 * (size_t)T * topk;
}

GQ8_EXPORT int gq8_moe_plan(const int32_t* ids, int T, int topk, int E, int32_t* plan,
                            void* stream) {
    if (T < 0 || topk < 0 || E < 0) return GQ8_EINVAL;
    if ((int64_t)T * topk > 256 || (T > 0 && topk < 1)) return GQ8_ESHAPE;
    if (T == 0) return GQ8_OK;
    if (ids == nullptr || plan == nullptr) return GQ8_EINVAL;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_moe_plan(ids, T, topk, E, plan, S(stream));
}

GQ8_EXPORT size_t gq8_moe_workspace_bytes(int T, int topk, int D, int F) {
    if (T < 1 || topk < 1 || D < 1 || F < 1) return 0;
    return moe_workspace_bytes(T, topk, D, F);
}

GQ8_EXPORT int gq8_moe_q8_0_routed(const int8_t* xq, const uint16_t* xd, const int32_t* ids,
                                   const float* weights, const void* w_gate_up, const void* w_down,
                                   uint16_t* out, int T, int topk, int E, int D, int F, void* ws,
                                   size_t ws_bytes, void* stream) {
    if (T < 0 || topk < 0 || E < 0 || D < 0 || F < 0) return GQ8_EINVAL;
    if (T == 0) return GQ8_OK;
    if (T > kMaxT || topk < 1 || (int64_t)T * topk > 256 || E < 1 || D < 32 || D % 32 != 0 || D > kMaxMoeD || F < 32 ||
        F % 32 != 0 || F > 1024)
        return GQ8_ESHAPE;
    if (xq == nullptr || xd == nullptr || ids == nullptr || weights == nullptr ||
        w_gate_up == nullptr || w_down == nullptr || out == nullptr)
        return GQ8_EINVAL;
    if (!aligned16(xq) || !aligned16(w_gate_up) || !aligned16(w_down)) return GQ8_EALIGN;
    int rc = check_ws(ws, ws_bytes, moe_workspace_bytes(T, topk, D, F));
    if (rc != GQ8_OK) return rc;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_moe_routed(xq, xd, nullptr, ids, weights, w_gate_up, w_down, out, T, topk, E, D,
                             F, false, false, ws, S(stream));
}

GQ8_EXPORT int gq8_moe_q8_0_routed_bf16(const uint16_t* x, const int32_t* ids, const float* weights,
                                        const void* w_gate_up, const void* w_down, uint16_t* out,
                                        int T, int topk, int E, int D, int F, void* ws,
                                        size_t ws_bytes, void* stream) {
    if (T < 0 || topk < 0 || E < 0 || D < 0 || F < 0) return GQ8_EINVAL;
    if (T == 0) return GQ8_OK;
    if (T > kMaxT || topk < 1 || (int64_t)T * topk > 256 || E < 1 || D < 32 || D % 32 != 0 || D > kMaxMoeD || F < 32 ||
        F % 32 != 0 || F > 1024)
        return GQ8_ESHAPE;
    if (x == nullptr || ids == nullptr || weights == nullptr || w_gate_up == nullptr ||
        w_down == nullptr || out == nullptr)
        return GQ8_EINVAL;
    if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down)) return GQ8_EALIGN;
    int rc = check_ws(ws, ws_bytes, moe_workspace_bytes(T, topk, D, F));
    if (rc != GQ8_OK) return rc;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_moe_routed(nullptr, nullptr, x, ids, weights, w_gate_up, w_down, out, T, topk, E,
                             D, F, false, false, ws, S(stream));
}

GQ8_EXPORT int gq8_moe_q8_0_routed_flags(const void* x, const uint16_t* xd, const int32_t* ids,
                                         const float* weights, const void* w_gate_up,
                                         const void* w_down, uint16_t* out, int T, int topk, int E,
                                         int D, int F, int flags, void* ws, size_t ws_bytes,
                                         void* stream) {
    if (T < 0 || topk < 0 || E < 0 || D < 0 || F < 0) return GQ8_EINVAL;
    if (flags & ~(GQ8_MOE_X_BF16 | GQ8_MOE_H_Q8_1 | GQ8_MOE_DOWN_TILED)) return GQ8_EINVAL;
    if (T == 0) return GQ8_OK;
    const bool xb = (flags & GQ8_MOE_X_BF16) != 0, hq = (flags & GQ8_MOE_H_Q8_1) != 0;
    const bool tl = (flags & GQ8_MOE_DOWN_TILED) != 0;
    if (T > kMaxT || topk < 1 || (int64_t)T * topk > 256 || E < 1 || D < 32 || D % 32 != 0 || D > kMaxMoeD || F < 32 ||
        F % 32 != 0 || F > 1024 || ((hq || tl) && ((F != 256 && F != 512 && F != 1024) || topk > 16)) ||
        (tl && D % 16 != 0))
        return GQ8_ESHAPE;
    if (x == nullptr || (!xb && xd == nullptr) || ids == nullptr || weights == nullptr ||
        w_gate_up == nullptr || w_down == nullptr || out == nullptr)
        return GQ8_EINVAL;
    if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down)) return GQ8_EALIGN;
    int rc = check_ws(ws, ws_bytes, moe_workspace_bytes(T, topk, D, F));
    if (rc != GQ8_OK) return rc;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_moe_routed(xb ? nullptr : static_cast<const int8_t*>(x), xb ? nullptr : xd,
                             xb ? static_cast<const uint16_t*>(x) : nullptr, ids, weights,
                             w_gate_up, w_down, out, T, topk, E, D, F, hq, tl, ws, S(stream));
}

// ---------------------------------------------------------------------------------- probe

GQ8_EXPORT size_t gq8_read_probe_sink_floats(size_t bytes) { return read_probe_blocks(bytes); }

GQ8_EXPORT int gq8_read_probe_ex(const void* src, size_t bytes, float* sink, int loads_per_lane,
                                 int threads, int work_groups, int nontemporal, void* stream) {
    if (bytes % 16 != 0 || bytes / 16 > kMaxItems) return GQ8_ESHAPE;
    if (!(loads_per_lane == 1 || loads_per_lane == 2 || loads_per_lane == 4 || loads_per_lane == 8) ||
        !(threads == 256 || threads == 512 || threads == 1024) || work_groups < 0 ||
        !(nontemporal == 0 || nontemporal == 1))
        return GQ8_ESHAPE;
    if (bytes == 0) return GQ8_OK;
    if (src == nullptr || sink == nullptr) return GQ8_EINVAL;
    if (!aligned16(src)) return GQ8_EALIGN;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_read_probe_ex(src, bytes, sink, loads_per_lane, threads, work_groups,
                                nontemporal != 0, S(stream));
}

GQ8_EXPORT int gq8_read_probe(const void* src, size_t bytes, float* sink, void* stream) {
    if (bytes % 16 != 0 || bytes / 16 > kMaxItems) return GQ8_ESHAPE;
    if (bytes == 0) return GQ8_OK;
    if (src == nullptr || sink == nullptr) return GQ8_EINVAL;
    if (!aligned16(src)) return GQ8_EALIGN;
    if (device_cus() == 0) return GQ8_ENODEV;
    return launch_read_probe(src, bytes, sink, S(stream));
}
