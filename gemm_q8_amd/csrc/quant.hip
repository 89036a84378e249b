// Weight / activation preparation kernels (not on the timed path): Q8_0 and q8_1 quantizers
// (HC-Q8 page, "What changed": ggml's rounding; EP page, "What changed": the q8_1 MoE input),
// the 34-byte-block to split-layout reorder, the W8A8 fragment packer (W8A8 page, "Cross-shape
// rules": pack the cold weight once), a zero fill, and the streaming-read probe.
#include "gq8_device.h"
#include "gq8_internal.h"

namespace gq8 {

// One Q8_0 block: scale bits and 32 quants from 32 fp32 values.
GQ8_DEV uint16_t quantize_block(const float* v, int8_t* q) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint16_t dbits = q8_scale_bits(amax);
    const float d = h2f(dbits);
#pragma unroll
    for (int i = 0; i < 32; ++i) q[i] = (int8_t)q8_quant(v[i], d);
    return dbits;
}

__global__ void fill_zero_kernel(uint4* p, size_t n16, uint8_t* tail, size_t ntail) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

int launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
    if (bytes == 0) return GQ8_OK;
    const size_t n16 = bytes / 16, ntail = bytes % 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<uint4*>(p), n16, static_cast<uint8_t*>(p) + n16 * 16, ntail);
    return launch_status();
}

// -------------------------------------------------------------------------------- Q8_0

__global__ void q8_0_quantize_kernel(const float* __restrict__ w, int rows, int K,
                                     int8_t* __restrict__ q, uint16_t* __restrict__ d) {
    const int nblk = K >> 5;
    const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= (size_t)rows * nblk) return;
    const size_t row = b / nblk, blk = b - row * nblk;
    const float* src = w + row * K + blk * 32;
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 f = reinterpret_cast<const float4*>(src)[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    alignas(16) int8_t qb[32];
    d[b] = quantize_block(v, qb);
    uint4* dst = reinterpret_cast<uint4*>(q + row * K + blk * 32);
    dst[0] = *reinterpret_cast<const uint4*>(qb);
    dst[1] = *reinterpret_cast<const uint4*>(qb + 16);
}

int launch_q8_0_quantize(const float* w, int rows, int K, void* w_split, hipStream_t st) {
    const size_t nb = (size_t)rows * (K / 32);
    if (nb == 0) return GQ8_OK;
    int8_t* q = static_cast<int8_t*>(w_split);
    uint16_t* d = reinterpret_cast<uint16_t*>(q + (size_t)rows * K);
    hipLaunchKernelGGL(q8_0_quantize_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st,
                       w, rows, K, q, d);
    return launch_status();
}

__global__ void q8_0_split_kernel(const uint8_t* __restrict__ b34, int rows, int K,
                                  int8_t* __restrict__ q, uint16_t* __restrict__ d) {
    const int nblk = K >> 5;
    const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= (size_t)rows * nblk) return;
    const size_t row = b / nblk, blk = b - row * nblk;
    const uint8_t* src = b34 + b * 34;
    d[b] = (uint16_t)(src[0] | (src[1] << 8));
    int8_t* dst = q + row * K + blk * 32;
#pragma unroll
    for (int i = 0; i < 32; ++i) dst[i] = (int8_t)src[2 + i];
}

int launch_q8_0_split_from_blocks(const void* b34, int rows, int K, void* w_split, hipStream_t st) {
    const size_t nb = (size_t)rows * (K / 32);
    if (nb == 0) return GQ8_OK;
    int8_t* q = static_cast<int8_t*>(w_split);
    uint16_t* d = reinterpret_cast<uint16_t*>(q + (size_t)rows * K);
    hipLaunchKernelGGL(q8_0_split_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st,
                       static_cast<const uint8_t*>(b34), rows, K, q, d);
    return launch_status();
}

// -------------------------------------------------------------------------------- q8_1

__global__ void q8_1_quantize_kernel(const uint16_t* __restrict__ x, int rows, int K,
                                     int8_t* __restrict__ q, uint16_t* __restrict__ d,
                                     uint16_t* __restrict__ s) {
    const int nblk = K >> 5;
    const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= (size_t)rows * nblk) return;
    const size_t row = b / nblk, blk = b - row * nblk;
    const uint16_t* src = x + row * K + blk * 32;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = bf2f(src[i]);
    int8_t qb[32];
    const uint16_t dbits = quantize_block(v, qb);
    d[b] = dbits;
    if (s != nullptr) {
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) sum += qb[i];
        s[b] = f2h_bits(h2f(dbits) * (float)sum);   // the product is exact in fp32
    }
    int8_t* dst = q + row * K + blk * 32;
#pragma unroll
    for (int i = 0; i < 32; ++i) dst[i] = qb[i];
}

int launch_q8_1_quantize(const uint16_t* x, int rows, int K, int8_t* q, uint16_t* d, uint16_t* s,
                         hipStream_t st) {
    const size_t nb = (size_t)rows * (K / 32);
    if (nb == 0) return GQ8_OK;
    hipLaunchKernelGGL(q8_1_quantize_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st,
                       x, rows, K, q, d, s);
    return launch_status();
}

// -------------------------------------------------------------------------------- W8A8 packing
// Packed layout: fragments of 16 columns x 64 k, [N/16][K/64][lane 0..63][16 bytes], lane l
// holding W[k0 + 16*(l/16) + e][n0 + l%16] for e = 0..15 (zero outside K x N). A wave reads one
// fragment as one contiguous 1 KiB load, 16 bytes per lane.

__global__ void w8a8_pack_kernel(const int8_t* __restrict__ W, int K, int N, int ksteps,
                                 int8_t* __restrict__ Wp, size_t nslots) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // (tile, kstep, lane)
    if (i >= nslots) return;
    const int lane = (int)(i & 63);
    const size_t frag = i >> 6;
    const int ks = (int)(frag % ksteps);
    const int nt = (int)(frag / ksteps);
    const int n = nt * 16 + (lane & 15);
    const int k0 = ks * 64 + 16 * (lane >> 4);
    int8_t v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int k = k0 + e;
        v[e] = (n < N && k < K) ? W[(size_t)k * N + n] : (int8_t)0;
    }
    *reinterpret_cast<uint4*>(Wp + i * 16) = *reinterpret_cast<const uint4*>(v);
}

int launch_w8a8_pack(const int8_t* W, int K, int N, int8_t* Wp, hipStream_t st) {
    const int ntiles = (N + 15) / 16, ksteps = (K + 63) / 64;
    const size_t nslots = (size_t)ntiles * ksteps * 64;
    if (nslots == 0) return GQ8_OK;
    hipLaunchKernelGGL(w8a8_pack_kernel, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0, st,
                       W, K, N, ksteps, Wp, nslots);
    return launch_status();
}

// -------------------------------------------------------------------------------- read probe
// 256 threads per work-group, one 16-byte non-temporal load each (4 KiB per work-group): the
// launch shape that streams a few MiB fastest on this chip.

constexpr size_t kProbeChunk = 4096;

size_t read_probe_blocks(size_t bytes) { return (bytes + kProbeChunk - 1) / kProbeChunk; }

__global__ void __launch_bounds__(256) read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         float* __restrict__ sink) {
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    i = i < n16 ? i : n16 - 1;
    const u32x4 v = __builtin_nontemporal_load(src + i);
    const uint32_t x = v.x ^ v.y ^ v.z ^ v.w;
    if (x == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x] = 1.0f;   // keeps the load alive
}

int launch_read_probe(const void* src, size_t bytes, float* sink, hipStream_t st) {
    const size_t blocks = read_probe_blocks(bytes);
    if (blocks == 0) return GQ8_OK;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const u32x4*>(src), bytes / 16, sink);
    return launch_status();
}

}  // namespace gq8
