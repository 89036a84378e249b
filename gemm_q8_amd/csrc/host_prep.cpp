// Host-side weight and activation preparation (plain C++ on host memory; no HIP call): the Q8_0
// quantizer (HC-Q8 page, "What changed": ggml's rounding, d = amax / 127 stored as fp16 and
// q = round(w / d)), the 34-byte-block to split-layout reorder, the q8_1 quantizer of a bf16
// activation (EP page, "What changed": the q8_1 MoE input), and the W8A8 weight packer (W8A8
// page, "Cross-shape rules": the cold weight packed once into the product's fragment layout).
// The rounding is that of the device quantizers: fp32 quotients, fp16 round to nearest even,
// round half away from zero, quants clamped to [-127, 127], all-zero quants for a zero scale.
// Compiled without floating-point contraction or fast-math.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/gq8.h"

#define GQ8_HOST_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// fp32 -> fp16 bits, round to nearest even (subnormals, overflow to infinity, NaN kept NaN)
uint16_t f32_to_f16(float f) {
    const uint32_t x = f32_bits(f);
    const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    const uint32_t a = x & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7e00u;
    if (a >= 0x477ff000u) return sign | 0x7c00u;          // |f| >= 65520 rounds to infinity
    if (a < 0x38800000u) {                                 // below 2^-14: subnormal or zero
        // units of 2^-24; the scaling is exact, nearbyintf rounds to nearest even
        const float units = bits_f32(a) * 16777216.0f;
        return sign | (uint16_t)nearbyintf(units);       // 1024 becomes the smallest normal
    }
    uint32_t h = ((((a >> 23) - 127 + 15) << 10) | ((a & 0x7fffffu) >> 13));
    const uint32_t rem = a & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;   // a carry moves the exponent
    return sign | (uint16_t)h;
}

float f16_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    if (e == 0) {
        const float v = ldexpf((float)m, -24);
        return sign ? -v : v;
    }
    if (e == 31) return bits_f32(sign | 0x7f800000u | (m << 13));
    return bits_f32(sign | ((e - 15 + 127) << 23) | (m << 13));
}

// one block of 32 values -> fp16 scale bits and 32 quants
uint16_t quantize_block(const float* v, int8_t* q) {
    float amax = 0.f;
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint16_t dbits = f32_to_f16(amax / 127.0f);
    const float d = f16_to_f32(dbits);
    for (int i = 0; i < 32; ++i) {
        if (d == 0.f) {
            q[i] = 0;
            continue;
        }
        const float r = roundf(v[i] / d);               // C round: half away from zero
        // a NaN quotient (only from non-finite input) gives 0, as the device conversion does,
        // instead of an undefined float -> int conversion
        q[i] = (int8_t)(r != r ? 0 : (r > 127.f ? 127 : (r < -127.f ? -127 : (int)r)));
    }
    return dbits;
}

int check_rows(int rows, int K) {
    if (rows < 0 || K < 0) return GQ8_EINVAL;
    if (K % 32 != 0) return GQ8_ESHAPE;
    return GQ8_OK;
}

}  // namespace

GQ8_HOST_EXPORT int gq8_q8_0_quantize_host(const float* w, int rows, int K, void* split_out) {
    const int rc = check_rows(rows, K);
    if (rc != GQ8_OK) return rc;
    if (rows == 0 || K == 0) return GQ8_OK;
    if (w == nullptr || split_out == nullptr) return GQ8_EINVAL;
    const int nblk = K / 32;
    int8_t* q = static_cast<int8_t*>(split_out);
    uint8_t* d = static_cast<uint8_t*>(split_out) + (size_t)rows * K;
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nblk; ++b) {
            const uint16_t db = quantize_block(w + (size_t)r * K + 32 * b, q + (size_t)r * K + 32 * b);
            memcpy(d + 2 * ((size_t)r * nblk + b), &db, 2);
        }
    return GQ8_OK;
}

GQ8_HOST_EXPORT int gq8_q8_0_split_from_blocks_host(const void* blocks34, int rows, int K, void* split_out) {
    const int rc = check_rows(rows, K);
    if (rc != GQ8_OK) return rc;
    if (rows == 0 || K == 0) return GQ8_OK;
    if (blocks34 == nullptr || split_out == nullptr) return GQ8_EINVAL;
    const int nblk = K / 32;
    const uint8_t* src = static_cast<const uint8_t*>(blocks34);
    uint8_t* q = static_cast<uint8_t*>(split_out);
    uint8_t* d = q + (size_t)rows * K;
    for (size_t b = 0; b < (size_t)rows * nblk; ++b) {
        const size_t r = b / nblk, j = b % nblk;
        d[2 * b] = src[34 * b];                           // fp16 scale, little-endian
        d[2 * b + 1] = src[34 * b + 1];
        memcpy(q + r * K + 32 * j, src + 34 * b + 2, 32);
    }
    return GQ8_OK;
}

GQ8_HOST_EXPORT int gq8_q8_1_quantize_host(const uint16_t* x_bf16, int rows, int K, int8_t* q,
                                           uint16_t* d, uint16_t* s) {
    const int rc = check_rows(rows, K);
    if (rc != GQ8_OK) return rc;
    if (rows == 0 || K == 0) return GQ8_OK;
    if (x_bf16 == nullptr || q == nullptr || d == nullptr) return GQ8_EINVAL;
    const int nblk = K / 32;
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nblk; ++b) {
            float v[32];
            for (int i = 0; i < 32; ++i) v[i] = bits_f32((uint32_t)x_bf16[(size_t)r * K + 32 * b + i] << 16);
            int8_t* qb = q + (size_t)r * K + 32 * b;
            const uint16_t db = quantize_block(v, qb);
            d[(size_t)r * nblk + b] = db;
            if (s != nullptr) {
                int sum = 0;
                for (int i = 0; i < 32; ++i) sum += qb[i];
                // d (11 significant bits) times |sum| <= 4064 (12 bits) is exact in fp32
                s[(size_t)r * nblk + b] = f32_to_f16(f16_to_f32(db) * (float)sum);
            }
        }
    return GQ8_OK;
}

// W[K][N] int8 (logical, row-major) -> 16-column x 64-k fragments: slot (tile nt, k-step ks, lane
// l) holds the 16 bytes W[64 ks + 16 (l / 16) + e][16 nt + l % 16], e = 0..15, zero past K or N;
// slots in (nt, ks, l) order. The layout of gq8_w8a8_pack.
GQ8_HOST_EXPORT int gq8_w8a8_pack_host(const int8_t* W, int K, int N, int8_t* W_packed) {
    if (K < 0 || N < 0) return GQ8_EINVAL;
    if (K % 16 != 0) return GQ8_ESHAPE;
    if (K == 0 || N == 0) return GQ8_OK;
    if (W == nullptr || W_packed == nullptr) return GQ8_EINVAL;
    const int ntiles = (N + 15) / 16, ksteps = (K + 63) / 64;
    int8_t* out = W_packed;
    for (int nt = 0; nt < ntiles; ++nt)
        for (int ks = 0; ks < ksteps; ++ks)
            for (int l = 0; l < 64; ++l) {
                const int n = 16 * nt + l % 16, k0 = 64 * ks + 16 * (l / 16);
                for (int e = 0; e < 16; ++e) {
                    const int k = k0 + e;
                    *out++ = (n < N && k < K) ? W[(size_t)k * N + n] : (int8_t)0;
                }
            }
    return GQ8_OK;
}
