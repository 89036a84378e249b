// Test driver (not product code): the host preparation routines of gemm_q8_amd/csrc/host_prep.cpp
// built into one program with AddressSanitizer and UndefinedBehaviorSanitizer, run over ragged
// and degenerate shapes with every buffer allocated at its exact size, so that any read or write
// past a buffer, any signed overflow and any out-of-range float -> int conversion stops the
// program. Each call's output is also checked against a property of its definition. Exit status
// 0 and the line "host_prep_driver ok" mean every check passed.
#include "../../gemm_q8_amd/csrc/host_prep.cpp"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

namespace {

int failures = 0;

void check(bool ok, const char* what, int a, int b) {
    if (!ok) {
        fprintf(stderr, "FAIL %s (%d, %d)\n", what, a, b);
        ++failures;
    }
}

uint64_t rng_state = 0x9e3779b97f4a7c15ull;

uint64_t next_u64() {  // splitmix64
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

float uniform_pm1() { return (float)((double)(next_u64() >> 11) * 0x1.0p-53 * 2.0 - 1.0); }

// the split layout's size (quants, then one fp16 scale per 32-block); the library's
// gq8_q8_0_bytes lives in the device part of the library
size_t split_bytes(int rows, int K) { return (size_t)rows * K + (size_t)rows * (K / 32) * 2; }

// a heap buffer of exactly n elements, so that the sanitizer sees the buffer's real end
template <class T>
T* exact(size_t n) {
    return static_cast<T*>(malloc(n == 0 ? 1 : n * sizeof(T)));
}

void q8_0_shapes() {
    const int shapes[][2] = {{1, 32}, {3, 64}, {7, 96}, {16, 1024}, {5, 4128}};
    for (const auto& sh : shapes) {
        const int rows = sh[0], K = sh[1], nblk = K / 32;
        float* w = exact<float>((size_t)rows * K);
        for (int i = 0; i < rows * K; ++i) w[i] = 0.02f * uniform_pm1();
        for (int i = 0; i < 32; ++i) w[i] = 0.f;                          // a zero block
        if (nblk > 1)
            for (int i = 32; i < 64; ++i) w[i] = 1e-9f * uniform_pm1();  // a block whose fp16 d is 0
        const size_t nb = split_bytes(rows, K);
        uint8_t* split = exact<uint8_t>(nb);
        check(gq8_q8_0_quantize_host(w, rows, K, split) == GQ8_OK, "quantize", rows, K);
        const int8_t* q = reinterpret_cast<const int8_t*>(split);
        const uint8_t* dbytes = split + (size_t)rows * K;
        for (int r = 0; r < rows; ++r)
            for (int b = 0; b < nblk; ++b) {
                uint16_t db;
                memcpy(&db, dbytes + 2 * ((size_t)r * nblk + b), 2);
                const double d = f16_to_f32(db);
                int qmax = 0;
                for (int i = 0; i < 32; ++i) {
                    const size_t k = (size_t)r * K + 32 * b + i;
                    qmax = abs(q[k]) > qmax ? abs(q[k]) : qmax;
                    if (d > 0) check(fabs(w[k] - d * q[k]) <= d * (0.5 + 0x1p-17), "dequant bound", r, b);
                    else check(q[k] == 0, "zero scale gives zero quants", r, b);
                }
                if (d > 0) check(qmax == 127, "a block's largest quant is 127", r, b);
            }
        // the 34-byte blocks of the same matrix, reordered back into the split layout
        uint8_t* blocks = exact<uint8_t>((size_t)rows * nblk * 34);
        for (size_t b = 0; b < (size_t)rows * nblk; ++b) {
            const size_t r = b / nblk, j = b % nblk;
            memcpy(blocks + 34 * b, dbytes + 2 * b, 2);
            memcpy(blocks + 34 * b + 2, split + r * K + 32 * j, 32);
        }
        uint8_t* split2 = exact<uint8_t>(nb);
        check(gq8_q8_0_split_from_blocks_host(blocks, rows, K, split2) == GQ8_OK, "split", rows, K);
        check(memcmp(split, split2, nb) == 0, "blocks -> split round trip", rows, K);
        free(w); free(split); free(blocks); free(split2);
    }
}

void q8_0_non_finite() {
    // one block with NaN and infinity: defined, in range, and the next block unaffected
    float* w = exact<float>(64);
    for (int i = 0; i < 64; ++i) w[i] = 0.01f * (float)(i - 32);
    w[3] = NAN;
    w[7] = INFINITY;
    uint8_t* split = exact<uint8_t>(split_bytes(1, 64));
    check(gq8_q8_0_quantize_host(w, 1, 64, split) == GQ8_OK, "quantize non-finite", 1, 64);
    const int8_t* q = reinterpret_cast<const int8_t*>(split);
    for (int i = 0; i < 32; ++i) check(q[i] >= -127 && q[i] <= 127, "non-finite block in range", i, 0);
    check(q[32 + 31] == 127, "finite block after a non-finite one", q[63], 127);
    free(w); free(split);
}

void q8_1_shapes() {
    const int shapes[][2] = {{1, 32}, {4, 2048}, {3, 160}};
    for (const auto& sh : shapes) {
        const int rows = sh[0], K = sh[1], nblk = K / 32;
        uint16_t* x = exact<uint16_t>((size_t)rows * K);
        for (int i = 0; i < rows * K; ++i) {
            const float f = 3.0f * uniform_pm1();
            uint32_t u;
            memcpy(&u, &f, 4);
            x[i] = (uint16_t)(u >> 16);
        }
        int8_t* q = exact<int8_t>((size_t)rows * K);
        uint16_t* d = exact<uint16_t>((size_t)rows * nblk);
        uint16_t* s = exact<uint16_t>((size_t)rows * nblk);
        check(gq8_q8_1_quantize_host(x, rows, K, q, d, s) == GQ8_OK, "q8_1", rows, K);
        for (int b = 0; b < rows * nblk; ++b) {
            int sum = 0;
            for (int i = 0; i < 32; ++i) sum += q[32 * b + i];
            check(s[b] == f32_to_f16(f16_to_f32(d[b]) * (float)sum), "q8_1 block sum", b, sum);
        }
        int8_t* q2 = exact<int8_t>((size_t)rows * K);
        uint16_t* d2 = exact<uint16_t>((size_t)rows * nblk);
        check(gq8_q8_1_quantize_host(x, rows, K, q2, d2, nullptr) == GQ8_OK, "q8_1 without s", rows, K);
        check(memcmp(q, q2, (size_t)rows * K) == 0 && memcmp(d, d2, (size_t)rows * nblk * 2) == 0,
              "q8_1 with and without s", rows, K);
        free(x); free(q); free(d); free(s); free(q2); free(d2);
    }
}

void w8a8_pack_shapes() {
    const int shapes[][2] = {{16, 1}, {48, 17}, {64, 16}, {128, 33}, {80, 100}, {4096, 40}};
    for (const auto& sh : shapes) {
        const int K = sh[0], N = sh[1];
        int8_t* W = exact<int8_t>((size_t)K * N);
        for (int i = 0; i < K * N; ++i) W[i] = (int8_t)((int)(next_u64() % 255) - 127);
        const int ntiles = (N + 15) / 16, ksteps = (K + 63) / 64;
        const size_t nb = (size_t)ntiles * 16 * (size_t)ksteps * 64;
        int8_t* P = exact<int8_t>(nb);
        check(gq8_w8a8_pack_host(W, K, N, P) == GQ8_OK, "pack", K, N);
        // every slot back to its (k, n): the weight inside the matrix, zero outside
        for (size_t i = 0; i < nb; ++i) {
            const size_t e = i % 16, l = (i / 16) % 64, ks = (i / 1024) % ksteps, nt = i / (1024 * (size_t)ksteps);
            const size_t n = 16 * nt + l % 16, k = 64 * ks + 16 * (l / 16) + e;
            const int8_t want = (n < (size_t)N && k < (size_t)K) ? W[k * N + n] : (int8_t)0;
            if (P[i] != want) {
                check(false, "pack slot", (int)k, (int)n);
                break;
            }
        }
        free(W); free(P);
    }
}

void argument_errors() {
    float w[32] = {0};
    uint8_t out[34];
    check(gq8_q8_0_quantize_host(w, 1, 48, out) == GQ8_ESHAPE, "K % 32", 1, 48);
    check(gq8_q8_0_quantize_host(w, -1, 32, out) == GQ8_EINVAL, "negative rows", -1, 32);
    check(gq8_q8_0_quantize_host(nullptr, 1, 32, out) == GQ8_EINVAL, "null w", 1, 32);
    check(gq8_q8_0_quantize_host(nullptr, 0, 32, nullptr) == GQ8_OK, "empty", 0, 32);
    check(gq8_w8a8_pack_host(nullptr, 20, 4, nullptr) == GQ8_ESHAPE, "pack K % 16", 20, 4);
    check(gq8_q8_1_quantize_host(nullptr, 1, 32, nullptr, nullptr, nullptr) == GQ8_EINVAL, "q8_1 null", 1, 32);
}

}  // namespace

int main() {
    q8_0_shapes();
    q8_0_non_finite();
    q8_1_shapes();
    w8a8_pack_shapes();
    argument_errors();
    if (failures != 0) {
        fprintf(stderr, "host_prep_driver: %d failures\n", failures);
        return 1;
    }
    printf("host_prep_driver ok\n");
    return 0;
}
