// Test driver: the C++ oracle (oracle/c/gq8_oracle.cpp, test infrastructure) built into one
// program with AddressSanitizer and UndefinedBehaviorSanitizer and run over small ragged shapes,
// every buffer allocated at its exact size. Each entry point runs on one thread and on several,
// and the two results must be bitwise equal (each output's sum has a fixed order). The numeric
// pins of the oracle live in tests/test_oracle_c.py; this program looks for memory and
// undefined-behaviour errors. Exit status 0 and "oracle_driver ok" mean every check passed.
#include "../../oracle/c/gq8_oracle.cpp"

#include <stdio.h>
#include <stdlib.h>

namespace {

int failures = 0;

void check(bool ok, const char* what, int a, int b) {
    if (!ok) {
        fprintf(stderr, "FAIL %s (%d, %d)\n", what, a, b);
        ++failures;
    }
}

uint64_t rng_state = 0x243f6a8885a308d3ull;

uint64_t next_u64() {  // splitmix64
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

float uniform_pm1() { return (float)((double)(next_u64() >> 11) * 0x1.0p-53 * 2.0 - 1.0); }

template <class T>
T* exact(size_t n) {
    return static_cast<T*>(malloc(n == 0 ? 1 : n * sizeof(T)));
}

bool same(const double* a, const double* b, size_t n) { return memcmp(a, b, n * sizeof(double)) == 0; }

// Q8_0 blocks of a random [rows][K] matrix: d [rows][K/32], q [rows][K]
void q8(int rows, int K, uint16_t** d, int8_t** q) {
    float* w = exact<float>((size_t)rows * K);
    for (int i = 0; i < rows * K; ++i) w[i] = 0.02f * uniform_pm1();
    *d = exact<uint16_t>((size_t)rows * (K / 32));
    *q = exact<int8_t>((size_t)rows * K);
    orc_q8_0_quantize(w, rows, K, *d, *q);
    free(w);
}

uint16_t bf16_of(float f) {
    uint16_t b;
    orc_f32_to_bf16(&f, 1, &b);
    return b;
}

void reads() {
    const int shapes[][3] = {{1, 5, 32}, {3, 17, 96}, {6, 40, 1056}};
    for (const auto& sh : shapes) {
        const int T = sh[0], N = sh[1], K = sh[2];
        uint16_t* d;
        int8_t* q;
        q8(N, K, &d, &q);
        float* x = exact<float>((size_t)T * K);
        for (int i = 0; i < T * K; ++i) x[i] = uniform_pm1();
        double *y1 = exact<double>((size_t)T * N), *ya = exact<double>((size_t)T * N);
        double *s1 = exact<double>((size_t)T * N), *sa = exact<double>((size_t)T * N);
        orc_q8_0_gemv(d, q, x, T, N, K, y1, s1, 1);
        orc_q8_0_gemv(d, q, x, T, N, K, ya, sa, 4);
        check(same(y1, ya, (size_t)T * N) && same(s1, sa, (size_t)T * N), "gemv threads", T, N);
        // the down read on bf16 rows and the up read of its output
        uint16_t* R = exact<uint16_t>((size_t)T * K);
        uint16_t* wn = exact<uint16_t>(K);
        for (int i = 0; i < T * K; ++i) R[i] = bf16_of(uniform_pm1());
        for (int k = 0; k < K; ++k) wn[k] = bf16_of(1.0f + 0.1f * uniform_pm1());
        double *lo1 = exact<double>((size_t)T * N), *loa = exact<double>((size_t)T * N);
        double *rs1 = exact<double>(T), *rsa = exact<double>(T);
        orc_hc_down(d, q, R, wn, T, N, K, 1e-6, lo1, rs1, s1, 1);
        orc_hc_down(d, q, R, wn, T, N, K, 1e-6, loa, rsa, sa, 4);
        check(same(lo1, loa, (size_t)T * N) && same(rs1, rsa, T), "down threads", T, N);
        {
            // up read: [K][N'] with N' = the down's N rounded up to a block multiple (zero-padded lo)
            const int Nu = (N + 31) / 32 * 32;
            uint16_t* lob = exact<uint16_t>((size_t)T * Nu);
            for (int t = 0; t < T; ++t)
                for (int n = 0; n < Nu; ++n) lob[(size_t)t * Nu + n] = n < N ? bf16_of((float)lo1[(size_t)t * N + n]) : 0;
            uint16_t* du;
            int8_t* qu;
            q8(K, Nu, &du, &qu);
            double *o1 = exact<double>((size_t)T * K), *oa = exact<double>((size_t)T * K);
            double *os = exact<double>((size_t)T * K);
            orc_hc_up(du, qu, lob, T, K, Nu, o1, os, 1);
            orc_hc_up(du, qu, lob, T, K, Nu, oa, os, 4);
            check(same(o1, oa, (size_t)T * K), "up threads", T, K);
            free(lob); free(du); free(qu); free(o1); free(oa); free(os);
        }
        free(d); free(q); free(x); free(y1); free(ya); free(s1); free(sa); free(R); free(wn);
        free(lo1); free(loa); free(rs1); free(rsa);
    }
}

void w8a8() {
    const int shapes[][3] = {{1, 17, 64}, {16, 40, 128}, {32, 3, 4096}};
    for (const auto& sh : shapes) {
        const int M = sh[0], N = sh[1], K = sh[2];
        int8_t* xq = exact<int8_t>((size_t)M * K);
        int8_t* W = exact<int8_t>((size_t)K * N);
        float* xs = exact<float>(M);
        float* ws = exact<float>(N);
        for (int i = 0; i < M * K; ++i) xq[i] = (int8_t)((int)(next_u64() % 255) - 127);
        for (int i = 0; i < K * N; ++i) W[i] = (int8_t)((int)(next_u64() % 255) - 127);
        for (int i = 0; i < M; ++i) xs[i] = 1e-3f + 9e-3f * (0.5f + 0.5f * uniform_pm1());
        for (int i = 0; i < N; ++i) ws[i] = 1e-3f + 9e-3f * (0.5f + 0.5f * uniform_pm1());
        int64_t *a1 = exact<int64_t>((size_t)M * N), *aa = exact<int64_t>((size_t)M * N);
        uint16_t *o1 = exact<uint16_t>((size_t)M * N), *oa = exact<uint16_t>((size_t)M * N);
        orc_w8a8(xq, xs, W, ws, M, N, K, a1, o1, 1);
        orc_w8a8(xq, xs, W, ws, M, N, K, aa, oa, 4);
        check(memcmp(a1, aa, (size_t)M * N * 8) == 0 && memcmp(o1, oa, (size_t)M * N * 2) == 0,
              "w8a8 threads", M, N);
        // one accumulator by hand
        int64_t want = 0;
        for (int k = 0; k < K; ++k) want += (int64_t)xq[k] * (int64_t)W[(size_t)k * N + N - 1];
        check(a1[N - 1] == want, "w8a8 accumulator", M, N);
        free(xq); free(W); free(xs); free(ws); free(a1); free(aa); free(o1); free(oa);
    }
}

void moe() {
    // T = 3 tokens, top-2 of E = 5 experts (3 routed), D = 64, F = 32
    const int T = 3, topk = 2, D = 64, F = 32, U = 3;
    int8_t* xq = exact<int8_t>((size_t)T * D);
    uint16_t* xd = exact<uint16_t>((size_t)T * (D / 32));
    for (int i = 0; i < T * D; ++i) xq[i] = (int8_t)((int)(next_u64() % 255) - 127);
    for (int i = 0; i < T * (D / 32); ++i) xd[i] = 0x2000;       // fp16 2^-7
    int64_t ids[T * topk] = {4, 1, 1, 2, 2, 4};
    double p[T * topk] = {0.6, 0.4, 0.7, 0.3, 0.55, 0.45};
    int* slot = exact<int>(5);
    slot[0] = slot[3] = 0;
    slot[1] = 0; slot[2] = 1; slot[4] = 2;
    uint16_t* gu_d = exact<uint16_t>((size_t)U * 2 * F * (D / 32));
    int8_t* gu_q = exact<int8_t>((size_t)U * 2 * F * D);
    uint16_t* dn_d = exact<uint16_t>((size_t)U * D * (F / 32));
    int8_t* dn_q = exact<int8_t>((size_t)U * D * F);
    for (int u = 0; u < U; ++u) {
        uint16_t* d;
        int8_t* q;
        q8(2 * F, D, &d, &q);
        memcpy(gu_d + (size_t)u * 2 * F * (D / 32), d, (size_t)2 * F * (D / 32) * 2);
        memcpy(gu_q + (size_t)u * 2 * F * D, q, (size_t)2 * F * D);
        free(d); free(q);
        q8(D, F, &d, &q);
        memcpy(dn_d + (size_t)u * D * (F / 32), d, (size_t)D * (F / 32) * 2);
        memcpy(dn_q + (size_t)u * D * F, q, (size_t)D * F);
        free(d); free(q);
    }
    double *y1 = exact<double>((size_t)T * D), *ya = exact<double>((size_t)T * D);
    double *s1 = exact<double>((size_t)T * D), *sa = exact<double>((size_t)T * D);
    double* h = exact<double>((size_t)T * topk * F);
    orc_moe_forward(xq, xd, ids, p, slot, gu_d, gu_q, dn_d, dn_q, T, topk, D, F, y1, s1, h, 1);
    orc_moe_forward(xq, xd, ids, p, slot, gu_d, gu_q, dn_d, dn_q, T, topk, D, F, ya, sa, h, 4);
    check(same(y1, ya, (size_t)T * D) && same(s1, sa, (size_t)T * D), "moe threads", T, D);
    for (int i = 0; i < T * D; ++i) check(fabs(y1[i]) <= s1[i], "moe |y| <= S", i, 0);
    free(xq); free(xd); free(slot); free(gu_d); free(gu_q); free(dn_d); free(dn_q);
    free(y1); free(ya); free(s1); free(sa); free(h);
}

}  // namespace

int main() {
    reads();
    w8a8();
    moe();
    if (failures != 0) {
        fprintf(stderr, "oracle_driver: %d failures\n", failures);
        return 1;
    }
    printf("oracle_driver ok\n");
    return 0;
}
