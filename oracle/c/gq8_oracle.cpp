// CPU oracle in plain C++ (test infrastructure; nothing in the product path builds, links or calls
// it). The same definitions as the numpy oracle in this directory's parent, written out as loops
// in float64 / int64 with a fixed k-ascending order per output, so that a run on one thread and a
// run on all host cores (OpenMP over output rows) give bitwise the same result:
//   * Q8_0 quantizer (HC-Q8 page, "What changed": ggml's rounding): d = fp16(amax / 127), the
//     quotient in fp32, round to nearest even; q = round(w / d) with the fp32 quotient by the
//     stored fp16 d, ties away from zero, clamped to +-127; a block whose fp16 d is 0 gets zeros;
//   * Q8_0 matrix-vector product: y[t][n] = sum_k d[n][k/32] q[n][k] x[t][k], S = sum |d q x|;
//   * fused RMSNorm + Q8_0 down read (HC-Q8 page, "What changed"): rs = 1 / sqrt(mean_k R^2 + eps)
//     over the token row, lo = rs * sum_k d q (R w_norm), applied after the dot;
//   * W8A8 (W8A8 page, operator statement): acc = sum_k x_q W as int64, then
//     bf16( (fp32(acc) * x_scale[m]) * w_scale[n] ), two separately rounded fp32 products;
//   * routed experts (EP page, "What changed"; defer page, "What it changes"): per entry, block
//     integer dots of the Q8_0 gate/up rows with the q8_1 input scaled by both scales, h = SiLU(g) u
//     (gate rows first), r = down . h, y[t] = sum_j p[t][j] r_{t,j} in slot order.
// Layouts are the oracle's own block structures: Q8_0 scales d[rows][K/32] (fp16 bits) and
// quants q[rows][K/32][32]; W8A8 weights W[K][N] row-major (the logical layout, not a packed one).
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

float f32_of_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
uint32_t bits_of_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

// IEEE binary16 bits -> value (exact in float)
float f16_to_f32(uint16_t h) {
    const int sign = (h >> 15) & 1, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                       // subnormal (or zero)
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1024.0 + m, e - 25);                          // (1 + m / 1024) 2^(e - 15)
    return (float)(sign ? -v : v);
}

// float -> binary16 bits, round to nearest even: the value is scaled so that the kept bits are
// the integer part, rounded with nearbyint (the default mode rounds ties to even), and re-encoded.
uint16_t f32_to_f16(float f) {
    const uint16_t sign = (bits_of_f32(f) >> 16) & 0x8000;
    if (isnan(f)) return sign | 0x7e00;
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                                                // a = mant 2^e, mant in [0.5, 1)
    int ex = e - 1;                                              // a in [2^ex, 2^(ex+1))
    if (ex < -14) ex = -14;                                      // subnormal spacing 2^-24
    const double q = nearbyint(ldexp(a, 10 - ex));               // integer, 1024 <= q <= 2048 (normal)
    double v = ldexp(q, ex - 10);
    if (v >= 65520.0 || v > 65504.0) return sign | 0x7c00;       // rounds past the largest half
    if (v < ldexp(1.0, -14)) return sign | (uint16_t)q;          // subnormal: q = v / 2^-24
    int e2;
    frexp(v, &e2);
    const int be = e2 - 1 + 15;
    const int man = (int)(ldexp(v, -(e2 - 1)) * 1024.0) - 1024;
    return sign | (uint16_t)((be << 10) | man);
}

float bf16_to_f32(uint16_t b) { return f32_of_bits((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even on the dropped 16 bits
uint16_t f32_to_bf16(float f) {
    if (isnan(f)) return 0x7fc0;
    const uint32_t u = bits_of_f32(f);
    const uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(r >> 16);
}

// round half away from zero (C round) on a float, as an integer
long round_away(float v) { return lround((double)v); }

// threads > 0: that many; otherwise every host core
void set_threads(int threads) {
#ifdef _OPENMP
    omp_set_num_threads(threads > 0 ? threads : omp_get_num_procs());
#else
    (void)threads;
#endif
}

}  // namespace

ORC_EXPORT int orc_threads_available(void) {
#ifdef _OPENMP
    return omp_get_num_procs();
#else
    return 1;
#endif
}

// --------------------------------------------------------------------------------- number formats

ORC_EXPORT void orc_f32_to_f16(const float* x, long n, uint16_t* out) {
    for (long i = 0; i < n; ++i) out[i] = f32_to_f16(x[i]);
}

ORC_EXPORT void orc_f32_to_bf16(const float* x, long n, uint16_t* out) {
    for (long i = 0; i < n; ++i) out[i] = f32_to_bf16(x[i]);
}

// --------------------------------------------------------------------------------- Q8_0 quantizer

ORC_EXPORT void orc_q8_0_quantize(const float* w, int rows, int K, uint16_t* d, int8_t* q) {
    const int nb = K / 32;
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < nb; ++b) {
            const float* blk = w + (size_t)r * K + 32 * b;
            float amax = 0.f;
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(blk[i]));
            const float d32 = amax / 127.0f;                       // fp32 quotient
            const uint16_t db = f32_to_f16(d32);
            const float dv = f16_to_f32(db);
            d[(size_t)r * nb + b] = db;
            int8_t* qb = q + ((size_t)r * nb + b) * 32;
            for (int i = 0; i < 32; ++i) {
                long qi = 0;
                if (dv != 0.f) {
                    const float t = blk[i] / dv;                      // fp32 quotient by the stored d
                    qi = round_away(t);
                    qi = qi > 127 ? 127 : (qi < -127 ? -127 : qi);
                }
                qb[i] = (int8_t)qi;
            }
        }
}

// --------------------------------------------------------------------------------- Q8_0 reads

// y[t][n] = sum_k d q x[t][k]; x is fp32 (xf) or bf16 (xb); S = sum_k |d q x|
static void q8_gemv(const uint16_t* d, const int8_t* q, const float* xf, const uint16_t* xb,
                    int T, int N, int K, double* y, double* S, int threads) {
    set_threads(threads);
    const int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int t = 0; t < T; ++t) {
            double acc = 0.0, sa = 0.0;
            for (int b = 0; b < nb; ++b) {
                const double dv = (double)f16_to_f32(d[(size_t)n * nb + b]);
                const int8_t* qb = q + ((size_t)n * nb + b) * 32;
                for (int i = 0; i < 32; ++i) {
                    const int k = 32 * b + i;
                    const double xv = xf ? (double)xf[(size_t)t * K + k] : (double)bf16_to_f32(xb[(size_t)t * K + k]);
                    const double term = dv * (double)qb[i] * xv;
                    acc += term;
                    sa += fabs(term);
                }
            }
            y[(size_t)t * N + n] = acc;
            if (S) S[(size_t)t * N + n] = sa;
        }
    }
}

ORC_EXPORT void orc_q8_0_gemv(const uint16_t* d, const int8_t* q, const float* x, int T, int N, int K,
                              double* y, double* S, int threads) {
    q8_gemv(d, q, x, nullptr, T, N, K, y, S, threads);
}

// the up read: the Q8_0 product on a bf16 input
ORC_EXPORT void orc_hc_up(const uint16_t* d, const int8_t* q, const uint16_t* lo, int T, int N, int K,
                          double* y, double* S, int threads) {
    q8_gemv(d, q, nullptr, lo, T, N, K, y, S, threads);
}

ORC_EXPORT void orc_hc_down(const uint16_t* d, const int8_t* q, const uint16_t* R, const uint16_t* wn,
                            int T, int N, int K, double eps, double* lo, double* rs, double* S,
                            int threads) {
    set_threads(threads);
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int k = 0; k < K; ++k) {
            const double r = (double)bf16_to_f32(R[(size_t)t * K + k]);
            ss += r * r;
        }
        rs[t] = 1.0 / sqrt(ss / K + eps);
    }
    const int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int t = 0; t < T; ++t) {
            double acc = 0.0, sa = 0.0;
            for (int b = 0; b < nb; ++b) {
                const double dv = (double)f16_to_f32(d[(size_t)n * nb + b]);
                const int8_t* qb = q + ((size_t)n * nb + b) * 32;
                for (int i = 0; i < 32; ++i) {
                    const int k = 32 * b + i;
                    const double u = (double)bf16_to_f32(R[(size_t)t * K + k]) * (double)bf16_to_f32(wn[k]);
                    const double term = dv * (double)qb[i] * u;
                    acc += term;
                    sa += fabs(term);
                }
            }
            lo[(size_t)t * N + n] = rs[t] * acc;
            if (S) S[(size_t)t * N + n] = rs[t] * sa;
        }
    }
}

// --------------------------------------------------------------------------------- W8A8

ORC_EXPORT void orc_w8a8(const int8_t* xq, const float* xs, const int8_t* W, const float* ws, int M,
                         int N, int K, int64_t* acc, uint16_t* out, int threads) {
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int m = 0; m < M; ++m) {
            int64_t a = 0;
            for (int k = 0; k < K; ++k) a += (int64_t)xq[(size_t)m * K + k] * (int64_t)W[(size_t)k * N + n];
            if (acc) acc[(size_t)m * N + n] = a;
            if (out) {
                volatile float f = (float)a;                     // nearest fp32, ties to even
                volatile float g = f * xs[m];                    // rounded fp32 product
                volatile float h = g * ws[n];                    // second rounded product
                out[(size_t)m * N + n] = f32_to_bf16(h);
            }
        }
    }
}

// --------------------------------------------------------------------------------- routed experts

// xq int8 [T][D], xd fp16 [T][D/32] (the q8_1 input); ids [T][topk] in [0, E); p [T][topk];
// slot_of[e] = index u of expert e's weights in the per-expert arrays (only routed experts):
//   gu_d [U][2F][D/32], gu_q [U][2F][D/32][32], dn_d [U][D][F/32], dn_q [U][D][F/32][32].
// y, S [T][D]. Entries run in parallel over the output rows of the down projection; every
// output's sum over slots runs j = 0..topk-1.
ORC_EXPORT void orc_moe_forward(const int8_t* xq, const uint16_t* xd, const int64_t* ids,
                                const double* p, const int* slot_of, const uint16_t* gu_d,
                                const int8_t* gu_q, const uint16_t* dn_d, const int8_t* dn_q,
                                int T, int topk, int D, int F, double* y, double* S, double* hbuf,
                                int threads) {
    set_threads(threads);
    const int nbd = D / 32, nbf = F / 32;
    // h for every entry: hbuf [T * topk][F]
#pragma omp parallel for schedule(static)
    for (int ent = 0; ent < T * topk; ++ent) {
        const int t = ent / topk;
        const int u = slot_of[ids[ent]];
        const uint16_t* gd = gu_d + (size_t)u * 2 * F * nbd;
        const int8_t* gq = gu_q + (size_t)u * 2 * F * nbd * 32;
        for (int n = 0; n < F; ++n) {
            double gv[2];
            for (int half = 0; half < 2; ++half) {
                const int rowi = half * F + n;                   // gate rows 0..F-1, up rows F..2F-1
                double acc = 0.0;
                for (int b = 0; b < nbd; ++b) {
                    int64_t qi = 0;
                    const int8_t* wq = gq + ((size_t)rowi * nbd + b) * 32;
                    const int8_t* xqb = xq + (size_t)t * D + 32 * b;
                    for (int i = 0; i < 32; ++i) qi += (int64_t)wq[i] * (int64_t)xqb[i];
                    acc += (double)f16_to_f32(gd[(size_t)rowi * nbd + b]) *
                           (double)f16_to_f32(xd[(size_t)t * nbd + b]) * (double)qi;
                }
                gv[half] = acc;
            }
            const double g = gv[0], uu = gv[1];
            hbuf[(size_t)ent * F + n] = g / (1.0 + exp(-g)) * uu;
        }
    }
#pragma omp parallel for schedule(static)
    for (int m = 0; m < D; ++m) {
        for (int t = 0; t < T; ++t) {
            double yv = 0.0, sv = 0.0;
            for (int j = 0; j < topk; ++j) {
                const int ent = t * topk + j;
                const int u = slot_of[ids[ent]];
                const uint16_t* dd = dn_d + (size_t)u * D * nbf;
                const int8_t* dq = dn_q + (size_t)u * D * nbf * 32;
                double r = 0.0, sa = 0.0;
                for (int b = 0; b < nbf; ++b) {
                    const double dv = (double)f16_to_f32(dd[(size_t)m * nbf + b]);
                    const int8_t* qb = dq + ((size_t)m * nbf + b) * 32;
                    for (int i = 0; i < 32; ++i) {
                        const double term = dv * (double)qb[i] * hbuf[(size_t)ent * F + 32 * b + i];
                        r += term;
                        sa += fabs(term);
                    }
                }
                yv += p[ent] * r;
                sv += fabs(p[ent]) * sa;
            }
            y[(size_t)t * D + m] = yv;
            S[(size_t)t * D + m] = sv;
        }
    }
}
