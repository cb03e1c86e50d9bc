/*
 * pq2_oracle.c -- plain, slow CPU oracle for the PQ2_0 ternary-weight GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * What it computes, and the passages it follows (page 1 = "Making a ternary
 * reasoning model fast in vLLM -- from CUDA to Triton and Gluon"; page 2 =
 * "Chasing llama.cpp at batch one"):
 *
 *  - Weight format (page 1, section "One token at a time: plain Triton is
 *    enough"): each weight is a 2-bit code c in {0,1,2} standing for c-1,
 *    four codes per byte. The code of weight k of row n is bits
 *    2*(k%4)..2*(k%4)+1 of byte n*K/4 + k/4 (the bit order matches the
 *    selector construction of page 2, section "Recover four weights with one
 *    lookup"). Code 3 is not a PQ2_0 code; page 2's lookup table maps it to
 *    +2, and c-1 gives the same, so the oracle decodes every code as c-1.
 *  - Activation quantisation per 128-weight group (page 1, section "Prompt
 *    processing: check configuration and launch costs": per call the
 *    quantiser writes int8 q [m][k], float32 s [m][G] and int32 t [m][G]).
 *    The pages do not state the rule; the workload definition does:
 *    scale = max|x| / 127, round half to even. Reading used here, all in
 *    float32 because the result decides an integer: s = fl32(amax / 127),
 *    q = clamp(rint(fl32(x / s)), -127, 127) with a correctly rounded
 *    division, t = sum of q. A group with s == 0 (all zero, or amax so small
 *    that the division underflows) gets q = 0 and t = 0.
 *  - Plane order (page 1, "One token at a time"): inside each 128-group the
 *    activation of weight 4*b+s is stored at position 32*s+b.
 *  - Group dot (page 1, "One token at a time"): the method computes
 *    dot(codes, q) - sum(q) per 128-group, which equals the ternary dot
 *    sum_k (c_k - 1) * q_k. The oracle writes out that plain definition in
 *    natural k order, with the decoded weight.
 *  - Epilogue (page 1, "One token at a time", and the ring-kernel listing in
 *    "Use a ring buffer for longer rows"): y[m][n] = sum_g D[m][n][g] *
 *    s[m][g] * ws[n][g]. The oracle evaluates it in float64; every term is
 *    exact in float64 (|D| < 2^15, s has 24 significant bits, ws 11).
 *
 * Built with plain gcc -O2, no fast-math, no FP contraction, no intrinsics.
 * OpenMP (when enabled) only splits independent output rows between threads;
 * each output is still the plain sequential loop above.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define PQ2_ORACLE_GROUP 128

int oracle_version(void) { return 1; }

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static void set_threads(int threads) {
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
}

/* IEEE 754 binary16 -> binary64, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                  /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);      /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Decoded ternary weight of row n, column k. */
int oracle_weight(const uint8_t *codes, int64_t K, int64_t n, int64_t k) {
    uint8_t byte = codes[n * (K / 4) + k / 4];
    int c = (byte >> (2 * (int)(k % 4))) & 3;
    return c - 1;
}

/* Per-(m, group) quantisation, natural k order. */
void oracle_quantize(const float *x, int64_t M, int64_t K,
                     int8_t *q, float *s, int32_t *t) {
    int64_t G = K / PQ2_ORACLE_GROUP;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t g = 0; g < G; ++g) {
            const float *xg = x + m * K + g * PQ2_ORACLE_GROUP;
            int8_t *qg = q + m * K + g * PQ2_ORACLE_GROUP;
            float amax = 0.0f;
            for (int i = 0; i < PQ2_ORACLE_GROUP; ++i) {
                float a = fabsf(xg[i]);
                if (a > amax) amax = a;
            }
            float sc = amax / 127.0f;
            int32_t sum = 0;
            for (int i = 0; i < PQ2_ORACLE_GROUP; ++i) {
                int v = 0;
                if (sc != 0.0f) {
                    float r = rintf(xg[i] / sc);   /* default mode: ties to even */
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    v = (int)r;
                }
                qg[i] = (int8_t)v;
                sum += v;
            }
            s[m * G + g] = sc;
            t[m * G + g] = sum;
        }
    }
}

/* Natural order -> plane order: position 32*s+b of a group receives the
 * activation of weight 4*b+s. */
void oracle_plane_order(const int8_t *q, int64_t M, int64_t K, int8_t *qp) {
    int64_t G = K / PQ2_ORACLE_GROUP;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < G; ++g)
            for (int s = 0; s < 4; ++s)
                for (int b = 0; b < 32; ++b)
                    qp[m * K + g * 128 + 32 * s + b] = q[m * K + g * 128 + 4 * b + s];
}

/* D[m][n][g] = sum over the group's k of (c - 1) * q, natural order. */
static int32_t group_dot(const int8_t *q, const uint8_t *codes, int64_t K,
                         int64_t m, int64_t n, int64_t g) {
    int32_t acc = 0;
    for (int64_t k = g * PQ2_ORACLE_GROUP; k < (g + 1) * PQ2_ORACLE_GROUP; ++k)
        acc += oracle_weight(codes, K, n, k) * (int32_t)q[m * K + k];
    return acc;
}

void oracle_group_dots(const int8_t *q, const uint8_t *codes,
                       int64_t M, int64_t N, int64_t K, int32_t *D, int threads) {
    int64_t G = K / PQ2_ORACLE_GROUP;
    set_threads(threads);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t g = 0; g < G; ++g)
                D[(m * N + n) * G + g] = group_dot(q, codes, K, m, n, g);
}

/* One output in float64, plus the sum of |term| used as the error scale. */
static void one_output(const int8_t *q, const float *s, const uint8_t *codes,
                       const uint16_t *ws, int64_t K, int64_t m, int64_t n,
                       double *y, double *tabs) {
    int64_t G = K / PQ2_ORACLE_GROUP;
    double acc = 0.0, mag = 0.0;
    for (int64_t g = 0; g < G; ++g) {
        double term = (double)group_dot(q, codes, K, m, n, g) * (double)s[m * G + g]
                      * oracle_half_to_double(ws[n * G + g]);
        acc += term;
        mag += fabs(term);
    }
    *y = acc;
    *tabs = mag;
}

void oracle_gemm_f64(const int8_t *q, const float *s, const uint8_t *codes,
                     const uint16_t *ws, int64_t M, int64_t N, int64_t K,
                     double *y, double *tabs, int threads) {
    set_threads(threads);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m)
            one_output(q, s, codes, ws, K, m, n, &y[m * N + n], &tabs[m * N + n]);
}

/* Outputs (mm[i], nn[i]) only, for spot checks at sizes where the full
 * product would take too long on the CPU. */
void oracle_gemm_f64_sampled(const int8_t *q, const float *s, const uint8_t *codes,
                             const uint16_t *ws, int64_t M, int64_t N, int64_t K,
                             const int64_t *mm, const int64_t *nn, int64_t P,
                             double *y, double *tabs, int threads) {
    (void)M; (void)N;
    set_threads(threads);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < P; ++i)
        one_output(q, s, codes, ws, K, mm[i], nn[i], &y[i], &tabs[i]);
}

void oracle_group_dots_sampled(const int8_t *q, const uint8_t *codes, int64_t K,
                               const int64_t *mm, const int64_t *nn, int64_t P,
                               int32_t *D, int threads) {
    int64_t G = K / PQ2_ORACLE_GROUP;
    set_threads(threads);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < P; ++i)
        for (int64_t g = 0; g < G; ++g)
            D[i * G + g] = group_dot(q, codes, K, mm[i], nn[i], g);
}
