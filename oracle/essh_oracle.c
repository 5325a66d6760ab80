/*
 * essh_oracle.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow, sequential CPU oracle for the core of the ESSH selective
 * spectral mixer ("Elastic Selective Spectral Hybrids for Train-Once,
 * Export-Many Budgeted Inference", Sec. 4.1 Eq. 5 and App. B Eq. 9).  Only the
 * tests, the package's smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header or table with the HIP library.
 *
 * What it computes, for every batch row b, retained channel k < K_T, mode j,
 * value coordinate p and position t = 0..L-1 (the paper counts from 1):
 *
 *   Mode state in complex form (App. B.1: a damped rotation rho R(theta)
 *   acting on a 2-vector is multiplication by rho e^{i theta}; injecting
 *   along e_1 adds to the real part; reading with (kc, -ks) is Re(c h) with
 *   c = kc + i ks):
 *
 *     lambda(t) = rho_kj * exp(-delta(t)) * exp(i theta_kj)          (Eq. 5)
 *     h(t)      = lambda(t) * h(t-1) + g_w(t) * v(t)                 (Eq. 5)
 *     y(t)      = sum_j g_r(t) * Re( c_kj * h(t) )                   (Eq. 9 readout)
 *
 *   delta, g_w, g_r are per channel ([B,L,K]) or per mode ([B,L,K,m], the
 *   paper's own granularity, Eq. 5 / App. C.2).  h(-1) is state_in, or zero.
 *   Channels k >= K_T are neither read nor written (truncation, App. C.4).
 *
 *   Optional zero-lag correction (App. C.3, Eq. 24): with coefficients
 *   a [K,m], the output becomes
 *     z(t) = y(t) - sum_j a_kj * g_r(t) * g_w(t) * kc_kj * v(t)
 *   (kc = Re c); without them (NULL) the output is the core readout y.
 *
 * Layouts (row-major):  v, y [B,L,K,P];  delta, g_w, g_r [B,L,K] or
 * [B,L,K,m];  rho, theta [K,m];  c [K,m,2] (re, im);  state [B,K,m,2,P]
 * (planar: real plane then imaginary plane).
 *
 * The same source is compiled twice: with ESSH_REAL=double (the parity
 * oracle) and with ESSH_REAL=float (only for the CPU timing baseline).
 */
#include <complex.h>
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ESSH_REAL
#define ESSH_REAL double
#endif
#ifndef ESSH_SUFFIX
#define ESSH_SUFFIX f64
#endif

typedef ESSH_REAL real;
typedef ESSH_REAL _Complex cplx;

#define CAT2(a, b) a##_##b
#define CAT(a, b) CAT2(a, b)
#define FN(name) CAT(name, ESSH_SUFFIX)

/* type-exact elementary functions (no tgmath tricks, so the float build is
 * really float) */
#if defined(ESSH_FLOAT)
#define R_EXP expf
#define R_COS cosf
#define R_SIN sinf
#define C_RE crealf
#define C_IM cimagf
#else
#define R_EXP exp
#define R_COS cos
#define R_SIN sin
#define C_RE creal
#define C_IM cimag
#endif

/* Number of OpenMP threads the last call used (1 without OpenMP). */
static int g_threads_used = 1;

int FN(essh_oracle_threads_used)(void) { return g_threads_used; }

/*
 * Sequential selective recurrence over one sequence of L positions.
 * Returns 0 on success, -1 on a bad argument, -2 if memory ran out.
 */
int FN(essh_oracle_prefill)(int B, int L, int K, int m, int P, int K_T, int per_mode,
                            const real* v, const real* delta, const real* g_w, const real* g_r,
                            const real* rho, const real* theta, const real* c, const real* zl,
                            const real* state_in, real* state_out, real* y, int nthreads)
{
    if (B < 0 || L < 0 || K < 1 || m < 1 || P < 1 || K_T < 1 || K_T > K) return -1;
    if (nthreads < 1) nthreads = 1;
    int failed = 0;
    g_threads_used = 1;

#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads)
    {
#pragma omp single
        g_threads_used = omp_get_num_threads();
#pragma omp for collapse(2) schedule(dynamic, 1)
#endif
    for (int b = 0; b < B; ++b) {
        for (int k = 0; k < K_T; ++k) {
            cplx* h = (cplx*)malloc(sizeof(cplx) * (size_t)m * (size_t)P);
            real* acc = (real*)malloc(sizeof(real) * (size_t)P);
            if (!h || !acc) {
                free(h);
                free(acc);
#ifdef _OPENMP
#pragma omp atomic write
#endif
                failed = 1;
                continue;
            }
            /* h(-1): the carried state, or zero (Eq. 5: H(0) = 0) */
            for (int j = 0; j < m; ++j)
                for (int p = 0; p < P; ++p) {
                    cplx h0 = 0;
                    if (state_in) {
                        size_t s = (((size_t)b * K + k) * m + j) * 2 * (size_t)P;
                        h0 = state_in[s + p] + I * state_in[s + P + p];
                    }
                    h[(size_t)j * P + p] = h0;
                }

            for (int t = 0; t < L; ++t) {
                size_t row = ((size_t)b * L + t) * K + k;   /* (b, t, k) */
                const real* vt = v + row * P;
                for (int p = 0; p < P; ++p) acc[p] = 0;
                for (int j = 0; j < m; ++j) {
                    size_t ci = per_mode ? row * m + j : row;
                    real rk = rho[(size_t)k * m + j];
                    real th = theta[(size_t)k * m + j];
                    cplx lam = rk * R_EXP(-delta[ci]) * (R_COS(th) + I * R_SIN(th));
                    cplx cc = c[((size_t)k * m + j) * 2] + I * c[((size_t)k * m + j) * 2 + 1];
                    real gw = g_w[ci], gr = g_r[ci];
                    for (int p = 0; p < P; ++p) {
                        cplx hn = lam * h[(size_t)j * P + p] + gw * vt[p];
                        h[(size_t)j * P + p] = hn;
                        acc[p] += gr * C_RE(cc * hn);
                    }
                    if (zl) {   /* Eq. 24: the lag-zero term of this mode, scaled by a */
                        real zc = zl[(size_t)k * m + j] * gr * gw * c[((size_t)k * m + j) * 2];
                        for (int p = 0; p < P; ++p) acc[p] -= zc * vt[p];
                    }
                }
                real* yt = y + row * P;
                for (int p = 0; p < P; ++p) yt[p] = acc[p];
            }

            if (state_out)
                for (int j = 0; j < m; ++j) {
                    size_t s = (((size_t)b * K + k) * m + j) * 2 * (size_t)P;
                    for (int p = 0; p < P; ++p) {
                        cplx hv = h[(size_t)j * P + p];
                        state_out[s + p] = C_RE(hv);
                        state_out[s + P + p] = C_IM(hv);
                    }
                }
            free(h);
            free(acc);
        }
    }
#ifdef _OPENMP
    }
#endif
    return failed ? -2 : 0;
}
