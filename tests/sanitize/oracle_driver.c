/* Drives every entry point of the fp64 oracle (oracle/kda_oracle.c, linked
 * in) on small ragged inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Checks two identities the oracle must satisfy
 * on the way: the chunkwise form equals the token-serial recurrence, and T
 * decode steps equal a T-token prefill.  Exit status 0 when both hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_gate(const double* z, const double* A, int64_t n_tok, int H, int dk, double g_min, double* g);
void oracle_prefill(const double* q, const double* k, const double* v, const double* g, const double* beta,
                    const int64_t* cu, int N, int H, int dk, int dv, const double* S0, double* o, double* S_final,
                    int nthreads);
void oracle_decode_step(const double* q, const double* k, const double* v, const double* g, const double* beta,
                        double* S, double* o, int B, int H, int dk, int dv);
void oracle_wy_T(const double* k, const double* g, const double* beta, int L, int dk, double* T);
void oracle_prefill_chunked(const double* q, const double* k, const double* v, const double* g,
                            const double* beta, const int64_t* cu, int N, int H, int dk, int dv, int C,
                            const double* S0, double* o, double* S_final, int nthreads);
void oracle_backward(const double* q, const double* k, const double* v, const double* g, const double* beta,
                     const int64_t* cu, int N, int H, int dk, int dv, const double* S0, const double* dO,
                     const double* dS_fin, double* dq, double* dk_out, double* dv_out, double* dg, double* dbeta,
                     double* dS0, int nthreads);
void oracle_round_bf16(double* x, int64_t n);

static uint64_t st = 88172645463325252ull;
static double uni(void) /* xorshift64, uniform in (-1, 1) */
{
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (double)(st >> 11) / 4503599627370496.0 - 1.0;
}
static double* arr(int64_t n, double scale)
{
    double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = scale * uni();
    return p;
}
static double maxdiff(const double* a, const double* b, int64_t n)
{
    double m = 0;
    for (int64_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
    return m;
}

int main(void)
{
    enum { N = 3, H = 2, DK = 8, DV = 4 };
    const int64_t cu[N + 1] = {0, 21, 21, 40}; /* a ragged, an empty and another sequence */
    const int64_t T = cu[N];
    double *q = arr(T * H * DK, 0.5), *k = arr(T * H * DK, 0.5), *v = arr(T * H * DV, 1.0);
    double *z = arr(T * H * DK, 2.0), *beta = arr(T * H, 0.5), *A = arr(H, 1.0);
    for (int64_t i = 0; i < T * H; ++i) beta[i] = 0.5 + 0.5 * beta[i];
    double* g = arr(T * H * DK, 0);
    oracle_gate(z, A, T, H, DK, -5.0, g);
    double* S0 = arr((int64_t)N * H * DK * DV, 0.1);
    double *o1 = arr(T * H * DV, 0), *o2 = arr(T * H * DV, 0);
    double *S1 = arr((int64_t)N * H * DK * DV, 0), *S2 = arr((int64_t)N * H * DK * DV, 0);
    oracle_prefill(q, k, v, g, beta, cu, N, H, DK, DV, S0, o1, S1, 2);
    oracle_prefill(q, k, v, g, beta, cu, N, H, DK, DV, NULL, NULL, S2, 1);
    oracle_prefill_chunked(q, k, v, g, beta, cu, N, H, DK, DV, 16, S0, o2, S2, 2);
    const double e_chunk = fmax(maxdiff(o1, o2, T * H * DV), maxdiff(S1, S2, (int64_t)N * H * DK * DV));
    /* decode: sequence 0 token by token from its initial states */
    double* Sd = arr((int64_t)H * DK * DV, 0);
    for (int64_t i = 0; i < (int64_t)H * DK * DV; ++i) Sd[i] = S0[i];
    double* od = arr(H * DV, 0);
    double e_dec = 0;
    for (int64_t t = cu[0]; t < cu[1]; ++t) {
        oracle_decode_step(q + t * H * DK, k + t * H * DK, v + t * H * DV, g + t * H * DK, beta + t * H, Sd, od, 1,
                           H, DK, DV);
        e_dec = fmax(e_dec, maxdiff(od, o1 + t * H * DV, H * DV));
    }
    e_dec = fmax(e_dec, maxdiff(Sd, S1, (int64_t)H * DK * DV));
    double* Tm = arr(16 * 16, 0);
    oracle_wy_T(k, g, beta, 16, DK, Tm);
    double *dO = arr(T * H * DV, 1.0), *dSf = arr((int64_t)N * H * DK * DV, 1.0);
    double *dq = arr(T * H * DK, 0), *dk = arr(T * H * DK, 0), *dv = arr(T * H * DV, 0), *dg = arr(T * H * DK, 0);
    double *db = arr(T * H, 0), *dS0 = arr((int64_t)N * H * DK * DV, 0);
    oracle_backward(q, k, v, g, beta, cu, N, H, DK, DV, S0, dO, dSf, dq, dk, dv, dg, db, dS0, 2);
    oracle_backward(q, k, v, g, beta, cu, N, H, DK, DV, NULL, NULL, NULL, dq, dk, dv, dg, db, dS0, 1);
    oracle_round_bf16(o1, T * H * DV);
    int finite = 1;
    for (int64_t i = 0; i < T * H * DK; ++i) finite &= isfinite(dq[i]) && isfinite(dg[i]);
    printf("oracle driver: chunked vs serial %.3e, decode vs prefill %.3e, gradients finite %d\n", e_chunk, e_dec,
           finite);
    free(q); free(k); free(v); free(z); free(beta); free(A); free(g); free(S0); free(o1); free(o2); free(S1);
    free(S2); free(Sd); free(od); free(Tm); free(dO); free(dSf); free(dq); free(dk); free(dv); free(dg); free(db);
    free(dS0);
    return (e_chunk < 1e-12 && e_dec < 1e-12 && finite) ? 0 : 1;
}
