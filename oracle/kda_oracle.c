/*
 * KDA fp64 CPU oracle.  TEST INFRASTRUCTURE ONLY: it is called by the tests,
 * by the smoke check and by the benchmark's CPU-baseline leg, never by the
 * product path.  It shares no source, header, table or helper with the HIP
 * library; the two meet only in the seeded input generators.
 *
 * Sources (cited by page title and section; a reader has the pages):
 *   [K3-notes]  "NLP——技术报告解读-Kimi-K3" (joezjh.github.io), section
 *               Model Architecture / Kimi Delta Attention (KDA): the state
 *               update S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
 *               the read-out o_t = S_t^T q_t, and the lower-bounded decay
 *               g_t^h = g_min * Sigmoid(e^{A_h} z_t^h) with g_min = -5.
 *   [K3-plain]  "Kimi K3 技术报告 · 大白话版" (aicoding.csdn.net), §2.1.1: per
 *               token the board is first decayed channel by channel, then
 *               corrected by the delta rule, then read; at most 99.33% is
 *               forgotten in one step.
 *
 * Everything is computed in double precision.  Layouts (row-major):
 *   q, k, g : [T, H, dk]     v, o : [T, H, dv]     beta : [T, H]
 *   states  : [N, H, dk, dv] (row index = key channel, column = value channel)
 *   cu      : [N + 1] token offsets of the packed sequences, cu[0] = 0.
 *
 * Functions:
 *   oracle_gate            the gate, as the formula states it.
 *   oracle_prefill         the token-serial recurrence (the definition).
 *   oracle_decode_step     one token of the same recurrence per (b, h), in place.
 *   oracle_prefill_chunked the chunkwise form (decay, UT/WY solve, state hand-off)
 *                          in fp64 with every e^{G_r - G_i} taken directly; used
 *                          only to check that chunking changes nothing.
 *   oracle_wy_T            the per-chunk triangular solve alone, for its pin.
 *   oracle_backward        reverse-mode gradients of the token-serial recurrence
 *                          (every state of a sequence is kept: small cases).
 *   oracle_round_bf16      round doubles to the nearest bf16 (ties to even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* [K3-notes] KDA gate: g = g_min * Sigmoid(exp(A_h) * z), per channel. */
void oracle_gate(const double* z, const double* A, int64_t n_tok, int H, int dk,
                 double g_min, double* g)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t)
        for (int h = 0; h < H; ++h) {
            const double s = exp(A[h]);
            const int64_t base = (t * H + h) * (int64_t)dk;
            for (int c = 0; c < dk; ++c) {
                const double x = s * z[base + c];
                g[base + c] = g_min / (1.0 + exp(-x));
            }
        }
}

/* One token of the recurrence ([K3-notes] state update; [K3-plain] §2.1.1
 * order: decay, then delta correction, then read):
 *   S <- Diag(alpha) S,  alpha = exp(g)
 *   u  = beta (v - S^T k)
 *   S <- S + k u^T        (equals (I - beta k k^T) S + beta k v^T)
 *   o  = S^T q            (read after the update)
 * `u` is caller scratch of length dv; `o` may be NULL. */
static void token_step(int dk, int dv, double* S, const double* q, const double* k,
                       const double* v, const double* g, double beta, double* o,
                       double* u)
{
    for (int c = 0; c < dk; ++c) {
        const double a = exp(g[c]);
        double* row = S + (int64_t)c * dv;
        for (int j = 0; j < dv; ++j) row[j] *= a;
    }
    for (int j = 0; j < dv; ++j) u[j] = 0.0;
    for (int c = 0; c < dk; ++c) {
        const double kc = k[c];
        const double* row = S + (int64_t)c * dv;
        for (int j = 0; j < dv; ++j) u[j] += kc * row[j];
    }
    for (int j = 0; j < dv; ++j) u[j] = beta * (v[j] - u[j]);
    for (int c = 0; c < dk; ++c) {
        const double kc = k[c];
        double* row = S + (int64_t)c * dv;
        for (int j = 0; j < dv; ++j) row[j] += kc * u[j];
    }
    if (o) {
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
            const double qc = q[c];
            const double* row = S + (int64_t)c * dv;
            for (int j = 0; j < dv; ++j) o[j] += qc * row[j];
        }
    }
}

static int pick_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* The token-serial recurrence over every packed sequence and head.
 * S0 may be NULL (zero initial states); o and S_final may be NULL. */
void oracle_prefill(const double* q, const double* k, const double* v, const double* g,
                    const double* beta, const int64_t* cu, int N, int H, int dk, int dv,
                    const double* S0, double* o, double* S_final, int nthreads)
{
    const int64_t units = (int64_t)N * H;
    const int64_t ssz = (int64_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int64_t w = 0; w < units; ++w) {
        const int n = (int)(w / H), h = (int)(w % H);
        double* S = (double*)malloc(sizeof(double) * (size_t)(ssz + dv));
        double* u = S + ssz;
        if (S0) memcpy(S, S0 + w * ssz, sizeof(double) * (size_t)ssz);
        else memset(S, 0, sizeof(double) * (size_t)ssz);
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const int64_t th = t * H + h;
            token_step(dk, dv, S, q + th * dk, k + th * dk, v + th * dv, g + th * dk,
                       beta[th], o ? o + th * dv : NULL, u);
        }
        if (S_final) memcpy(S_final + w * ssz, S, sizeof(double) * (size_t)ssz);
        free(S);
    }
}

/* One decode step: each of the B*H states takes one token, in place. */
void oracle_decode_step(const double* q, const double* k, const double* v, const double* g,
                        const double* beta, double* S, double* o, int B, int H, int dk, int dv)
{
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    for (int64_t w = 0; w < (int64_t)B * H; ++w)
        token_step(dk, dv, S + w * dk * dv, q + w * dk, k + w * dk, v + w * dv, g + w * dk,
                   beta[w], o ? o + w * dv : NULL, u);
    free(u);
}

/* Per-chunk UT/WY matrix T = (I + A)^{-1} Diag(beta), with the strictly lower
 * A[r][i] = beta_r * sum_c k[r][c] k[i][c] exp(G[r][c] - G[i][c]) and G the
 * running sum of g inside the chunk.  Forward substitution, column by column.
 * k, g: [L][ld] (row stride ld, first dk used); T: [L][L]. */
static void wy_T(const double* k, const double* g, const double* beta, int L, int dk,
                 int64_t ld, int64_t bstride, double* G, double* A, double* T)
{
    for (int r = 0; r < L; ++r)
        for (int c = 0; c < dk; ++c)
            G[r * dk + c] = g[r * ld + c] + (r ? G[(r - 1) * dk + c] : 0.0);
    for (int r = 0; r < L; ++r)
        for (int i = 0; i < L; ++i) {
            double s = 0.0;
            if (i < r)
                for (int c = 0; c < dk; ++c)
                    s += k[r * ld + c] * k[i * ld + c] * exp(G[r * dk + c] - G[i * dk + c]);
            A[r * L + i] = beta[r * bstride] * s;
        }
    for (int j = 0; j < L; ++j)
        for (int r = 0; r < L; ++r) {
            double x = (r == j) ? beta[j * bstride] : 0.0;
            for (int i = 0; i < r; ++i) x -= A[r * L + i] * T[i * L + j];
            T[r * L + j] = x;
        }
}

void oracle_wy_T(const double* k, const double* g, const double* beta, int L, int dk, double* T)
{
    double* G = (double*)malloc(sizeof(double) * (size_t)L * dk);
    double* A = (double*)malloc(sizeof(double) * (size_t)L * L);
    wy_T(k, g, beta, L, dk, dk, 1, G, A, T);
    free(G);
    free(A);
}

/* The chunkwise form: for each chunk of at most C tokens, with incoming S,
 *   W  = T (K . e^{G}),  U' = T V,  U = U' - W S
 *   P[r][i] = sum_c q[r][c] k[i][c] e^{G[r][c]-G[i][c]}   (i <= r)
 *   O  = (Q . e^{G}) S + P U
 *   S <- Diag(e^{G_last}) S + (K . e^{G_last - G})^T U
 * Chunks restart at every sequence start; the last one may be short. */
void oracle_prefill_chunked(const double* q, const double* k, const double* v,
                            const double* g, const double* beta, const int64_t* cu, int N,
                            int H, int dk, int dv, int C, const double* S0, double* o,
                            double* S_final, int nthreads)
{
    const int64_t units = (int64_t)N * H;
    const int64_t ssz = (int64_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int64_t w = 0; w < units; ++w) {
        const int n = (int)(w / H), h = (int)(w % H);
        const int64_t ld = (int64_t)H * dk, ldv = (int64_t)H * dv;
        double* S = (double*)malloc(sizeof(double) * (size_t)ssz);
        double* G = (double*)malloc(sizeof(double) * (size_t)C * dk);
        double* A = (double*)malloc(sizeof(double) * (size_t)C * C);
        double* T = (double*)malloc(sizeof(double) * (size_t)C * C);
        double* W = (double*)malloc(sizeof(double) * (size_t)C * dk);
        double* U = (double*)malloc(sizeof(double) * (size_t)C * dv);
        double* P = (double*)malloc(sizeof(double) * (size_t)C * C);
        if (S0) memcpy(S, S0 + w * ssz, sizeof(double) * (size_t)ssz);
        else memset(S, 0, sizeof(double) * (size_t)ssz);
        for (int64_t t0 = cu[n]; t0 < cu[n + 1]; t0 += C) {
            const int L = (int)((cu[n + 1] - t0) < C ? (cu[n + 1] - t0) : C);
            const double* kc = k + (t0 * H + h) * dk;
            const double* qc = q + (t0 * H + h) * dk;
            const double* gc = g + (t0 * H + h) * dk;
            const double* vc = v + (t0 * H + h) * dv;
            const double* bc = beta + t0 * H + h;
            wy_T(kc, gc, bc, L, dk, ld, H, G, A, T);
            for (int r = 0; r < L; ++r)
                for (int c = 0; c < dk; ++c) {
                    double s = 0.0;
                    for (int j = 0; j <= r; ++j)
                        s += T[r * L + j] * kc[j * ld + c] * exp(G[j * dk + c]);
                    W[r * dk + c] = s;
                }
            for (int r = 0; r < L; ++r)
                for (int jv = 0; jv < dv; ++jv) {
                    double s = 0.0;
                    for (int i = 0; i <= r; ++i) s += T[r * L + i] * vc[i * ldv + jv];
                    for (int c = 0; c < dk; ++c) s -= W[r * dk + c] * S[c * dv + jv];
                    U[r * dv + jv] = s;
                }
            for (int r = 0; r < L; ++r)
                for (int i = 0; i < L; ++i) {
                    double s = 0.0;
                    if (i <= r)
                        for (int c = 0; c < dk; ++c)
                            s += qc[r * ld + c] * kc[i * ld + c] *
                                 exp(G[r * dk + c] - G[i * dk + c]);
                    P[r * L + i] = s;
                }
            if (o)
                for (int r = 0; r < L; ++r)
                    for (int jv = 0; jv < dv; ++jv) {
                        double s = 0.0;
                        for (int c = 0; c < dk; ++c)
                            s += qc[r * ld + c] * exp(G[r * dk + c]) * S[c * dv + jv];
                        for (int i = 0; i <= r; ++i) s += P[r * L + i] * U[i * dv + jv];
                        o[((t0 + r) * H + h) * dv + jv] = s;
                    }
            for (int c = 0; c < dk; ++c) {
                const double gl = G[(L - 1) * dk + c];
                for (int jv = 0; jv < dv; ++jv) {
                    double s = exp(gl) * S[c * dv + jv];
                    for (int i = 0; i < L; ++i)
                        s += kc[i * ld + c] * exp(gl - G[i * dk + c]) * U[i * dv + jv];
                    S[c * dv + jv] = s;
                }
            }
        }
        if (S_final) memcpy(S_final + w * ssz, S, sizeof(double) * (size_t)ssz);
        free(S); free(G); free(A); free(T); free(W); free(U); free(P);
    }
}

/* Gradients of L = sum_t <dO_t, o_t> + <dS_fin, S_T> through the recurrence
 * of token_step, taken backwards token by token (reverse-mode, the chain rule
 * applied to each line of the step).  With Sp = Diag(a) S_prev, a = exp(g),
 * w = Sp^T k, r = v - w, u = beta r, S = Sp + k u^T, o = S^T q:
 *   dS += q dO^T            dq = S dO
 *   du = dS^T k             dk = dS u
 *   dv = beta du            dbeta = <du, r>
 *   dw = -beta du           dk += Sp dw      dSp = dS + k dw^T
 *   dg_c = a_c <dSp[c,:], S_prev[c,:]>        dS_prev = Diag(a) dSp
 * S0, dO and dS_fin may be NULL (zero).  Every state of a sequence is kept,
 * so memory grows as T dk dv per unit: for small cases. */
void oracle_backward(const double* q, const double* k, const double* v, const double* g,
                     const double* beta, const int64_t* cu, int N, int H, int dk, int dv,
                     const double* S0, const double* dO, const double* dS_fin, double* dq,
                     double* dk_out, double* dv_out, double* dg, double* dbeta, double* dS0,
                     int nthreads)
{
    const int64_t units = (int64_t)N * H;
    const int64_t ssz = (int64_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads))
    for (int64_t w = 0; w < units; ++w) {
        const int n = (int)(w / H), h = (int)(w % H);
        const int64_t T0 = cu[n], L = cu[n + 1] - cu[n];
        /* states[i] = S before token T0 + i, for i = 0 .. L (states[L] = S_T) */
        double* states = (double*)malloc(sizeof(double) * (size_t)((L + 1) * ssz));
        double* dS = (double*)malloc(sizeof(double) * (size_t)(3 * ssz + 4 * dv + dk));
        double* Sp = dS + ssz;
        double* Sc = Sp + ssz;
        double* u = Sc + ssz;
        double* r = u + dv;
        double* du = r + dv;
        double* dw = du + dv;
        double* a = dw + dv;
        if (S0) memcpy(states, S0 + w * ssz, sizeof(double) * (size_t)ssz);
        else memset(states, 0, sizeof(double) * (size_t)ssz);
        for (int64_t i = 0; i < L; ++i) {
            const int64_t th = (T0 + i) * H + h;
            memcpy(states + (i + 1) * ssz, states + i * ssz, sizeof(double) * (size_t)ssz);
            token_step(dk, dv, states + (i + 1) * ssz, q + th * dk, k + th * dk, v + th * dv, g + th * dk,
                       beta[th], NULL, u);
        }
        if (dS_fin) memcpy(dS, dS_fin + w * ssz, sizeof(double) * (size_t)ssz);
        else memset(dS, 0, sizeof(double) * (size_t)ssz);
        for (int64_t i = L - 1; i >= 0; --i) {
            const int64_t th = (T0 + i) * H + h;
            const double* Sprev = states + i * ssz;
            const double *qt = q + th * dk, *kt = k + th * dk, *vt = v + th * dv, *gt = g + th * dk;
            const double bt = beta[th];
            /* forward quantities of this token */
            for (int c = 0; c < dk; ++c) a[c] = exp(gt[c]);
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j) Sp[c * dv + j] = a[c] * Sprev[c * dv + j];
            for (int j = 0; j < dv; ++j) {
                double wj = 0.0;
                for (int c = 0; c < dk; ++c) wj += kt[c] * Sp[c * dv + j];
                r[j] = vt[j] - wj;
                u[j] = bt * r[j];
            }
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j) Sc[c * dv + j] = Sp[c * dv + j] + kt[c] * u[j];
            /* o = S^T q */
            if (dO) {
                const double* dOt = dO + th * dv;
                for (int c = 0; c < dk; ++c) {
                    double s = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        dS[c * dv + j] += qt[c] * dOt[j];
                        s += Sc[c * dv + j] * dOt[j];
                    }
                    dq[th * dk + c] = s;
                }
            } else {
                for (int c = 0; c < dk; ++c) dq[th * dk + c] = 0.0;
            }
            /* S = Sp + k u^T */
            for (int j = 0; j < dv; ++j) {
                double s = 0.0;
                for (int c = 0; c < dk; ++c) s += kt[c] * dS[c * dv + j];
                du[j] = s;
            }
            double db = 0.0;
            for (int j = 0; j < dv; ++j) {
                dv_out[th * dv + j] = bt * du[j];
                db += du[j] * r[j];
                dw[j] = -bt * du[j];
            }
            dbeta[th] = db;
            for (int c = 0; c < dk; ++c) {
                double s = 0.0;
                for (int j = 0; j < dv; ++j) s += dS[c * dv + j] * u[j] + Sp[c * dv + j] * dw[j];
                dk_out[th * dk + c] = s;
            }
            /* dSp = dS + k dw^T; then through Sp = Diag(a) S_prev */
            for (int c = 0; c < dk; ++c) {
                double s = 0.0;
                for (int j = 0; j < dv; ++j) {
                    const double dsp = dS[c * dv + j] + kt[c] * dw[j];
                    s += dsp * Sprev[c * dv + j];
                    dS[c * dv + j] = a[c] * dsp;
                }
                dg[th * dk + c] = a[c] * s;
            }
        }
        memcpy(dS0 + w * ssz, dS, sizeof(double) * (size_t)ssz);
        free(dS);
        free(states);
    }
}

/* Nearest bf16 value (8 significant bits, ties to even), computed from the
 * double directly so no intermediate float rounding intervenes. */
void oracle_round_bf16(double* x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        const double v = x[i];
        if (v == 0.0 || !isfinite(v)) continue;
        int e;
        frexp(v, &e); /* v = m * 2^e, 0.5 <= |m| < 1 */
        int sc = e - 8;
        if (sc < -133) sc = -133; /* bf16 subnormal spacing */
        x[i] = ldexp(nearbyint(ldexp(v, -sc)), sc);
    }
}
