/*
 * CPU oracle for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain fp64 reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and the
 * CPU leg of the benchmark may load it.  It shares no code, header, table or
 * helper with the GPU library, and the GPU library never calls it.
 *
 * Sources.  The pages ("cuLA PR #131: SM100/SM103 KDA forward to pure CuTeDSL",
 * sections Summary and Numerical behavior; "cuLA REPO_LAYOUT.md", the kda/ and
 * ops/ directory entries for chunk_delta_h and fwd_o) name the method and its
 * stages (gate cumsum, chunk intra with per-channel decay, causal mask and beta
 * scaling, FP32 inversion of the Akk system, recompute of W and U, the chunk
 * delta-H state scan and the forward output) but print no equation.  The
 * recurrence implemented here is the plain KDA (gated delta rule with a
 * per-channel decay) reading, for every sequence n and value head hv:
 *
 *     S_t = (I - alpha_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * with alpha_t = beta_t for KDA.  alpha is a separate argument only so that the
 * tests can switch the erase term off and compare with quadratic gated linear
 * attention.  S is dk x dv; the decay scales the rows (key channels).
 *
 * Two evaluations are provided:
 *   kda_oracle_recurrence  token by token (the definition itself);
 *   kda_oracle_chunked     the chunked (WY / UT) form, derived from the
 *                          recurrence, with every intermediate of the chunked
 *                          method optionally returned:
 *       G     chunk-local inclusive cumsum of g
 *       Aqk   scale * sum_c q_i k_j exp(G_i - G_j), j <= i
 *       Akk   beta_i * sum_c k_i k_j exp(G_i - G_j), j < i
 *       T     (I + Akk)^{-1} (forward substitution)
 *       W     T (beta k exp(G)),  U = T (beta v)
 *       v_new U - W h
 *       o     (scale q exp(G)) h + Aqk v_new
 *       h'    Diag(exp G_last) h + (k exp(G_last - G))^T v_new
 *
 * Layout (all arrays row-major, token-major, sequences packed back to back):
 *   q, k   [Ttot][Hq][dk]       v     [Ttot][Hv][dv]
 *   g      [Ttot][Hv][dk]       beta  [Ttot][Hv]       alpha [Ttot][Hv] or NULL
 *   cu     [N+1] token offsets (non-decreasing, cu[0] = 0, cu[N] = Ttot)
 *   h0     [N][Hv][dk][dv] or NULL (zero)
 *   o      [Ttot][Hv][dv]       hT    [N][Hv][dk][dv]
 * Grouped-value heads: value head hv reads q/k head hv / (Hv / Hq).
 * Partial chunks: a sequence is cut into chunks of C tokens from its own start;
 * the last chunk may be shorter.
 *
 * A third function gives the optional QG output of the forward:
 *   kda_oracle_qg          qg[t][hv][c] = q[t][hq(hv)][c] * exp(G[t][hv][c]), G the
 *                          chunk-local inclusive cumsum of g.  The pages ("cuLA PR
 *                          #131", Summary, and the Changes table of its walkthrough)
 *                          list an optional QG output of the intra and recompute
 *                          paths without defining it; this is the decayed query the
 *                          output product uses, before the scale.
 *
 * Every function returns 0 on success and -1 on invalid sizes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of OpenMP threads the oracle's parallel loops use. */
int kda_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int check_sizes(int64_t N, int64_t Hq, int64_t Hv, int64_t dk, int64_t dv, const int64_t* cu) {
    if (N < 0 || Hq <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hq != 0 || !cu) return -1;
    if (cu[0] != 0) return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    return 0;
}

/* Token-by-token recurrence.  One (sequence, value head) pair per OpenMP task. */
int kda_oracle_recurrence(const double* q, const double* k, const double* v, const double* g,
                          const double* beta, const double* alpha, double scale,
                          const int64_t* cu, int64_t N, int64_t Hq, int64_t Hv, int64_t dk,
                          int64_t dv, const double* h0, double* o, double* hT) {
    if (check_sizes(N, Hq, Hv, dk, dv, cu)) return -1;
    const int64_t group = Hv / Hq;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < N * Hv; ++task) {
        const int64_t n = task / Hv, hv = task % Hv, hq = hv / group;
        double* S = (double*)malloc(sizeof(double) * dk * dv);
        double* kS = (double*)malloc(sizeof(double) * dv);
        if (!S || !kS) {
            free(S);
            free(kS);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        if (h0)
            memcpy(S, h0 + (n * Hv + hv) * dk * dv, sizeof(double) * dk * dv);
        else
            memset(S, 0, sizeof(double) * dk * dv);
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const double* qt = q + (t * Hq + hq) * dk;
            const double* kt = k + (t * Hq + hq) * dk;
            const double* vt = v + (t * Hv + hv) * dv;
            const double* gt = g + (t * Hv + hv) * dk;
            const double bt = beta[t * Hv + hv];
            const double at = alpha ? alpha[t * Hv + hv] : bt;
            /* S <- Diag(exp g_t) S */
            for (int64_t c = 0; c < dk; ++c) {
                const double d = exp(gt[c]);
                for (int64_t e = 0; e < dv; ++e) S[c * dv + e] *= d;
            }
            /* kS = k_t^T S */
            for (int64_t e = 0; e < dv; ++e) kS[e] = 0.0;
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t e = 0; e < dv; ++e) kS[e] += kt[c] * S[c * dv + e];
            /* S <- S - alpha k (k^T S) + beta k v^T */
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t e = 0; e < dv; ++e)
                    S[c * dv + e] += kt[c] * (bt * vt[e] - at * kS[e]);
            /* o_t = scale S^T q_t */
            double* ot = o + (t * Hv + hv) * dv;
            for (int64_t e = 0; e < dv; ++e) {
                double acc = 0.0;
                for (int64_t c = 0; c < dk; ++c) acc += S[c * dv + e] * qt[c];
                ot[e] = scale * acc;
            }
        }
        memcpy(hT + (n * Hv + hv) * dk * dv, S, sizeof(double) * dk * dv);
        free(S);
        free(kS);
    }
    return bad ? -1 : 0;
}

/* Number of chunks of C tokens needed for every sequence, and their total. */
int64_t kda_oracle_num_chunks(const int64_t* cu, int64_t N, int64_t C) {
    int64_t total = 0;
    for (int64_t n = 0; n < N; ++n) total += (cu[n + 1] - cu[n] + C - 1) / C;
    return total;
}

/*
 * Chunked form.  Optional intermediate outputs (any may be NULL):
 *   G_out   [Ttot][Hv][dk]     chunk-local inclusive cumsum of g
 *   Aqk_out [Ttot][Hv][C]      row of Aqk for the token's position in its chunk
 *   Akk_out [Ttot][Hv][C]      row of Akk (strictly lower)
 *   T_out   [Ttot][Hv][C]      row of T = (I + Akk)^{-1}
 *   W_out   [Ttot][Hv][dk]     U_out [Ttot][Hv][dv]     vnew_out [Ttot][Hv][dv]
 *   hc_out  [num_chunks][Hv][dk][dv]  state entering each chunk, chunks numbered
 *           in sequence order, then chunk order
 * Columns of Aqk/Akk/T beyond the chunk's length are zero.
 */
int kda_oracle_chunked(const double* q, const double* k, const double* v, const double* g,
                       const double* beta, double scale, const int64_t* cu, int64_t N,
                       int64_t Hq, int64_t Hv, int64_t dk, int64_t dv, int64_t C,
                       const double* h0, double* o, double* hT, double* G_out,
                       double* Aqk_out, double* Akk_out, double* T_out, double* W_out,
                       double* U_out, double* vnew_out, double* hc_out) {
    if (check_sizes(N, Hq, Hv, dk, dv, cu) || C <= 0) return -1;
    const int64_t group = Hv / Hq;
    int64_t* chunk_base = (int64_t*)malloc(sizeof(int64_t) * (N + 1));
    if (!chunk_base) return -1;
    chunk_base[0] = 0;
    for (int64_t n = 0; n < N; ++n) chunk_base[n + 1] = chunk_base[n] + (cu[n + 1] - cu[n] + C - 1) / C;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < N * Hv; ++task) {
        const int64_t n = task / Hv, hv = task % Hv, hq = hv / group;
        double* h = (double*)malloc(sizeof(double) * dk * dv);
        double* G = (double*)malloc(sizeof(double) * C * dk);
        double* Aqk = (double*)malloc(sizeof(double) * C * C);
        double* Akk = (double*)malloc(sizeof(double) * C * C);
        double* T = (double*)malloc(sizeof(double) * C * C);
        double* W = (double*)malloc(sizeof(double) * C * dk);
        double* U = (double*)malloc(sizeof(double) * C * dv);
        double* VN = (double*)malloc(sizeof(double) * C * dv);
        if (!h || !G || !Aqk || !Akk || !T || !W || !U || !VN) {
#pragma omp atomic write
            bad = 1;
            goto done;
        }
        if (h0)
            memcpy(h, h0 + (n * Hv + hv) * dk * dv, sizeof(double) * dk * dv);
        else
            memset(h, 0, sizeof(double) * dk * dv);
        for (int64_t start = cu[n], ci = 0; start < cu[n + 1]; start += C, ++ci) {
            const int64_t L = (cu[n + 1] - start < C) ? cu[n + 1] - start : C;
#define Q(i, c) q[((start + (i)) * Hq + hq) * dk + (c)]
#define K(i, c) k[((start + (i)) * Hq + hq) * dk + (c)]
#define V(i, e) v[((start + (i)) * Hv + hv) * dv + (e)]
#define BETA(i) beta[(start + (i)) * Hv + hv]
            if (hc_out)
                memcpy(hc_out + ((chunk_base[n] + ci) * Hv + hv) * dk * dv, h, sizeof(double) * dk * dv);
            /* gate cumsum, restarted at the chunk start */
            for (int64_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int64_t i = 0; i < L; ++i) {
                    acc += g[((start + i) * Hv + hv) * dk + c];
                    G[i * dk + c] = acc;
                }
            }
            /* intra-chunk Aqk (diagonal included) and Akk (strictly lower) */
            for (int64_t i = 0; i < L; ++i)
                for (int64_t j = 0; j < L; ++j) {
                    double sq = 0.0, sk = 0.0;
                    if (j <= i)
                        for (int64_t c = 0; c < dk; ++c) {
                            const double d = exp(G[i * dk + c] - G[j * dk + c]);
                            sq += Q(i, c) * K(j, c) * d;
                            sk += K(i, c) * K(j, c) * d;
                        }
                    Aqk[i * C + j] = (j <= i) ? scale * sq : 0.0;
                    Akk[i * C + j] = (j < i) ? BETA(i) * sk : 0.0;
                }
            /* T = (I + Akk)^{-1} by forward substitution, row by row */
            for (int64_t i = 0; i < L; ++i)
                for (int64_t j = 0; j < L; ++j) {
                    double acc = (i == j) ? 1.0 : 0.0;
                    for (int64_t m = j; m < i; ++m) acc -= Akk[i * C + m] * T[m * C + j];
                    T[i * C + j] = (j <= i) ? acc : 0.0;
                }
            /* W = T (beta k exp G),  U = T (beta v) */
            for (int64_t i = 0; i < L; ++i) {
                for (int64_t c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int64_t j = 0; j <= i; ++j) acc += T[i * C + j] * BETA(j) * K(j, c) * exp(G[j * dk + c]);
                    W[i * dk + c] = acc;
                }
                for (int64_t e = 0; e < dv; ++e) {
                    double acc = 0.0;
                    for (int64_t j = 0; j <= i; ++j) acc += T[i * C + j] * BETA(j) * V(j, e);
                    U[i * dv + e] = acc;
                }
            }
            /* v_new = U - W h */
            for (int64_t i = 0; i < L; ++i)
                for (int64_t e = 0; e < dv; ++e) {
                    double acc = U[i * dv + e];
                    for (int64_t c = 0; c < dk; ++c) acc -= W[i * dk + c] * h[c * dv + e];
                    VN[i * dv + e] = acc;
                }
            /* o = (scale q exp G) h + Aqk v_new */
            for (int64_t i = 0; i < L; ++i)
                for (int64_t e = 0; e < dv; ++e) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < dk; ++c) acc += scale * Q(i, c) * exp(G[i * dk + c]) * h[c * dv + e];
                    for (int64_t j = 0; j <= i; ++j) acc += Aqk[i * C + j] * VN[j * dv + e];
                    o[((start + i) * Hv + hv) * dv + e] = acc;
                }
            /* h <- Diag(exp G_last) h + (k exp(G_last - G))^T v_new */
            for (int64_t c = 0; c < dk; ++c) {
                const double glast = G[(L - 1) * dk + c];
                const double dl = exp(glast);
                for (int64_t e = 0; e < dv; ++e) {
                    double acc = dl * h[c * dv + e];
                    for (int64_t j = 0; j < L; ++j) acc += K(j, c) * exp(glast - G[j * dk + c]) * VN[j * dv + e];
                    h[c * dv + e] = acc;
                }
            }
            /* optional intermediates, token-major */
            for (int64_t i = 0; i < L; ++i) {
                const int64_t row = (start + i) * Hv + hv;
                if (G_out) memcpy(G_out + row * dk, G + i * dk, sizeof(double) * dk);
                if (Aqk_out) for (int64_t j = 0; j < C; ++j) Aqk_out[row * C + j] = (j < L) ? Aqk[i * C + j] : 0.0;
                if (Akk_out) for (int64_t j = 0; j < C; ++j) Akk_out[row * C + j] = (j < L) ? Akk[i * C + j] : 0.0;
                if (T_out) for (int64_t j = 0; j < C; ++j) T_out[row * C + j] = (j < L) ? T[i * C + j] : 0.0;
                if (W_out) memcpy(W_out + row * dk, W + i * dk, sizeof(double) * dk);
                if (U_out) memcpy(U_out + row * dv, U + i * dv, sizeof(double) * dv);
                if (vnew_out) memcpy(vnew_out + row * dv, VN + i * dv, sizeof(double) * dv);
            }
#undef Q
#undef K
#undef V
#undef BETA
        }
        memcpy(hT + (n * Hv + hv) * dk * dv, h, sizeof(double) * dk * dv);
    done:
        free(h);
        free(G);
        free(Aqk);
        free(Akk);
        free(T);
        free(W);
        free(U);
        free(VN);
    }
    free(chunk_base);
    return bad ? -1 : 0;
}

/* qg = q exp(G) per token, value head and key channel, with G the inclusive cumsum
 * of g over the token's chunk (chunks of C tokens from each sequence's start).
 * qg is [Ttot][Hv][dk]; tokens in no sequence are left as they are. */
int kda_oracle_qg(const double* q, const double* g, const int64_t* cu, int64_t N, int64_t Hq, int64_t Hv,
                  int64_t dk, int64_t C, double* qg) {
    if (check_sizes(N, Hq, Hv, dk, 1, cu) != 0 || C <= 0) return -1;
    const int64_t group = Hv / Hq;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t hv = 0; hv < Hv; ++hv)
            for (int64_t c = 0; c < dk; ++c) {
                const int64_t hq = hv / group;
                double G = 0.0;
                for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
                    if ((t - cu[n]) % C == 0) G = 0.0;   /* a chunk starts: the cumsum restarts */
                    G += g[(t * Hv + hv) * dk + c];
                    qg[(t * Hv + hv) * dk + c] = q[(t * Hq + hq) * dk + c] * exp(G);
                }
            }
    return 0;
}
