/*
 * WKV7 state recurrence -- CPU ORACLE (test infrastructure only).
 *
 * Plain, slow, f64 implementation of the RWKV-7 WKV7 recurrence, its exact
 * reverse-mode derivative, and nothing else.  It exists to check the HIP
 * kernels; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may load it.  It shares no code, header or constant with the
 * HIP library.
 *
 * Sources (page title, section):
 *  - "Foundry/cuda_kernels/timemix.cu", the forward driver tm_fwd_device and
 *    kernel k_composites: the WKV7 kernel is handed (r, w, k', v', A, B) with
 *    A = -kk and B = kk*a, token vectors [B][T][H][N], state [B][H][N][N].
 *  - "infotheory .../rwkv7/model.rs", accumulate_token_step_gradients, the
 *    per-head WKV state-backward block: the read-out gradient uses the UPDATED
 *    state (dr = S_new^T dy), the rank-1 term uses the OLD state
 *    (u = S_old kk), and S_new = S_old diag(w) - u (kk*a)^T + v k^T.
 *  With A = -kk and B = kk*a this is, per (b,h), for t = 0..T-1:
 *      sa[i]   = sum_j S[i][j] a_t[j]                 (old state)
 *      S[i][j] = S[i][j] w_t[j] + sa[i] b_t[j] + v_t[i] k_t[j]
 *      y_t[i]  = sum_j S[i][j] r_t[j]                 (updated state)
 *  i indexes values (rows), j indexes keys (columns).
 *
 * The backward is the chain rule of exactly these three lines, run in
 * reverse over a stored history of all T+1 states (no checkpointing, no
 * recompute), so each line can be checked by eye against the forward.
 *
 * Parallelism: OpenMP over independent (b,h) pairs only; the arithmetic of
 * each pair is the serial loop above.
 */
#include <stdlib.h>
#include <string.h>

#define IDX_VEC(b, t, h, T, H, N) ((((size_t)(b) * (T) + (t)) * (H) + (h)) * (size_t)(N))
#define IDX_ST(b, h, H, N) (((size_t)(b) * (H) + (h)) * (size_t)(N) * (size_t)(N))

/* Forward.  s0 may be NULL (zero initial state); y and sT may be NULL. */
int oracle_wkv7_forward(int B, int T, int H, int N,
                        const double *r, const double *w, const double *k,
                        const double *v, const double *a, const double *b,
                        const double *s0, double *y, double *sT)
{
    int fail = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) reduction(| : fail)
    for (int bb = 0; bb < B; bb++) {
        for (int h = 0; h < H; h++) {
            double *S = (double *)malloc((size_t)N * N * sizeof(double));
            double *sa = (double *)malloc((size_t)N * sizeof(double));
            if (!S || !sa) { free(S); free(sa); fail |= 1; continue; }
            if (s0) memcpy(S, s0 + IDX_ST(bb, h, H, N), (size_t)N * N * sizeof(double));
            else memset(S, 0, (size_t)N * N * sizeof(double));
            for (int t = 0; t < T; t++) {
                size_t o = IDX_VEC(bb, t, h, T, H, N);
                for (int i = 0; i < N; i++) {
                    double acc = 0.0;
                    for (int j = 0; j < N; j++) acc += S[i * N + j] * a[o + j];
                    sa[i] = acc;
                }
                for (int i = 0; i < N; i++)
                    for (int j = 0; j < N; j++)
                        S[i * N + j] = S[i * N + j] * w[o + j] + sa[i] * b[o + j] + v[o + i] * k[o + j];
                if (y) {
                    for (int i = 0; i < N; i++) {
                        double acc = 0.0;
                        for (int j = 0; j < N; j++) acc += S[i * N + j] * r[o + j];
                        y[o + i] = acc;
                    }
                }
            }
            if (sT) memcpy(sT + IDX_ST(bb, h, H, N), S, (size_t)N * N * sizeof(double));
            free(S);
            free(sa);
        }
    }
    return fail ? -1 : 0;
}

/*
 * Backward of the forward above for the scalar loss
 *     L = <dy, y> + <dsT, S_T>
 * i.e. dy is dL/dy and dsT (NULL = 0) is dL/dS_T.  Writes dr, dw, dk, dv,
 * da, db ([B][T][H][N]) and ds0 = dL/dS_0 (NULL = not wanted).
 *
 * With G = dL/dS_t (everything downstream of S_t), reverse step t:
 *     G       += dy_t r_t^T                    (y_t = S_t r_t)
 *     dr_t     = S_t^T dy_t
 *     dv_t[i]  = sum_j G[i][j] k_t[j]           (term v_t k_t^T)
 *     dk_t[j]  = sum_i G[i][j] v_t[i]
 *     sa[i]    = sum_j S_{t-1}[i][j] a_t[j]
 *     db_t[j]  = sum_i G[i][j] sa[i]            (term sa b_t^T)
 *     dsa[i]   = sum_j G[i][j] b_t[j]
 *     dw_t[j]  = sum_i G[i][j] S_{t-1}[i][j]    (term S_{t-1} diag(w_t))
 *     da_t[j]  = sum_i dsa[i] S_{t-1}[i][j]     (sa = S_{t-1} a_t)
 *     G       <- G diag(w_t) + dsa a_t^T        (= dL/dS_{t-1})
 */
int oracle_wkv7_backward(int B, int T, int H, int N,
                         const double *r, const double *w, const double *k,
                         const double *v, const double *a, const double *b,
                         const double *s0, const double *dy, const double *dsT,
                         double *dr, double *dw, double *dk, double *dv,
                         double *da, double *db, double *ds0)
{
    int fail = 0;
    const size_t NN = (size_t)N * N;
#pragma omp parallel for collapse(2) schedule(dynamic) reduction(| : fail)
    for (int bb = 0; bb < B; bb++) {
        for (int h = 0; h < H; h++) {
            /* hist[t] = state after t tokens, t = 0..T (hist[0] = s0) */
            double *hist = (double *)malloc((size_t)(T + 1) * NN * sizeof(double));
            double *G = (double *)malloc(NN * sizeof(double));
            double *sa = (double *)malloc((size_t)N * sizeof(double));
            double *dsa = (double *)malloc((size_t)N * sizeof(double));
            if (!hist || !G || !sa || !dsa) {
                free(hist); free(G); free(sa); free(dsa);
                fail |= 1;
                continue;
            }
            if (s0) memcpy(hist, s0 + IDX_ST(bb, h, H, N), NN * sizeof(double));
            else memset(hist, 0, NN * sizeof(double));
            for (int t = 0; t < T; t++) {
                size_t o = IDX_VEC(bb, t, h, T, H, N);
                const double *Sp = hist + (size_t)t * NN;
                double *Sn = hist + (size_t)(t + 1) * NN;
                for (int i = 0; i < N; i++) {
                    double acc = 0.0;
                    for (int j = 0; j < N; j++) acc += Sp[i * N + j] * a[o + j];
                    sa[i] = acc;
                }
                for (int i = 0; i < N; i++)
                    for (int j = 0; j < N; j++)
                        Sn[i * N + j] = Sp[i * N + j] * w[o + j] + sa[i] * b[o + j] + v[o + i] * k[o + j];
            }

            if (dsT) memcpy(G, dsT + IDX_ST(bb, h, H, N), NN * sizeof(double));
            else memset(G, 0, NN * sizeof(double));
            for (int t = T - 1; t >= 0; t--) {
                size_t o = IDX_VEC(bb, t, h, T, H, N);
                const double *Sp = hist + (size_t)t * NN;
                const double *Sn = hist + (size_t)(t + 1) * NN;
                for (int i = 0; i < N; i++)
                    for (int j = 0; j < N; j++) G[i * N + j] += dy[o + i] * r[o + j];
                for (int j = 0; j < N; j++) {
                    double acc = 0.0;
                    for (int i = 0; i < N; i++) acc += Sn[i * N + j] * dy[o + i];
                    dr[o + j] = acc;
                }
                for (int i = 0; i < N; i++) {
                    double acc = 0.0;
                    for (int j = 0; j < N; j++) acc += G[i * N + j] * k[o + j];
                    dv[o + i] = acc;
                }
                for (int j = 0; j < N; j++) {
                    double acc = 0.0;
                    for (int i = 0; i < N; i++) acc += G[i * N + j] * v[o + i];
                    dk[o + j] = acc;
                }
                for (int i = 0; i < N; i++) {
                    double acc = 0.0;
                    for (int j = 0; j < N; j++) acc += Sp[i * N + j] * a[o + j];
                    sa[i] = acc;
                }
                for (int j = 0; j < N; j++) {
                    double acc = 0.0;
                    for (int i = 0; i < N; i++) acc += G[i * N + j] * sa[i];
                    db[o + j] = acc;
                }
                for (int i = 0; i < N; i++) {
                    double acc = 0.0;
                    for (int j = 0; j < N; j++) acc += G[i * N + j] * b[o + j];
                    dsa[i] = acc;
                }
                for (int j = 0; j < N; j++) {
                    double acc = 0.0;
                    for (int i = 0; i < N; i++) acc += G[i * N + j] * Sp[i * N + j];
                    dw[o + j] = acc;
                }
                for (int j = 0; j < N; j++) {
                    double acc = 0.0;
                    for (int i = 0; i < N; i++) acc += dsa[i] * Sp[i * N + j];
                    da[o + j] = acc;
                }
                for (int i = 0; i < N; i++)
                    for (int j = 0; j < N; j++) G[i * N + j] = G[i * N + j] * w[o + j] + dsa[i] * a[o + j];
            }
            if (ds0) memcpy(ds0 + IDX_ST(bb, h, H, N), G, NN * sizeof(double));
            free(hist);
            free(G);
            free(sa);
            free(dsa);
        }
    }
    return fail ? -1 : 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
