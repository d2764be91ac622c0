/*
 * flare_oracle.c -- plain, slow, fp64 CPU oracle of the FLARE / FLARE++
 * routing forward.  TEST INFRASTRUCTURE ONLY: it is called by the tests, by
 * the smoke check and by the CPU-baseline leg of the benchmark, never by the
 * product path, and it shares no code with the GPU library.
 *
 * What it computes (FLARE++ paper, "FLARE++: Low-rank attention with
 * attention-synthesized routing"):
 *   SDPA(Q,K,V) = softmax(Q K^T / sqrt(D)) V, softmax row-wise    (Sec. 3.1)
 *   FLARE:   Z_h = SDPA(Q_h, K_h, V_h)   (M latents, softmax over N tokens)
 *            Y_h = SDPA(K_h, Q_h, Z_h)   (N tokens, softmax over M latents)
 *                                                        (App. A.1, Table 2)
 *   FLARE++: Q^d_h = SDPA(Qs_h, Ks_h, Vs_h);  Q_h = Qf_h + g_h Q^d_h
 *            followed by the FLARE pair with Q_h          (App. A.1, A.4)
 *   The encoder also returns the log-normaliser
 *            L_m = log sum_n exp(s q_m . k_n)             (App. B.2)
 *   and a row with no keys returns L = -inf, Z = 0        (App. B.3)
 *
 * Everything is the plain definition in double precision: for each output
 * row the scores are formed, their maximum taken (a stability shift only,
 * App. B.3), and the exponentials and weighted sums accumulated sequentially
 * in ascending index order.  OpenMP (when enabled) only distributes
 * independent rows, so results do not depend on the thread count.
 *
 * Layouts (all contiguous, D innermost):
 *   K, V            [B,H,N,D]
 *   Q               [H,M,D] when q_batched == 0, else [B,H,M,D]
 *   Z               [B,H,M,D];  L [B,H,M];  Y [B,H,N,D]
 * scale <= 0 selects s = 1/sqrt(D).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

static double pick_scale(double scale, int D) { return scale > 0.0 ? scale : 1.0 / sqrt((double)D); }

static const double* q_ptr(const double* Q, int q_batched, int b, int h, int H, int M, int D) {
    size_t head = q_batched ? (size_t)b * H + h : (size_t)h;
    return Q + head * (size_t)M * D;
}

static double dot(const double* a, const double* b, int D) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += a[d] * b[d];
    return acc;
}

/* Encoder, one latent row: z[d] = sum_n softmax_n(t)_n v_n[d], with
 * t_n = s q . k_n; returns L = log sum_n exp(t_n).  Two passes over the
 * tokens (maximum, then sums). */
static double encode_row(const double* q, const double* K, const double* V, int N, int D, double s,
                         double* z) {
    for (int d = 0; d < D; ++d) z[d] = 0.0;
    if (N <= 0) return -INFINITY;
    double a = -INFINITY;
    for (int n = 0; n < N; ++n) {
        double t = s * dot(q, K + (size_t)n * D, D);
        if (t > a) a = t;
    }
    double l = 0.0;
    for (int n = 0; n < N; ++n) {
        double w = exp(s * dot(q, K + (size_t)n * D, D) - a);
        l += w;
        const double* v = V + (size_t)n * D;
        for (int d = 0; d < D; ++d) z[d] += w * v[d];
    }
    for (int d = 0; d < D; ++d) z[d] /= l;
    return a + log(l);
}

/* Decoder, one token row: y[d] = sum_m softmax_m(u)_m z_m[d], with
 * u_m = s k . q_m (the decoder's query is the token key, its keys are the
 * latent queries and its values the latents). */
static void decode_row(const double* k, const double* Q, const double* Z, int M, int D, double s,
                       double* y, double* u) {
    double c = -INFINITY;
    for (int m = 0; m < M; ++m) {
        u[m] = s * dot(k, Q + (size_t)m * D, D);
        if (u[m] > c) c = u[m];
    }
    double l = 0.0;
    for (int d = 0; d < D; ++d) y[d] = 0.0;
    for (int m = 0; m < M; ++m) {
        double w = exp(u[m] - c);
        l += w;
        const double* zm = Z + (size_t)m * D;
        for (int d = 0; d < D; ++d) y[d] += w * zm[d];
    }
    for (int d = 0; d < D; ++d) y[d] /= l;
}

int oracle_encode(const double* Q, int q_batched, const double* K, const double* V, int B, int H, int N,
                  int M, int D, double scale, double* Z, double* L) {
    if (B <= 0 || H <= 0 || N < 0 || M <= 0 || D <= 0) return 1;
    const double s = pick_scale(scale, D);
    const long rows = (long)B * H * M;
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < rows; ++r) {
        int m = (int)(r % M);
        int bh = (int)(r / M);
        int b = bh / H, h = bh % H;
        const double* q = q_ptr(Q, q_batched, b, h, H, M, D) + (size_t)m * D;
        const double* Kh = K + (size_t)bh * N * D;
        const double* Vh = V + (size_t)bh * N * D;
        double lse = encode_row(q, Kh, Vh, N, D, s, Z + (size_t)r * D);
        if (L) L[r] = lse;
    }
    return 0;
}

/* Decoder over a list of token indices (all tokens when idx == NULL, then
 * count must equal N).  Y rows are written in list order: Y is
 * [B,H,count,D]. */
int oracle_decode_rows(const double* Q, int q_batched, const double* K, const double* Z, int B, int H,
                       int N, int M, int D, double scale, const long* idx, long count, double* Y) {
    if (B <= 0 || H <= 0 || N < 0 || M <= 0 || D <= 0 || count < 0) return 1;
    if (!idx && count != N) return 1;
    if (count == 0) return 0; /* no token rows (also every N = 0 call) */
    if (N == 0) return 1;     /* indices into an empty token axis */
    const double s = pick_scale(scale, D);
    const long rows = (long)B * H * count;
    int bad = 0;
#pragma omp parallel
    {
        double* u = (double*)malloc(sizeof(double) * (size_t)M);
        if (!u) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (long r = 0; r < rows; ++r) {
                long i = r % count;
                int bh = (int)(r / count);
                int b = bh / H, h = bh % H;
                long n = idx ? idx[i] : i;
                if (n < 0 || n >= N) continue;
                const double* k = K + ((size_t)bh * N + (size_t)n) * D;
                decode_row(k, q_ptr(Q, q_batched, b, h, H, M, D), Z + (size_t)bh * M * D, M, D, s,
                           Y + (size_t)r * D, u);
            }
            free(u);
        }
    }
    return bad;
}

int oracle_decode(const double* Q, int q_batched, const double* K, const double* Z, int B, int H, int N,
                  int M, int D, double scale, double* Y) {
    return oracle_decode_rows(Q, q_batched, K, Z, B, H, N, M, D, scale, NULL, N, Y);
}

/* FLARE: encode then decode with the same latent queries. */
int oracle_flare_forward(const double* Q, int q_batched, const double* K, const double* V, int B, int H,
                         int N, int M, int D, double scale, double* Y, double* Z, double* L) {
    int rc = oracle_encode(Q, q_batched, K, V, B, H, N, M, D, scale, Z, L);
    if (rc) return rc;
    return oracle_decode(Q, q_batched, K, Z, B, H, N, M, D, scale, Y);
}

/* FLARE++ query synthesis: Qout[b,h] = Qf[h] + gate[h] * SDPA(Qs[h], Ks[b,h], Vs[b,h]).
 * Qs and Qf are [H,M,D]; Qout is [B,H,M,D]. */
int oracle_pp_queries(const double* Qs, const double* Ks, const double* Vs, const double* Qf,
                      const double* gate, int B, int H, int N, int M, int D, double scale, double* Qout) {
    int rc = oracle_encode(Qs, 0, Ks, Vs, B, H, N, M, D, scale, Qout, NULL);
    if (rc) return rc;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            double* qb = Qout + ((size_t)b * H + h) * (size_t)M * D;
            const double* qf = Qf + (size_t)h * M * D;
            for (long i = 0; i < (long)M * D; ++i) qb[i] = qf[i] + gate[h] * qb[i];
        }
    return 0;
}

/* FLARE++: synthesis, then the FLARE pair with the per-batch queries. */
int oracle_flare_pp_forward(const double* Qs, const double* Ks, const double* Vs, const double* Qf,
                            const double* gate, const double* K, const double* V, int B, int H, int N,
                            int M, int D, double scale, double* Y, double* Qout, double* Z, double* L) {
    int rc = oracle_pp_queries(Qs, Ks, Vs, Qf, gate, B, H, N, M, D, scale, Qout);
    if (rc) return rc;
    return oracle_flare_forward(Qout, 1, K, V, B, H, N, M, D, scale, Y, Z, L);
}

/* Materialised weights of one head (tiny inputs only):
 *   Wenc [M,N] = softmax over n of s Q K^T   (rows sum to 1)
 *   Wdec [N,M] = softmax over m of s K Q^T   (rows sum to 1)
 * so that Z = Wenc V and Y = Wdec Z = (Wdec Wenc) V. */
int oracle_materialize(const double* Q, const double* K, int N, int M, int D, double scale, double* Wenc,
                       double* Wdec) {
    if (N <= 0 || M <= 0 || D <= 0) return 1;
    const double s = pick_scale(scale, D);
    for (int m = 0; m < M; ++m) {
        double a = -INFINITY, l = 0.0;
        for (int n = 0; n < N; ++n) {
            double t = s * dot(Q + (size_t)m * D, K + (size_t)n * D, D);
            Wenc[(size_t)m * N + n] = t;
            if (t > a) a = t;
        }
        for (int n = 0; n < N; ++n) {
            double w = exp(Wenc[(size_t)m * N + n] - a);
            Wenc[(size_t)m * N + n] = w;
            l += w;
        }
        for (int n = 0; n < N; ++n) Wenc[(size_t)m * N + n] /= l;
    }
    for (int n = 0; n < N; ++n) {
        double c = -INFINITY, l = 0.0;
        for (int m = 0; m < M; ++m) {
            double u = s * dot(K + (size_t)n * D, Q + (size_t)m * D, D);
            Wdec[(size_t)n * M + m] = u;
            if (u > c) c = u;
        }
        for (int m = 0; m < M; ++m) {
            double w = exp(Wdec[(size_t)n * M + m] - c);
            Wdec[(size_t)n * M + m] = w;
            l += w;
        }
        for (int m = 0; m < M; ++m) Wdec[(size_t)n * M + m] /= l;
    }
    return 0;
}

/* Thread control for timing runs (results never depend on it). */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
}
#else
int oracle_threads(int n) { (void)n; return 1; }
#endif

/* ------------------------------------------------------------------------
 * Backward (reverse mode) of the encoder and the decoder.
 *
 * Encoder, App. B.5 "Local backward" with a single shard (R = 1): given the
 * cotangents dZ and dL of the encoder outputs (Z, L), with
 *   S = s Q K^T,  P = softmax over the tokens of S,  c_m = dZ_m . Z_m
 *   (the row term of the softmax derivative, which the pages write as c),
 *   dS = P o (dZ V^T - c + dL)     (c and dL broadcast along the tokens)
 *   dV = P^T dZ,  dK = s dS^T Q,  dQ = s dS K.
 * Decoder: the same derivative for Y = SDPA(K, Q, Z), whose softmax runs over
 * the latents (App. A.1): with U = s K Q^T, W = softmax over the latents,
 * delta_n = dY_n . Y_n and no log-normaliser output,
 *   dU = W o (dY Z^T - delta)     (delta broadcast along the latents)
 *   dZ = W^T dY,  dK = s dU Q,  dQ = s dU^T K.
 * When Q is shared over the batch (q_batched == 0) its cotangent is the sum
 * of the per-batch ones.
 *
 * Each output element is a plain sum in ascending index order; the row
 * statistics (max shift, sum, row term) are formed first, so no parallel
 * reduction is involved and results do not depend on the thread count.
 * ------------------------------------------------------------------------ */

/* Encoder row statistics of one head: L_m, Z_m (via encode_row) and c_m. */
static void enc_stats(const double* Qh, const double* Kh, const double* Vh, const double* dZh, int N, int M,
                      int D, double s, double* L, double* Zh, double* c) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        L[m] = encode_row(Qh + (size_t)m * D, Kh, Vh, N, D, s, Zh + (size_t)m * D);
        c[m] = dot(dZh + (size_t)m * D, Zh + (size_t)m * D, D);
    }
}

/* dS_mn of the encoder (see above); P = exp(S - L). */
static double enc_dscore(const double* q, const double* k, const double* v, const double* dz, double Lm, double cm,
                         double dLm, int D, double s, double* p) {
    *p = exp(s * dot(q, k, D) - Lm);
    return *p * (dot(dz, v, D) - cm + dLm);
}

int oracle_encode_backward(const double* Q, int q_batched, const double* K, const double* V, const double* dZ,
                           const double* dL, int B, int H, int N, int M, int D, double scale, double* dQ,
                           double* dK, double* dV) {
    if (B <= 0 || H <= 0 || N < 0 || M <= 0 || D <= 0) return 1;
    const double s = pick_scale(scale, D);
    const size_t nq = (size_t)(q_batched ? B : 1) * H * M * D;
    memset(dQ, 0, sizeof(double) * nq);
    if (N == 0) return 0;
    double* L = (double*)malloc(sizeof(double) * (size_t)M);
    double* c = (double*)malloc(sizeof(double) * (size_t)M);
    double* Zh = (double*)malloc(sizeof(double) * (size_t)M * D);
    if (!L || !c || !Zh) { free(L); free(c); free(Zh); return 2; }
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const size_t bh = (size_t)b * H + h;
            const double* Qh = q_ptr(Q, q_batched, b, h, H, M, D);
            const double* Kh = K + bh * N * D;
            const double* Vh = V + bh * N * D;
            const double* dZh = dZ + bh * M * D;
            const double* dLh = dL ? dL + bh * M : NULL;
            enc_stats(Qh, Kh, Vh, dZh, N, M, D, s, L, Zh, c);
            /* per token: dV_n = sum_m P_mn dZ_m, dK_n = s sum_m dS_mn q_m */
#pragma omp parallel for schedule(static)
            for (int n = 0; n < N; ++n) {
                const double* k = Kh + (size_t)n * D;
                const double* v = Vh + (size_t)n * D;
                double* dk = dK + (bh * N + n) * D;
                double* dv = dV + (bh * N + n) * D;
                for (int d = 0; d < D; ++d) { dk[d] = 0.0; dv[d] = 0.0; }
                for (int m = 0; m < M; ++m) {
                    double p;
                    const double* q = Qh + (size_t)m * D;
                    const double* dz = dZh + (size_t)m * D;
                    const double ds = enc_dscore(q, k, v, dz, L[m], c[m], dLh ? dLh[m] : 0.0, D, s, &p);
                    for (int d = 0; d < D; ++d) {
                        dv[d] += p * dz[d];
                        dk[d] += s * ds * q[d];
                    }
                }
            }
            /* per latent: dQ_m += s sum_n dS_mn k_n */
            double* dQh = dQ + (q_batched ? bh : (size_t)h) * M * D;
#pragma omp parallel for schedule(dynamic, 1)
            for (int m = 0; m < M; ++m) {
                const double* q = Qh + (size_t)m * D;
                const double* dz = dZh + (size_t)m * D;
                double* dq = dQh + (size_t)m * D;
                for (int n = 0; n < N; ++n) {
                    double p;
                    const double* k = Kh + (size_t)n * D;
                    const double ds = enc_dscore(q, k, Vh + (size_t)n * D, dz, L[m], c[m], dLh ? dLh[m] : 0.0, D, s, &p);
                    for (int d = 0; d < D; ++d) dq[d] += s * ds * k[d];
                }
            }
        }
    free(L); free(c); free(Zh);
    return 0;
}

/* Decoder token statistics of one head: shift cmax_n, sum l_n and delta_n. */
static int dec_stats(const double* Qh, const double* Kh, const double* Zh, const double* dYh, int N, int M, int D,
                     double s, double* cmax, double* l, double* delta) {
    int bad = 0;
#pragma omp parallel
    {
        double* u = (double*)malloc(sizeof(double) * (size_t)M);
        double* y = (double*)malloc(sizeof(double) * (size_t)D);
        if (!u || !y) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int n = 0; n < N; ++n) {
                const double* k = Kh + (size_t)n * D;
                decode_row(k, Qh, Zh, M, D, s, y, u);
                double c = -INFINITY, sum = 0.0;
                for (int m = 0; m < M; ++m) c = u[m] > c ? u[m] : c;
                for (int m = 0; m < M; ++m) sum += exp(u[m] - c);
                cmax[n] = c;
                l[n] = sum;
                delta[n] = dot(dYh + (size_t)n * D, y, D);
            }
        }
        free(u); free(y);
    }
    return bad;
}

/* dU_nm of the decoder (see above); W = exp(U - c) / l. */
static double dec_dscore(const double* k, const double* q, const double* z, const double* dy, double c, double l,
                         double delta, int D, double s, double* w) {
    *w = exp(s * dot(k, q, D) - c) / l;
    return *w * (dot(dy, z, D) - delta);
}

int oracle_decode_backward(const double* Q, int q_batched, const double* K, const double* Z, const double* dY,
                           int B, int H, int N, int M, int D, double scale, double* dQ, double* dK, double* dZ) {
    if (B <= 0 || H <= 0 || N < 0 || M <= 0 || D <= 0) return 1;
    const double s = pick_scale(scale, D);
    const size_t nq = (size_t)(q_batched ? B : 1) * H * M * D;
    memset(dQ, 0, sizeof(double) * nq);
    memset(dZ, 0, sizeof(double) * (size_t)B * H * M * D);
    if (N == 0) return 0;
    double* cmax = (double*)malloc(sizeof(double) * (size_t)N);
    double* l = (double*)malloc(sizeof(double) * (size_t)N);
    double* delta = (double*)malloc(sizeof(double) * (size_t)N);
    if (!cmax || !l || !delta) { free(cmax); free(l); free(delta); return 2; }
    int bad = 0;
    for (int b = 0; b < B && !bad; ++b)
        for (int h = 0; h < H && !bad; ++h) {
            const size_t bh = (size_t)b * H + h;
            const double* Qh = q_ptr(Q, q_batched, b, h, H, M, D);
            const double* Kh = K + bh * N * D;
            const double* Zh = Z + bh * M * D;
            const double* dYh = dY + bh * N * D;
            if (dec_stats(Qh, Kh, Zh, dYh, N, M, D, s, cmax, l, delta)) { bad = 2; break; }
            /* per token: dK_n = s sum_m dU_nm q_m */
#pragma omp parallel for schedule(static)
            for (int n = 0; n < N; ++n) {
                const double* k = Kh + (size_t)n * D;
                const double* dy = dYh + (size_t)n * D;
                double* dk = dK + (bh * N + n) * D;
                for (int d = 0; d < D; ++d) dk[d] = 0.0;
                for (int m = 0; m < M; ++m) {
                    double w;
                    const double* q = Qh + (size_t)m * D;
                    const double du = dec_dscore(k, q, Zh + (size_t)m * D, dy, cmax[n], l[n], delta[n], D, s, &w);
                    for (int d = 0; d < D; ++d) dk[d] += s * du * q[d];
                }
            }
            /* per latent: dZ_m = sum_n W_nm dY_n, dQ_m += s sum_n dU_nm k_n */
            double* dQh = dQ + (q_batched ? bh : (size_t)h) * M * D;
#pragma omp parallel for schedule(dynamic, 1)
            for (int m = 0; m < M; ++m) {
                const double* q = Qh + (size_t)m * D;
                const double* z = Zh + (size_t)m * D;
                double* dq = dQh + (size_t)m * D;
                double* dz = dZ + (bh * M + m) * D;
                for (int n = 0; n < N; ++n) {
                    double w;
                    const double* k = Kh + (size_t)n * D;
                    const double* dy = dYh + (size_t)n * D;
                    const double du = dec_dscore(k, q, z, dy, cmax[n], l[n], delta[n], D, s, &w);
                    for (int d = 0; d < D; ++d) {
                        dz[d] += w * dy[d];
                        dq[d] += s * du * k[d];
                    }
                }
            }
        }
    free(cmax); free(l); free(delta);
    return bad;
}
