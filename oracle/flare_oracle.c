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
    if (B <= 0 || H <= 0 || N <= 0 || M <= 0 || D <= 0 || count < 0) return 1;
    if (!idx && count != N) return 1;
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
