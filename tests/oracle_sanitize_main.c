/*
 * Memory and undefined-behaviour check of the fp64 oracle: every entry point
 * of oracle/flare_oracle.c runs on small inputs in exactly sized heap buffers
 * (so that AddressSanitizer sees any access past them), including the edge
 * cases the oracle handles specially: no tokens, one token, one latent, one
 * feature, out-of-range token indices in the decode list, and a query shared
 * over the batch or given per batch.  Built with gcc -fsanitize=address,
 * undefined by test_sanitize.py; prints "ok" or the first failed property.
 *
 * The properties checked besides memory safety are ones the definition fixes
 * (softmax rows sum to one, an empty token axis gives Z = 0 and L = -inf, the
 * factored forward equals the materialised operator applied to V); the
 * oracle's numerical pins live in the Python tests.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../oracle/flare_oracle.c"

static unsigned long long rng_state = 0x9E3779B97F4A7C15ull;

static double urand(void) { /* splitmix64 -> [-1, 1) */
    unsigned long long z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static double* buf(size_t n) {
    double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
    if (!p) { printf("out of memory\n"); exit(1); }
    for (size_t i = 0; i < n; ++i) p[i] = urand();
    return p;
}

static int fail(const char* what, int B, int H, int N, int M, int D) {
    printf("%s failed at B=%d H=%d N=%d M=%d D=%d\n", what, B, H, N, M, D);
    return 1;
}

static int all_finite(const double* x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

/* every entry point on one shape */
static int run_shape(int B, int H, int N, int M, int D, int qb) {
    const size_t nq = (size_t)(qb ? B : 1) * H * M * D, nkv = (size_t)B * H * N * D;
    const size_t nz = (size_t)B * H * M * D, nl = (size_t)B * H * M;
    double *Q = buf(nq), *K = buf(nkv), *V = buf(nkv), *Z = buf(nz), *L = buf(nl), *Y = buf(nkv);
    int bad = 0;
    if (oracle_flare_forward(Q, qb, K, V, B, H, N, M, D, 0.0, Y, Z, L) != 0) bad = 1;
    if (!bad && N == 0) { /* no token rows: empty latents */
        for (size_t i = 0; i < nz; ++i) bad |= Z[i] != 0.0;
        for (size_t i = 0; i < nl; ++i) bad |= !(isinf(L[i]) && L[i] < 0);
    }
    if (oracle_encode(Q, qb, K, V, B, H, N, M, D, 0.0, Z, L) != 0) bad = 1;
    if (!bad && N == 0) {
        for (size_t i = 0; i < nz; ++i) bad |= Z[i] != 0.0;
        for (size_t i = 0; i < nl; ++i) bad |= !(isinf(L[i]) && L[i] < 0);
    }
    if (!bad && N > 0) bad = !all_finite(Z, nz) || !all_finite(L, nl) || !all_finite(Y, nkv);
    if (bad) return fail("forward", B, H, N, M, D);

    if (N > 0) {
        /* a token list with indices outside [0, N): those rows are skipped */
        const long count = 5;
        long idx[5] = {0, N - 1, -1, N, N / 2};
        double* Yr = buf((size_t)B * H * count * D);
        if (oracle_decode_rows(Q, qb, K, Z, B, H, N, M, D, 0.0, idx, count, Yr) != 0) bad = 1;
        free(Yr);
        if (bad) return fail("decode_rows", B, H, N, M, D);
    }

    /* backward of both halves (the cotangents are random) */
    double *dZ = buf(nz), *dL = buf(nl), *dY = buf(nkv);
    double *dQ = buf(nq), *dK = buf(nkv), *dV = buf(nkv), *dK2 = buf(nkv), *dZ2 = buf(nz), *dQ2 = buf(nq);
    if (oracle_encode_backward(Q, qb, K, V, dZ, dL, B, H, N, M, D, 0.0, dQ, dK, dV) != 0) bad = 1;
    if (oracle_decode_backward(Q, qb, K, Z, dY, B, H, N, M, D, 0.0, dQ2, dK2, dZ2) != 0) bad = 1;
    if (!bad) bad = !all_finite(dQ, nq) || !all_finite(dQ2, nq) || !all_finite(dZ2, nz);
    if (!bad && N > 0) bad = !all_finite(dK, nkv) || !all_finite(dV, nkv) || !all_finite(dK2, nkv);
    free(dZ); free(dL); free(dY); free(dQ); free(dK); free(dV); free(dK2); free(dZ2); free(dQ2);
    if (bad) return fail("backward", B, H, N, M, D);

    /* FLARE++: synthesis queries from their own keys and values */
    if (N > 0) {
        const size_t nsq = (size_t)H * M * D;
        double *Qs = buf(nsq), *Qf = buf(nsq), *gate = buf((size_t)H), *Qo = buf(nz);
        if (oracle_flare_pp_forward(Qs, K, V, Qf, gate, K, V, B, H, N, M, D, 0.0, Y, Qo, Z, L) != 0) bad = 1;
        if (!bad) bad = !all_finite(Qo, nz) || !all_finite(Y, nkv);
        free(Qs); free(Qf); free(gate); free(Qo);
        if (bad) return fail("pp_forward", B, H, N, M, D);
    }
    free(Q); free(K); free(V); free(Z); free(L); free(Y);
    return 0;
}

/* one head: rows of the materialised weights sum to one, and the factored
 * forward equals Wdec (Wenc V) */
static int run_materialized(int N, int M, int D) {
    double *Q = buf((size_t)M * D), *K = buf((size_t)N * D), *V = buf((size_t)N * D);
    double *We = buf((size_t)M * N), *Wd = buf((size_t)N * M);
    double *Y = buf((size_t)N * D), *Z = buf((size_t)M * D), *L = buf((size_t)M);
    int bad = oracle_materialize(Q, K, N, M, D, 0.0, We, Wd) != 0;
    bad |= oracle_flare_forward(Q, 0, K, V, 1, 1, N, M, D, 0.0, Y, Z, L) != 0;
    for (int m = 0; m < M && !bad; ++m) {
        double s = 0.0;
        for (int n = 0; n < N; ++n) s += We[(size_t)m * N + n];
        bad |= fabs(s - 1.0) > 1e-12;
    }
    for (int n = 0; n < N && !bad; ++n) {
        double s = 0.0;
        for (int m = 0; m < M; ++m) s += Wd[(size_t)n * M + m];
        bad |= fabs(s - 1.0) > 1e-12;
        for (int d = 0; d < D; ++d) {
            double y = 0.0;
            for (int m = 0; m < M; ++m) {
                double z = 0.0;
                for (int k = 0; k < N; ++k) z += We[(size_t)m * N + k] * V[(size_t)k * D + d];
                y += Wd[(size_t)n * M + m] * z;
            }
            bad |= fabs(y - Y[(size_t)n * D + d]) > 1e-12;
        }
    }
    free(Q); free(K); free(V); free(We); free(Wd); free(Y); free(Z); free(L);
    return bad ? fail("materialize", 1, 1, N, M, D) : 0;
}

int main(void) {
    static const int shapes[][5] = {
        /* B, H, N, M, D */
        {1, 1, 1, 1, 1},  {1, 1, 0, 3, 4},  {2, 3, 17, 5, 16}, {1, 2, 33, 32, 32},
        {2, 1, 64, 1, 8}, {1, 1, 7, 40, 16}, {3, 2, 0, 2, 2},  {1, 1, 129, 64, 32},
    };
    oracle_threads(1);
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        for (int qb = 0; qb < 2; ++qb)
            if (run_shape(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4], qb)) return 1;
    if (run_materialized(1, 1, 1) || run_materialized(9, 4, 3) || run_materialized(23, 7, 16)) return 1;
    printf("ok\n");
    return 0;
}
