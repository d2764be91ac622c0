/*
 * flare.h -- C ABI of the MI355X (gfx950) FLARE / FLARE++ routing forward.
 *
 * The operations are those of the FLARE++ paper ("FLARE++: Low-rank attention
 * with attention-synthesized routing", Puri et al.):
 *
 *   SDPA(Q, K, V) = softmax(s Q K^T) V, softmax taken row-wise, s = 1/sqrt(D)
 *                                                     (Sec. 3.1, "Full self-attention")
 *   FLARE encode  Z_h = SDPA(Q_h, K_h, V_h): M latent queries attend over the
 *                 N tokens, softmax over N                (App. A.1; Table 2 in A.7)
 *   FLARE decode  Y_h = SDPA(K_h, Q_h, Z_h): every token attends over the M
 *                 latents, softmax over M                 (App. A.1; Table 2 in A.7)
 *   Log-normaliser of the encode  L_m = log sum_n exp(s q_m . k_n), natural log
 *                                                     (App. B.2, B.3)
 *   FLARE++ query synthesis  Q_b,h = Qf_h + g_h SDPA(Qs_h, Ks_b,h, Vs_b,h)
 *                                                     (Sec. 3.2; App. A.1, A.4, A.6)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers of the current HIP device,
 *   contiguous, row-major, D innermost, 16-byte aligned.
 *     K, V, Ks, Vs, Y : [B, H, N, D] in `dtype`
 *     Q               : [H, M, D] (q_batched == 0, shared by the batch, the
 *                       learned queries of Sec. 3.1) or [B, H, M, D]
 *                       (q_batched == 1), in `dtype`
 *     Z               : [B, H, M, D] float32;  L : [B, H, M] float32
 *     Q_out           : [B, H, M, D] float32
 *     gate            : [H] float32, already g_h = sigmoid(gamma_h) (App. A.4)
 * - dtype: FLARE_F32 or FLARE_BF16.  Softmax statistics and every
 *   accumulation are float32.  FLARE_F32 forms the scores with float32
 *   matrix-core products.  FLARE_BF16 feeds bf16 matrix-core products: keys
 *   and values as given; the queries scaled by s*log2(e) and rounded to bf16
 *   wherever that rounding provably moves no score by more than 2^-5 (log2
 *   units; checked per unit of work from the queries' rounding error and the
 *   largest key norm), and otherwise split into a bf16 hi + lo pair so the
 *   scores are exact to float32 accumulation; the softmax weights as bf16
 *   (their sums are taken over the same bf16 weights).
 * - scale <= 0 selects s = 1/sqrt(D); any positive value overrides it.  The
 *   same s is used by the encode and by the decode (whose query, a token
 *   key, also has width D).
 * - Supported sizes: B >= 1, H >= 1, N >= 0, 1 <= M <= 256, D in {16, 32},
 *   B*H*N < 2^31.  N == 0 is the empty-row case of App. B.3: Z = 0 and
 *   L = -inf, and nothing is written to Y.
 * - ws / ws_bytes: caller-owned DEVICE scratch of at least
 *   flare_workspace_size(op, ...) bytes, 256-byte aligned.  It may be NULL
 *   when that size is 0.  Its contents on entry do not matter.
 * - stream: a hipStream_t (NULL = the default stream).  Calls only enqueue
 *   work; they never synchronise the host, allocate memory or keep state
 *   between calls, so they are reentrant.  Results are bitwise reproducible
 *   for a fixed (shape, dtype, device).
 * - Ownership: the caller owns every buffer; the library never frees or
 *   retains a pointer after the call returns.
 * - Errors: every argument is validated before anything is enqueued; a
 *   failed check returns a nonzero status and leaves all outputs untouched.
 *   A launch failure returns FLARE_ERR_HIP.  NaN or Inf inputs give
 *   undefined (but finite-time) results.
 */
#ifndef FLARE_H
#define FLARE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define FLARE_F32 0
#define FLARE_BF16 1

/* status codes */
#define FLARE_OK 0
#define FLARE_ERR_INVALID_ARG 1 /* null pointer, negative size, misalignment, bad flag */
#define FLARE_ERR_UNSUPPORTED 2 /* D not in {16,32}, M > 256, unknown dtype, size overflow */
#define FLARE_ERR_WORKSPACE 3   /* ws smaller than flare_workspace_size() */
#define FLARE_ERR_HIP 4         /* the HIP runtime rejected a query or a launch */

/* operation codes for flare_workspace_size */
#define FLARE_OP_ENCODE 0
#define FLARE_OP_DECODE 1
#define FLARE_OP_FORWARD 2
#define FLARE_OP_PP_FORWARD 3
#define FLARE_OP_BACKWARD 4
#define FLARE_OP_ENCODE_BACKWARD 5
#define FLARE_OP_PP_BACKWARD 6
#define FLARE_OP_PP_BACKWARD_NORM 7
#define FLARE_OP_FORWARD_PROJ 8
#define FLARE_OP_PP_FORWARD_PROJ 9

/* Scratch bytes that `op` needs for this problem (0 when none); returns 0 for
 * arguments the op would reject.  Depends only on its arguments and on the
 * compute-unit count of the current device. */
size_t flare_workspace_size(int op, int B, int H, int N, int M, int D, int dtype);

/* FLARE encode (App. A.1 with the log-normaliser of App. B.2):
 *   Z[b,h,m,:] = sum_n softmax_n(s q_m . k_n) v_n ,  L[b,h,m] = log sum_n exp(s q_m . k_n).
 * The token axis is split over workgroups; each split keeps a running
 * (max, sum, accumulator) triple and the splits are combined with the
 * log-sum-exp merge of Sec. 3.3 / App. B.3 in a fixed order.
 * Q: [H,M,D] or [B,H,M,D] (q_batched); K, V: [B,H,N,D]; Z: [B,H,M,D] f32 (required);
 * L: [B,H,M] f32 or NULL. */
int flare_encode(const void* Q, int q_batched, const void* K, const void* V, float* Z, float* L, int B,
                 int H, int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes,
                 void* stream);

/* FLARE decode (App. A.1): Y[b,h,n,:] = sum_m softmax_m(s k_n . q_m) Z[b,h,m,:].
 * Q: [H,M,D] or [B,H,M,D] (q_batched) in dtype; K: [B,H,N,D]; Z: [B,H,M,D] f32;
 * Y: [B,H,N,D] in dtype.  Needs no workspace (ws may be NULL). */
int flare_decode(const void* Q, int q_batched, const void* K, const float* Z, void* Y, int B, int H, int N,
                 int M, int D, int dtype, float scale, void* ws, size_t ws_bytes, void* stream);

/* FLARE routing forward, encode then decode on one stream (App. A.1, Table 2):
 * Y = SDPA(K, Q, SDPA(Q, K, V)).  The N x M scores are never stored; the
 * decode recomputes them.  Z_out / L_out (may be NULL) receive the latents
 * and log-normalisers. */
int flare_forward(const void* Q, int q_batched, const void* K, const void* V, void* Y, float* Z_out,
                  float* L_out, int B, int H, int N, int M, int D, int dtype, float scale, void* ws,
                  size_t ws_bytes, void* stream);

/* flare_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments as flare_forward minus ws / ws_bytes.
 * The scratch it needs (the encode's split partials, and Z / L when Z_out /
 * L_out are NULL) lives in a file-scope device array of
 * FLARE_NOALLOC_SCRATCH_BYTES, one per GPU, held from the library's load
 * until the process ends; this call allocates nothing.  A problem whose
 * scratch, flare_workspace_size(FLARE_OP_FORWARD, ...), exceeds that size
 * returns FLARE_ERR_WORKSPACE before anything is enqueued (the million-token
 * shape B1 H8 N2^20 M256 D32 needs about 18 MB).  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  Nothing in the array
 * needs clearing between calls. */
#define FLARE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int flare_forward_noalloc(const void* Q, int q_batched, const void* K, const void* V, void* Y, float* Z_out,
                          float* L_out, int B, int H, int N, int M, int D, int dtype, float scale, void* stream);

/* FLARE++ routing forward (Sec. 3.2; App. A.1, A.4, A.6):
 *   Qd[b,h] = SDPA(Qs[h], Ks[b,h], Vs[b,h])            (synthesis encode)
 *   Q[b,h]  = Qf[h] + gate[h] * Qd[b,h]                 (float32 blend)
 *   Y       = SDPA(K, Q, SDPA(Q, K, V))                 (routing with the per-batch Q)
 * Qs, Qf: [H,M,D] in dtype (already normalised by the caller); Ks, Vs:
 * [B,H,N,D] in dtype, Vs may equal Ks (shared synthesis keys and values,
 * App. A.6: each tile is then read once); gate: [H] f32; K, V: [B,H,N,D];
 * Y: [B,H,N,D] in dtype.  Q_out [B,H,M,D] f32, Z_out, L_out may be NULL. */
int flare_pp_forward(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                     const void* K, const void* V, void* Y, float* Q_out, float* Z_out, float* L_out, int B,
                     int H, int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes,
                     void* stream);

/* Per-head input normalisations of FLARE++ (App. A.3, A.4, A.6 and Table 2 in
 * App. A.7), fused into flare_pp_forward_norm.  Each is an RMS norm over the
 * head dimension D of every row: N(x) = x / sqrt(mean_d x_d^2 + eps), then,
 * for N_a, times a per-channel scale alpha[h, :] (N_0 when alpha is NULL). */
#define FLARE_NORM_QS 1  /* synthesis seeds Qs, scale alpha_qs (FLARE++ and simplified: N_a) */
#define FLARE_NORM_KS 2  /* synthesis keys Ks, scale alpha_ks (FLARE++: N_0; simplified: N_a); when
                            Vs == Ks the values are the normalised keys (App. A.6) */
#define FLARE_NORM_QF 4  /* fixed queries Qf, N_0 (FLARE++, App. A.4) */
#define FLARE_NORM_K 8   /* routing keys K, scale alpha_k (FLARE++: N_a); V is never normalised */
#define FLARE_NORM_ALL 15

/* FLARE++ routing forward with its input normalisations applied inside the
 * kernels, as they load each tensor (no normalised copy is written):
 *   FLARE++            norm_flags = QS | KS | QF | K, alpha_qs, alpha_k given,
 *                      alpha_ks NULL, Vs == Ks;
 *   simplified FLARE++ norm_flags = QS | KS, alpha_qs, alpha_ks given, separate
 *                      Vs, Qf all zeros and gate all ones (Q = Qd, no blend).
 * Arguments as flare_pp_forward, plus:
 *   norm_flags  OR of FLARE_NORM_*; 0 makes this call flare_pp_forward;
 *   alpha_qs, alpha_ks, alpha_k  [H, D] float32 device arrays (16-byte aligned)
 *               or NULL; each is read only when its flag is set;
 *   eps         > 0 when any flag is set (the pages do not fix it; 1e-6 is
 *               the value this library's tests use).
 * Normalisation needs dtype FLARE_BF16 (else FLARE_ERR_UNSUPPORTED); a bad
 * flag or eps gives FLARE_ERR_INVALID_ARG.  Keys normalised on the fly are
 * rounded to fp16 for the score products (their elements are at most sqrt(D)
 * in magnitude), with the queries they meet rounded to fp16 as well; keys
 * that are also the values (Vs == Ks) are rounded to bf16 instead, as the
 * value products take them. */
int flare_pp_forward_norm(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                          const void* K, const void* V, void* Y, float* Q_out, float* Z_out, float* L_out,
                          int B, int H, int N, int M, int D, int dtype, float scale, int norm_flags,
                          const float* alpha_qs, const float* alpha_ks, const float* alpha_k, float eps,
                          void* ws, size_t ws_bytes, void* stream);

/* FLARE routing forward from the block input (FLARE++ paper, Sec. 3.1 "FLARE:
 * fixed-query latent routing": K_h = X W_K,h, V_h = X W_V,h; then App. A.1):
 *   K[b,h] = X[b] WK[h],  V[b,h] = X[b] WV[h],  Y = SDPA(K, Q, SDPA(Q, K, V)).
 * The projections run on the matrix cores inside the encode, per tile of
 * tokens, from X tiles in LDS: V is never stored; K is written once (to K_out,
 * or to the workspace) and read by the decode.  The projected keys and values
 * are rounded to bf16 before the attention products, as stored inputs are.
 * X: [B, N, C] bf16 (shared by the heads); WK, WV: [H, C, D] bf16; Q, Y, Z_out,
 * L_out as flare_forward; K_out: [B, H, N, D] bf16 or NULL.
 * Supported: dtype FLARE_BF16, D = 32, C = 128 (else FLARE_ERR_UNSUPPORTED).
 * ws of flare_workspace_size(FLARE_OP_FORWARD_PROJ, ...) bytes (it includes
 * room for the projected keys). */
int flare_forward_proj(const void* X, const void* WK, const void* WV, const void* Q, int q_batched, void* Y,
                       void* K_out, float* Z_out, float* L_out, int B, int H, int N, int M, int D, int C, int dtype,
                       float scale, void* ws, size_t ws_bytes, void* stream);

/* FLARE++ routing forward from the block input (Sec. 3.1, 3.2; App. A.1, A.4,
 * A.6; Table 2 for the norms): synthesis keys X WKs[h] (also the synthesis
 * values), routing keys X WK[h] and values X WV[h], formed inside the two
 * encodes as in flare_forward_proj, then the per-head norms of norm_flags
 * (FLARE_NORM_QS with alpha_qs, FLARE_NORM_KS as N_0, FLARE_NORM_QF,
 * FLARE_NORM_K with alpha_k) and the FLARE++ forward as flare_pp_forward_norm.
 * K_out (NULL or [B, H, N, D] bf16) receives the routing keys, normalised when
 * FLARE_NORM_K is set.  Same support and workspace rules as flare_forward_proj
 * (op FLARE_OP_PP_FORWARD_PROJ). */
int flare_pp_forward_proj(const void* X, const void* WKs, const void* WK, const void* WV, const void* Qs,
                          const void* Qf, const float* gate, void* Y, float* Q_out, void* K_out, float* Z_out,
                          float* L_out, int B, int H, int N, int M, int D, int C, int dtype, float scale,
                          int norm_flags, const float* alpha_qs, const float* alpha_k, float eps, void* ws,
                          size_t ws_bytes, void* stream);

/* Backward of the FLARE pair Y = SDPA(K, Q, SDPA(Q, K, V)) (reverse mode;
 * FLARE++ paper, App. B.5 "Local backward" for the encoder with one shard,
 * and the derivative of the decoder's softmax over the latents, App. A.1).
 * Given the output cotangent dY, with S = s Q K^T:
 *   decoder  W = softmax over latents,  delta_n = dY_n . Y_n,
 *            dS_dec = W o (Z dY^T - delta),  dZ = W dY
 *   encoder  P = softmax over tokens,  c_m = dZ_m . Z_m,
 *            dS_enc = P o (dZ V^T - c),  dV = P^T dZ
 *   dK = s (dS_dec + dS_enc)^T Q,  dQ = s (dS_dec + dS_enc) K.
 * Inputs: Q, K, V as for flare_forward, dtype FLARE_BF16 or FLARE_F32;
 * Z [B,H,M,D] f32 and L [B,H,M] f32 are the latents and log-normalisers
 * flare_forward returned for the same Q, K, V (the scores are recomputed,
 * never stored); dY [B,H,N,D] in the input dtype.
 * Outputs: dQ f32 in Q's layout ([H,M,D] shared queries receive the sum
 * over the batch); dK, dV [B,H,N,D] in the input dtype; dZ_out [B,H,M,D]
 * f32 or NULL.  bf16 inputs use bf16 matrix-core operands with float32
 * accumulation; float32 inputs are computed in float32 throughout (every
 * exponential with its exact shift).
 * All device pointers 16-byte aligned; ws of
 * flare_workspace_size(FLARE_OP_BACKWARD, ...) bytes is required.  The result
 * is deterministic (fixed split plan, fixed summation order). */
int flare_backward(const void* Q, int q_batched, const void* K, const void* V, const float* Z, const float* L,
                   const void* dY, float* dQ, void* dK, void* dV, float* dZ_out, int B, int H, int N, int M,
                   int D, int dtype, float scale, void* ws, size_t ws_bytes, void* stream);

/* Backward of the encoder alone (App. B.5 with one shard): given the
 * cotangents dZ [B,H,M,D] f32 and dL [B,H,M] f32 (NULL = 0) of its outputs
 * (Z, L) = flare_encode(Q, K, V),
 *   P = softmax over tokens,  c_m = dZ_m . Z_m,
 *   dS = P o (dZ V^T - c + dL),  dV = P^T dZ,  dK = s dS^T Q,  dQ = s dS K.
 * Z and L are the encoder's own outputs for the same inputs.  Layouts,
 * dtype and alignment as flare_backward; ws of
 * flare_workspace_size(FLARE_OP_ENCODE_BACKWARD, ...) bytes. */
int flare_encode_backward(const void* Q, int q_batched, const void* K, const void* V, const float* Z,
                          const float* L, const float* dZ, const float* dL, float* dQ, void* dK, void* dV,
                          int B, int H, int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes,
                          void* stream);

/* Backward of the FLARE++ forward (App. B.5, last paragraph; App. A.4 for
 * the blend): the routing pair's backward gives dK, dV and the cotangent dQ
 * of the per-batch routing queries; the blend Q = Qf + g Qd gives
 *   dQf[h] = sum_b dQ[b,h],  dgate[h] = sum_{b,m,d} dQ Qd,  dQd = g dQ;
 * and dQd is handed once to the synthesis encoder's backward (as
 * flare_encode_backward with dL = 0), which gives dQs (summed over the
 * batch), dKs and dVs.  The synthesis latents Qd are recomputed.
 * Inputs: those of flare_pp_forward (dtype FLARE_BF16 or FLARE_F32, inputs
 * already normalised) plus what it returned for them: Q [B,H,M,D] f32 (its
 * Q_out), Z [B,H,M,D] f32 and L [B,H,M] f32; dY [B,H,N,D] in the input dtype.
 * Outputs: dQs, dQf [H,M,D] f32; dgate [H] f32; dKs, dVs, dK, dV [B,H,N,D]
 * in the input dtype; dQ_out [B,H,M,D] f32 or NULL.  When Vs == Ks (shared synthesis keys
 * and values, App. A.6) dKs receives the sum of the key and value
 * cotangents and dVs is not written (it may be NULL).
 * ws of flare_workspace_size(FLARE_OP_PP_BACKWARD, ...) bytes. */
int flare_pp_backward(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                      const void* K, const void* V, const float* Q, const float* Z, const float* L, const void* dY,
                      float* dQs, void* dKs, void* dVs, float* dQf, float* dgate, float* dQ_out, void* dK, void* dV,
                      int B, int H, int N, int M, int D, int dtype, float scale, void* ws, size_t ws_bytes,
                      void* stream);

/* Backward of flare_pp_forward_norm: the FLARE++ backward through the
 * per-head RMS norms of norm_flags (App. A.3, A.4 and Table 2 in A.7 for the
 * norms; App. B.5 for the rest).  The normalised inputs are formed again
 * (bf16, like the inputs), the FLARE++ backward runs on them as
 * flare_pp_backward does, and then each norm's reverse mode: with
 * r = (mean_d x^2 + eps)^(-1/2) per row, xh = r x and dy the cotangent of
 * N(x) = xh * alpha,
 *   dx = r (dy * alpha - xh mean_d(dy * alpha * xh)),
 *   dalpha[h, :] = sum over the rows of head h of dy * xh.
 * Arguments as flare_pp_backward (cotangents of the raw inputs in the same
 * places; with Vs == Ks the values' cotangent is added to dKs before the
 * norm's backward), plus those of flare_pp_forward_norm (norm_flags, alpha_*,
 * eps) and:
 *   dalpha_qs, dalpha_ks, dalpha_k  [H, D] float32 outputs, required exactly
 *               when the matching alpha is given and its flag is set (else
 *               not written; may be NULL).
 * Q, Z, L are the routing queries, latents and log-normalisers that
 * flare_pp_forward_norm returned for the same inputs.  norm_flags = 0 makes
 * this call flare_pp_backward.  ws of
 * flare_workspace_size(FLARE_OP_PP_BACKWARD_NORM, ...) bytes (it holds the
 * normalised seeds and keys).  Deterministic, like the other entry points. */
int flare_pp_backward_norm(const void* Qs, const void* Ks, const void* Vs, const void* Qf, const float* gate,
                           const void* K, const void* V, const float* Q, const float* Z, const float* L,
                           const void* dY, float* dQs, void* dKs, void* dVs, float* dQf, float* dgate, float* dQ_out,
                           void* dK, void* dV, float* dalpha_qs, float* dalpha_ks, float* dalpha_k, int B, int H,
                           int N, int M, int D, int dtype, float scale, int norm_flags, const float* alpha_qs,
                           const float* alpha_ks, const float* alpha_k, float eps, void* ws, size_t ws_bytes,
                           void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* flare_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FLARE_H */
