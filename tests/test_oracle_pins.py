"""Pins of the fp64 oracle against what the FLARE++ paper and plain mathematics fix.

Each test names the passage it follows.  None of them re-types the oracle's
own formula: they check closed forms worked by hand, invariants the method
must satisfy, degenerate cases with known answers, and an independent
textbook routine (PyTorch's CPU scaled_dot_product_attention in float64).
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _num(x):
    if isinstance(x, str):
        assert x.startswith("ln")
        return math.log(float(x[2:]))
    return float(x)


def _arr(v):
    return np.array([[_num(e) for e in row] for row in v]) if isinstance(v[0], list) else np.array([_num(e) for e in v])


def _rand(seed, *shape, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# --- hand-worked closed forms (SDPA definition, Sec. 3.1; FLARE pair, App. A.1) ---

@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_hand_examples(orc, ex):
    Q, K, V = _arr(ex["Q"]), _arr(ex["K"]), _arr(ex["V"])
    Y, Z, L = orc.flare_forward(Q[None], K[None, None], V[None, None], scale=ex["scale"])
    np.testing.assert_allclose(Z[0, 0], _arr(ex["Z"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[0, 0], _arr(ex["L"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(Y[0, 0], _arr(ex["Y"]), rtol=0, atol=1e-14)


def test_hand_example_default_scale(orc):
    """Same example with s = 1/sqrt(D): keys scaled by sqrt(D) give the same scores."""
    ex = json.load(open(GOLDEN))["examples"][1]
    Q, K, V = _arr(ex["Q"]), _arr(ex["K"]), _arr(ex["V"])
    Y, Z, _ = orc.flare_forward(Q[None], (K * math.sqrt(2.0))[None, None], V[None, None])
    np.testing.assert_allclose(Z[0, 0], _arr(ex["Z"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(Y[0, 0], _arr(ex["Y"]), rtol=1e-14, atol=1e-14)


# --- P1 / P14: rank <= M of the token mixer (Sec. 1; slide "rank(W_encode W_decode) <= M") ---

def test_p1_factorisation_and_rank(orc):
    N, M, D = 64, 4, 4
    Q, K, V = _rand(1, M, D), _rand(2, N, D), _rand(3, N, D)
    Wenc, Wdec = orc.materialize(Q, K)
    A = Wdec @ Wenc                                   # N x N token mixer
    Y, _, _ = orc.flare_forward(Q[None], K[None, None], V[None, None])
    np.testing.assert_allclose(A @ V, Y[0, 0], rtol=1e-12, atol=1e-13)
    sv = np.linalg.svd(A, compute_uv=False)
    assert sv[M] < 1e-12 * sv[0]
    assert sv[M - 1] > 1e-6 * sv[0]                   # generic inputs reach rank M


def test_p14_pp_operator_rank(orc):
    N, M, D = 48, 3, 4
    Qs, Ks, Qf = _rand(1, 1, M, D), _rand(2, 1, 1, N, D), _rand(3, 1, M, D)
    K, V = _rand(4, 1, 1, N, D), _rand(5, 1, 1, N, D)
    gate = np.array([0.6])
    Y, Qb, _, _ = orc.flare_pp_forward(Qs, Ks, Ks, Qf, gate, K, V)
    Wenc, Wdec = orc.materialize(Qb[0, 0], K[0, 0])
    A = Wdec @ Wenc
    np.testing.assert_allclose(A @ V[0, 0], Y[0, 0], rtol=1e-12, atol=1e-13)
    sv = np.linalg.svd(A, compute_uv=False)
    assert sv[M] < 1e-12 * sv[0]


# --- P2: softmax axes; rows sum to one (row-wise softmax definition) ---

def test_p2_rows_sum_to_one_and_convex_hull(orc):
    N, M, D = 40, 6, 8
    Q, K, V = _rand(4, M, D), _rand(5, N, D), _rand(6, N, D)
    Wenc, Wdec = orc.materialize(Q, K)
    np.testing.assert_allclose(Wenc.sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(Wdec.sum(axis=1), 1.0, atol=1e-14)
    assert Wenc.min() >= 0 and Wdec.min() >= 0
    Y, Z, _ = orc.flare_forward(Q[None], K[None, None], V[None, None])
    lo, hi = V.min(axis=0), V.max(axis=0)
    assert np.all(Z[0, 0] >= lo - 1e-14) and np.all(Z[0, 0] <= hi + 1e-14)
    assert np.all(Y[0, 0] >= lo - 1e-14) and np.all(Y[0, 0] <= hi + 1e-14)


# --- P3: identical keys -> every latent and every token gets mean(V) ---

def test_p3_identical_keys_give_mean(orc):
    N, M, D = 33, 5, 4
    Q, V = _rand(7, M, D), _rand(8, N, D)
    K = np.tile(_rand(9, 1, D), (N, 1))
    Y, Z, L = orc.flare_forward(Q[None], K[None, None], V[None, None])
    mean = V.mean(axis=0)
    np.testing.assert_allclose(Z[0, 0], np.tile(mean, (M, 1)), atol=1e-13)
    np.testing.assert_allclose(Y[0, 0], np.tile(mean, (N, 1)), atol=1e-13)
    # L_m = s q_m.k + log N for identical keys
    np.testing.assert_allclose(L[0, 0], (Q @ K[0]) / math.sqrt(D) + math.log(N), atol=1e-13)


# --- P4 / P5: token permutation equivariance, latent permutation ---

def test_p4_token_permutation(orc):
    B, H, N, M, D = 2, 2, 37, 5, 4
    Q, K, V = _rand(10, H, M, D), _rand(11, B, H, N, D), _rand(12, B, H, N, D)
    perm = np.random.default_rng(13).permutation(N)
    Y, Z, L = orc.flare_forward(Q, K, V)
    Yp, Zp, Lp = orc.flare_forward(Q, K[:, :, perm], V[:, :, perm])
    np.testing.assert_allclose(Yp, Y[:, :, perm], atol=1e-13)
    np.testing.assert_allclose(Zp, Z, atol=1e-13)
    np.testing.assert_allclose(Lp, L, atol=1e-13)


def test_p5_latent_permutation(orc):
    B, H, N, M, D = 1, 2, 29, 6, 4
    Q, K, V = _rand(14, H, M, D), _rand(15, B, H, N, D), _rand(16, B, H, N, D)
    perm = np.random.default_rng(17).permutation(M)
    Y, Z, L = orc.flare_forward(Q, K, V)
    Yp, Zp, Lp = orc.flare_forward(Q[:, perm], K, V)
    np.testing.assert_allclose(Zp, Z[:, :, perm], atol=1e-13)
    np.testing.assert_allclose(Lp, L[:, :, perm], atol=1e-13)
    np.testing.assert_allclose(Yp, Y, atol=1e-13)


# --- P6: shift invariances of the max-subtracted softmax (App. B.3) ---

def test_p6_key_shift_leaves_latents(orc):
    N, M, D = 50, 4, 4
    Q, K, V = _rand(18, M, D), _rand(19, N, D), _rand(20, N, D)
    c = _rand(21, D) * 3
    _, Z, L = orc.flare_forward(Q[None], K[None, None], V[None, None])
    _, Z2, L2 = orc.flare_forward(Q[None], (K + c)[None, None], V[None, None])
    np.testing.assert_allclose(Z2, Z, atol=1e-12)
    np.testing.assert_allclose(L2[0, 0], L[0, 0] + Q @ c / math.sqrt(D), atol=1e-12)


def test_p6_query_shift_leaves_decoder_weights(orc):
    N, M, D = 30, 5, 4
    Q, K = _rand(22, M, D), _rand(23, N, D)
    c = _rand(24, D) * 3
    _, Wdec = orc.materialize(Q, K)
    _, Wdec2 = orc.materialize(Q + c, K)
    np.testing.assert_allclose(Wdec2, Wdec, atol=1e-13)


def test_p6_large_scores_do_not_overflow(orc):
    N, M, D = 64, 4, 4
    Q, K, V = _rand(25, M, D), _rand(26, N, D), _rand(27, N, D)
    big = 2000.0                                    # scores of order 1e3 to 1e4
    Y, Z, L = orc.flare_forward(Q[None] * big, K[None, None], V[None, None])
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(Z)) and np.all(np.isfinite(L))
    # near-hard attention: a latent whose best score leads the runner-up by > 60
    # takes its arg-max token's value to within exp(-60)
    S = (Q * big) @ K.T / math.sqrt(D)
    top2 = np.sort(S, axis=1)[:, -2:]
    hard = (top2[:, 1] - top2[:, 0]) > 60.0
    assert hard.sum() >= M // 2
    np.testing.assert_allclose(Z[0, 0][hard], V[S.argmax(axis=1)][hard], atol=1e-12)
    np.testing.assert_allclose(L[0, 0][hard], S.max(axis=1)[hard], rtol=1e-12)
    # for every latent: max_n S <= L <= max_n S + log N
    smax, tol = S.max(axis=1), 1e-12 * np.abs(S).max()
    assert np.all(L[0, 0] >= smax - tol) and np.all(L[0, 0] <= smax + math.log(N) + tol)


# --- P7: token-split partials merged with the log-sum-exp rule (Sec. 3.3, App. B.2-B.3) ---

def test_p7_split_merge_with_empty_shard(orc):
    B, H, N, M, D = 1, 2, 61, 5, 4
    Q, K, V = _rand(28, H, M, D), _rand(29, B, H, N, D), _rand(30, B, H, N, D)
    Z, L = orc.encode(Q, K, V)
    bounds = [0, 17, 17, 40, 61]                    # shard 1 is empty
    parts = [orc.encode(Q, K[:, :, a:b], V[:, :, a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
    assert np.all(parts[1][0] == 0.0) and np.all(np.isneginf(parts[1][1]))   # empty-row rule
    Ls = np.stack([p[1] for p in parts])            # [R,B,H,M]
    Zs = np.stack([p[0] for p in parts])            # [R,B,H,M,D]
    Lm = np.logaddexp.reduce(Ls, axis=0)
    Zm = np.sum(np.exp(Ls - Lm)[..., None] * Zs, axis=0)
    np.testing.assert_allclose(Lm, L, atol=1e-13)
    np.testing.assert_allclose(Zm, Z, atol=1e-13)


# --- P8: degenerate axes ---

def test_p8_no_tokens(orc):
    """N = 0: every latent is an empty row (Z = 0, L = -inf, App. B.3) and Y
    has no rows, for the forward as for the encode alone."""
    B, H, M, D = 2, 3, 5, 4
    Q = _rand(34, H, M, D)
    K = np.zeros((B, H, 0, D))
    Y, Z, L = orc.flare_forward(Q, K, K)
    assert Y.shape == (B, H, 0, D)
    assert np.all(Z == 0.0) and np.all(np.isneginf(L))
    Ze, Le = orc.encode(Q, K, K)
    assert np.all(Ze == 0.0) and np.all(np.isneginf(Le))


def test_p8_single_latent_and_single_token(orc):
    N, D = 23, 4
    Q1, K, V = _rand(31, 1, D), _rand(32, N, D), _rand(33, N, D)
    Y, Z, _ = orc.flare_forward(Q1[None], K[None, None], V[None, None])
    np.testing.assert_allclose(Y[0, 0], np.tile(Z[0, 0, 0], (N, 1)), atol=1e-15)
    Q = _rand(34, 7, D)
    Y, Z, L = orc.flare_forward(Q[None], K[None, None, :1], V[None, None, :1])
    np.testing.assert_allclose(Z[0, 0], np.tile(V[0], (7, 1)), atol=1e-15)
    np.testing.assert_allclose(Y[0, 0, 0], V[0], atol=1e-15)
    np.testing.assert_allclose(L[0, 0], Q @ K[0] / math.sqrt(D), atol=1e-15)


# --- P9: linearity in the values ---

def test_p9_linear_in_values(orc):
    N, M, D = 31, 4, 4
    Q, K, V1, V2 = _rand(35, M, D), _rand(36, N, D), _rand(37, N, D), _rand(38, N, D)
    a, b = 0.7, -1.3
    Y1, _, _ = orc.flare_forward(Q[None], K[None, None], V1[None, None])
    Y2, _, _ = orc.flare_forward(Q[None], K[None, None], V2[None, None])
    Y, _, _ = orc.flare_forward(Q[None], K[None, None], (a * V1 + b * V2)[None, None])
    np.testing.assert_allclose(Y, a * Y1 + b * Y2, atol=1e-13)


# --- P10: independent textbook routine (torch CPU SDPA in float64) ---

def _torch_sdpa(q, k, v, scale=None):
    import torch
    import torch.nn.functional as F
    return F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                          scale=scale).numpy()


@pytest.mark.parametrize("shape", [(2, 3, 50, 8, 16), (1, 2, 129, 32, 32), (1, 1, 7, 3, 16)])
def test_p10_flare_matches_torch_sdpa(orc, shape):
    B, H, N, M, D = shape
    Q, K, V = _rand(40, H, M, D, std=0.7), _rand(41, B, H, N, D), _rand(42, B, H, N, D)
    Y, Z, L = orc.flare_forward(Q, K, V)
    Qb = np.broadcast_to(Q, (B, H, M, D)).copy()
    Zt = _torch_sdpa(Qb, K, V)
    Yt = _torch_sdpa(K, Qb, Zt)
    np.testing.assert_allclose(Z, Zt, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Y, Yt, rtol=1e-12, atol=1e-13)
    # log-normaliser: identical-value trick, SDPA over a value column of exp(-max) is not
    # available, so check L through the normalisation identity sum_n exp(S_mn - L_m) = 1
    S = np.einsum("hmd,bhnd->bhmn", Q, K) / math.sqrt(D)
    np.testing.assert_allclose(np.exp(S - L[..., None]).sum(-1), 1.0, atol=1e-13)


def test_p10_pp_matches_torch_sdpa(orc):
    B, H, N, M, D = 2, 2, 70, 8, 16
    Qs, Ks, Vs = _rand(43, H, M, D), _rand(44, B, H, N, D), _rand(45, B, H, N, D)
    Qf, K, V = _rand(46, H, M, D), _rand(47, B, H, N, D), _rand(48, B, H, N, D)
    gate = np.array([0.3, 0.8])
    Y, Qb, Z, L = orc.flare_pp_forward(Qs, Ks, Vs, Qf, gate, K, V)
    Qd = _torch_sdpa(np.broadcast_to(Qs, (B, H, M, D)).copy(), Ks, Vs)
    Qt = Qf[None] + gate[None, :, None, None] * Qd
    Zt = _torch_sdpa(Qt, K, V)
    Yt = _torch_sdpa(K, Qt, Zt)
    np.testing.assert_allclose(Qb, Qt, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Z, Zt, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Y, Yt, rtol=1e-12, atol=1e-13)


def test_explicit_scale(orc):
    B, H, N, M, D = 1, 1, 20, 4, 8
    Q, K, V = _rand(49, H, M, D), _rand(50, B, H, N, D), _rand(51, B, H, N, D)
    Y, Z, _ = orc.flare_forward(Q, K, V, scale=0.37)
    Qb = np.broadcast_to(Q, (B, H, M, D)).copy()
    Zt = _torch_sdpa(Qb, K, V, scale=0.37)
    np.testing.assert_allclose(Z, Zt, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Y, _torch_sdpa(K, Qb, Zt, scale=0.37), rtol=1e-12, atol=1e-13)


# --- P12 / P13: FLARE++ wiring (App. A.4, A.8 "g -> 0 limit") ---

def test_p12_zero_gate_is_flare(orc):
    B, H, N, M, D = 2, 2, 40, 6, 8
    Qs, Ks = _rand(52, H, M, D), _rand(53, B, H, N, D)
    Qf, K, V = _rand(54, H, M, D), _rand(55, B, H, N, D), _rand(56, B, H, N, D)
    Y, Qb, Z, L = orc.flare_pp_forward(Qs, Ks, Ks, Qf, np.zeros(H), K, V)
    Y0, Z0, L0 = orc.flare_forward(Qf, K, V)
    assert np.array_equal(Qb, np.broadcast_to(Qf, Qb.shape))
    assert np.array_equal(Y, Y0) and np.array_equal(Z, Z0) and np.array_equal(L, L0)


def test_p13_normalised_values_bound_synthesised_queries(orc):
    B, H, N, M, D = 1, 2, 45, 6, 8
    Ks = _rand(57, B, H, N, D)
    Ks = Ks / np.sqrt(np.mean(Ks * Ks, axis=-1, keepdims=True))        # RMS(row) = 1
    Qs = _rand(58, H, M, D)
    Qd = orc.pp_queries(Qs, Ks, Ks, np.zeros((H, M, D)), np.ones(H))   # gate 1, Qf 0 -> Q^d
    rms = np.sqrt(np.mean(Qd * Qd, axis=-1))
    assert np.all(rms <= 1.0 + 1e-12)                                  # convex combination of unit-RMS rows
    perm = np.random.default_rng(59).permutation(N)
    Qd2 = orc.pp_queries(Qs, Ks[:, :, perm], Ks[:, :, perm], np.zeros((H, M, D)), np.ones(H))
    np.testing.assert_allclose(Qd2, Qd, atol=1e-13)


def test_pp_blend_against_hand_values(orc):
    """Synthesis encode equal to the d1 hand example, blended with gate 0.5 onto Qf = 1."""
    Qs = np.array([[0.0], [1.0]])[None]
    Ks = np.array([[0.0], [math.log(3)]])[None, None]
    Vs = np.array([[1.0], [5.0]])[None, None]
    Qf = np.ones((1, 2, 1))
    Qb = orc.pp_queries(Qs, Ks, Vs, Qf, np.array([0.5]), scale=1.0)
    np.testing.assert_allclose(Qb[0, 0, :, 0], [1 + 0.5 * 3.0, 1 + 0.5 * 4.0], atol=1e-15)


# --- sampled decode rows agree with the full decode ---

def test_decode_rows_subset(orc):
    B, H, N, M, D = 2, 3, 57, 9, 16
    Q, K, V = _rand(60, B, H, M, D), _rand(61, B, H, N, D), _rand(62, B, H, N, D)
    Y, Z, _ = orc.flare_forward(Q, K, V)
    idx = np.array([0, 5, 56, 13, 13])
    Ys = orc.decode(Q, K, Z, idx=idx)
    np.testing.assert_array_equal(Ys, Y[:, :, idx])


def test_thread_count_does_not_change_results(orc):
    B, H, N, M, D = 1, 2, 300, 16, 16
    Q, K, V = _rand(63, H, M, D), _rand(64, B, H, N, D), _rand(65, B, H, N, D)
    n0 = orc.threads()
    try:
        orc.threads(1)
        a = orc.flare_forward(Q, K, V)
        orc.threads(max(2, n0))
        b = orc.flare_forward(Q, K, V)
    finally:
        orc.threads(n0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
