"""Pins of the oracle's per-head RMS normalisation and of the normalised
FLARE++ forward (FLARE++ paper, App. A.3, A.4, A.6 and Table 2 in A.7).

Hand-worked rows, invariants the definition implies, PyTorch's float64
rms_norm and scaled_dot_product_attention as independent library routines,
and the value-normalisation bound of App. A.4.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rms_norm_examples.json")


def _rand(seed, *shape, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_rms_norm_hand_rows(orc, ex):
    x = np.array(ex["x"])[None, None, :]  # one head, one row
    alpha = None if ex["alpha"] is None else np.array(ex["alpha"])[None, :]
    y = orc.rms_norm(x, alpha, eps=0.0)
    np.testing.assert_allclose(y[0, 0], ex["y"], rtol=1e-15, atol=1e-15)


def test_rms_norm_unit_rms_scale_invariance_and_sign(orc):
    # App. A.4: an N_0 row has RMS 1; the definition is invariant to a positive
    # rescaling of the row and odd in its sign
    x = _rand(1, 2, 3, 17, 32)
    y = orc.rms_norm(x, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    t = np.exp(_rand(2, 2, 3, 17, 1))  # one positive factor per row
    np.testing.assert_allclose(orc.rms_norm(x * t, eps=0.0), y, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(orc.rms_norm(-x, eps=0.0), -y, rtol=0, atol=0)


def test_rms_norm_scale_is_per_head_per_channel(orc):
    # Table 2: N_a carries D parameters per head, one per channel of the head dimension
    x = _rand(3, 2, 4, 9, 16)
    alpha = 1.0 + _rand(4, 4, 16, std=0.3)
    y0 = orc.rms_norm(x, eps=1e-6)
    ya = orc.rms_norm(x, alpha, eps=1e-6)
    for h in range(4):
        np.testing.assert_allclose(ya[:, h], y0[:, h] * alpha[h][None, None, :], rtol=1e-15)


def test_rms_norm_matches_torch(orc):
    torch = pytest.importorskip("torch")
    x = _rand(5, 3, 4, 33, 32)
    alpha = 1.0 + _rand(6, 4, 32, std=0.2)
    ref = np.stack([torch.nn.functional.rms_norm(torch.from_numpy(x[:, h]), (32,), weight=torch.from_numpy(alpha[h]),
                                                 eps=1e-6).numpy() for h in range(4)], axis=1)
    np.testing.assert_allclose(orc.rms_norm(x, alpha, eps=1e-6), ref, rtol=1e-13, atol=1e-15)


def _shapes(B=2, H=3, N=50, M=8, D=16, seed=10):
    Qs = _rand(seed, H, M, D, std=0.7)
    Ks = _rand(seed + 1, B, H, N, D, std=1.7)
    Qf = _rand(seed + 2, H, M, D, std=0.4)
    K = _rand(seed + 3, B, H, N, D, std=2.1)
    V = _rand(seed + 4, B, H, N, D)
    gate = np.array([0.3, 0.56, 0.9])[:H]
    return Qs, Ks, Qf, K, V, gate


def test_normed_pp_without_flags_is_pp(orc):
    Qs, Ks, Qf, K, V, gate = _shapes()
    a = orc.flare_pp_forward(Qs, Ks, Ks, Qf, gate, K, V)
    b = orc.flare_pp_forward_normed(Qs, Ks, Ks, Qf, gate, K, V)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def _sdpa(torch, q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(q, k, v)


def test_shared_value_synthesis_matches_sdpa_form(orc):
    # App. A.6: Q^d = softmax(N_a(Q~) N_0(K~)^T / sqrt D) N_0(K~); with Q^f = 0
    # and g = 1 the routing query returned is Q^d itself (App. A.4)
    torch = pytest.importorskip("torch")
    Qs, Ks, _, K, V, _ = _shapes(seed=20)
    H, M, D = Qs.shape
    alpha_qs = 1.0 + _rand(21, H, D, std=0.3)
    zeros, ones = np.zeros((H, M, D)), np.ones(H)
    _, Q, _, _ = orc.flare_pp_forward_normed(Qs, Ks, Ks, zeros, ones, K, V, norm_qs=True, norm_ks=True,
                                             norm_qf=True, alpha_qs=alpha_qs)
    tq = torch.from_numpy(Qs)
    nq = torch.stack([torch.nn.functional.rms_norm(tq[h], (D,), weight=torch.from_numpy(alpha_qs[h]), eps=1e-6)
                      for h in range(H)])
    nk = torch.nn.functional.rms_norm(torch.from_numpy(Ks), (D,), eps=1e-6)
    ref = _sdpa(torch, nq.unsqueeze(0).expand(Ks.shape[0], -1, -1, -1), nk, nk).numpy()
    np.testing.assert_allclose(Q, ref, rtol=1e-12, atol=1e-14)


def test_value_normalisation_bounds_synthesised_queries(orc):
    # App. A.4: Q^d is a convex combination of value rows of RMS 1, so its RMS is at most 1
    Qs, Ks, _, K, V, _ = _shapes(seed=30)
    H, M, D = Qs.shape
    Ks40 = Ks * 40.0  # one array: V~ is then the normalised K~ (App. A.6)
    _, Q, _, _ = orc.flare_pp_forward_normed(Qs * 25.0, Ks40, Ks40, np.zeros((H, M, D)), np.ones(H), K, V,
                                             norm_ks=True, eps=0.0)
    assert float(np.sqrt(np.mean(Q * Q, axis=-1)).max()) <= 1.0 + 1e-12


def test_simplified_variant_leaves_values_unnormalised(orc):
    # Table 2, simplified FLARE++: N_a on Q~ and K~, a separate V~ without norm,
    # Q = Q^d; routing keys unnormalised
    torch = pytest.importorskip("torch")
    Qs, Ks, _, K, V, _ = _shapes(seed=40)
    Vs = _rand(45, *Ks.shape, std=3.0)
    H, M, D = Qs.shape
    aq, ak = 1.0 + _rand(41, H, D, std=0.2), 1.0 + _rand(42, H, D, std=0.2)
    Y, Q, Z, L = orc.flare_pp_forward_normed(Qs, Ks, Vs, np.zeros((H, M, D)), np.ones(H), K, V, norm_qs=True,
                                             norm_ks=True, alpha_qs=aq, alpha_ks=ak)
    nq = torch.stack([torch.nn.functional.rms_norm(torch.from_numpy(Qs[h]), (D,), weight=torch.from_numpy(aq[h]),
                                                   eps=1e-6) for h in range(H)])
    nk = torch.stack([torch.nn.functional.rms_norm(torch.from_numpy(Ks[:, h]), (D,), weight=torch.from_numpy(ak[h]),
                                                   eps=1e-6) for h in range(H)], dim=1)
    Qd = _sdpa(torch, nq.unsqueeze(0).expand(Ks.shape[0], -1, -1, -1), nk, torch.from_numpy(Vs))
    np.testing.assert_allclose(Q, Qd.numpy(), rtol=1e-12, atol=1e-14)
    Z_ref = _sdpa(torch, Qd, torch.from_numpy(K), torch.from_numpy(V))
    Y_ref = _sdpa(torch, torch.from_numpy(K), Qd, Z_ref)
    np.testing.assert_allclose(Z, Z_ref.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(Y, Y_ref.numpy(), rtol=1e-11, atol=1e-13)


def test_routing_key_scale_moves_to_queries(orc):
    # N_a(K) = alpha * N_0(K) channel by channel, so the routing scores
    # q . N_a(k) equal (q * alpha) . N_0(k): the same forward with alpha moved
    # onto the queries (the identity the GPU kernels use)
    Qs, Ks, Qf, K, V, gate = _shapes(seed=50)
    H, M, D = Qs.shape
    ak = 1.0 + _rand(51, H, D, std=0.3)
    Y1, Q1, Z1, L1 = orc.flare_pp_forward_normed(Qs, Ks, Ks, Qf, gate, K, V, norm_k=True, alpha_k=ak)
    Kn = orc.rms_norm(K, None)
    Z2, L2 = orc.encode(Q1 * ak[None, :, None, :], Kn, V)
    np.testing.assert_allclose(Z1, Z2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L1, L2, rtol=1e-12, atol=1e-12)
