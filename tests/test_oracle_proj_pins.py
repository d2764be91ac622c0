"""Pins of the oracle's fused-projection forwards (oracle.flare_forward_proj,
oracle.flare_pp_forward_proj): the per-head projections K = X W_K, V = X W_V
of the FLARE++ paper's Sec. 3.1 feeding the FLARE pair, and for FLARE++ the
synthesis keys X W~_K with the Table 2 norms.

Each is checked against things other than itself: an independent PyTorch
float64 composition (torch.matmul, F.rms_norm and F.scaled_dot_product_attention,
CPU), the identity projection reducing to the unprojected oracle, linearity in
the value projection and head equivariance.  A transposed W, a wrong head
index or a dropped norm fails the first two; a projection applied to the wrong
operand fails the torch pins."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F


def _gauss(seed, shape, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _torch(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))


def _sdpa(q, k, v, s):
    return F.scaled_dot_product_attention(q, k, v, scale=s)


def torch_flare_proj(X, WK, WV, Q, s):
    X, WK, WV, Q = map(_torch, (X, WK, WV, Q))
    K = torch.matmul(X.unsqueeze(1), WK.unsqueeze(0))       # [B,H,N,D]
    V = torch.matmul(X.unsqueeze(1), WV.unsqueeze(0))
    Qb = Q.unsqueeze(0).expand(K.shape[0], -1, -1, -1)
    Z = _sdpa(Qb, K, V, s)
    return _sdpa(K, Qb, Z, s).numpy(), Z.numpy()


def torch_flare_pp_proj(X, WKs, WK, WV, Qs, Qf, gate, a_qs, a_k, s, eps=1e-6):
    X, WKs, WK, WV, Qs, Qf, gate, a_qs, a_k = map(_torch, (X, WKs, WK, WV, Qs, Qf, gate, a_qs, a_k))
    D = WK.shape[-1]

    def proj(W):
        return torch.matmul(X.unsqueeze(1), W.unsqueeze(0))
    Ks = F.rms_norm(proj(WKs), (D,), eps=eps)               # N_0, shared keys and values
    K = F.rms_norm(proj(WK), (D,), eps=eps) * a_k[None, :, None, :]
    V = proj(WV)
    B = X.shape[0]
    Qsn = (F.rms_norm(Qs, (D,), eps=eps) * a_qs[:, None, :]).unsqueeze(0).expand(B, -1, -1, -1)
    Qd = _sdpa(Qsn, Ks, Ks, s)
    Q = F.rms_norm(Qf, (D,), eps=eps).unsqueeze(0) + gate[None, :, None, None] * Qd
    Z = _sdpa(Q, K, V, s)
    return _sdpa(K, Q, Z, s).numpy(), Q.numpy(), Z.numpy()


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


@pytest.mark.parametrize("B,H,N,M,C,D", [(2, 3, 97, 8, 24, 8), (1, 2, 300, 16, 128, 32)])
def test_proj_matches_torch_float64(orc, B, H, N, M, C, D):
    X = _gauss(1, (B, N, C))
    WK, WV = _gauss(2, (H, C, D), 1 / math.sqrt(C)), _gauss(3, (H, C, D), 1 / math.sqrt(C))
    Q = _gauss(4, (H, M, D), 1 / math.sqrt(D))
    Y, Z, L = orc.flare_forward_proj(X, WK, WV, Q)
    Yt, Zt = torch_flare_proj(X, WK, WV, Q, 1 / math.sqrt(D))
    assert rel(Y, Yt) < 1e-12 and rel(Z, Zt) < 1e-12


def test_pp_proj_matches_torch_float64(orc):
    B, H, N, M, C, D = 2, 2, 150, 8, 32, 16
    X = _gauss(5, (B, N, C))
    WKs, WK, WV = (_gauss(6 + i, (H, C, D), 1 / math.sqrt(C)) for i in range(3))
    Qs, Qf = _gauss(9, (H, M, D), 0.3), _gauss(10, (H, M, D), 0.3)
    gate = np.array([0.3, 0.7])
    a_qs, a_k = 1 + _gauss(11, (H, D), 0.1), 1 + _gauss(12, (H, D), 0.1)
    Y, Q, Z, L = orc.flare_pp_forward_proj(X, WKs, WK, WV, Qs, Qf, gate, norm_qs=True, norm_ks=True, norm_qf=True,
                                           norm_k=True, alpha_qs=a_qs, alpha_k=a_k)
    Yt, Qt, Zt = torch_flare_pp_proj(X, WKs, WK, WV, Qs, Qf, gate, a_qs, a_k, 1 / math.sqrt(D))
    assert rel(Q, Qt) < 1e-12 and rel(Z, Zt) < 1e-12 and rel(Y, Yt) < 1e-12


def test_identity_projection_is_the_unprojected_forward(orc):
    """C = D and W = I for every head: K = V = X for every head."""
    B, H, N, M, D = 2, 3, 200, 8, 16
    X = _gauss(13, (B, N, D))
    I = np.broadcast_to(np.eye(D), (H, D, D))
    Q = _gauss(14, (H, M, D), 0.25)
    Y, Z, L = orc.flare_forward_proj(X, I, I, Q)
    Kh = np.broadcast_to(X[:, None], (B, H, N, D))
    Yr, Zr, Lr = orc.flare_forward(Q, Kh, Kh)
    assert rel(Y, Yr) < 1e-14 and rel(Z, Zr) < 1e-14 and np.allclose(L, Lr, rtol=1e-14, atol=1e-14)


def test_linear_in_the_value_projection(orc):
    """V = X W_V is linear in W_V and Y is linear in V (the weights do not see V)."""
    B, H, N, M, C, D = 1, 2, 120, 8, 24, 8
    X = _gauss(15, (B, N, C))
    WK, W1, W2 = (_gauss(16 + i, (H, C, D), 0.2) for i in range(3))
    Q = _gauss(19, (H, M, D), 0.3)
    Y1, _, _ = orc.flare_forward_proj(X, WK, W1, Q)
    Y2, _, _ = orc.flare_forward_proj(X, WK, W2, Q)
    Y12, _, _ = orc.flare_forward_proj(X, WK, 2.0 * W1 - 0.5 * W2, Q)
    assert rel(Y12, 2.0 * Y1 - 0.5 * Y2) < 1e-12


def test_head_permutation_is_equivariant(orc):
    """Permuting the heads of W_K, W_V and Q permutes the heads of Y and Z."""
    B, H, N, M, C, D = 1, 3, 90, 8, 16, 8
    X = _gauss(20, (B, N, C))
    WK, WV = _gauss(21, (H, C, D), 0.3), _gauss(22, (H, C, D), 0.3)
    Q = _gauss(23, (H, M, D), 0.3)
    p = [2, 0, 1]
    Y, Z, _ = orc.flare_forward_proj(X, WK, WV, Q)
    Yp, Zp, _ = orc.flare_forward_proj(X, WK[p], WV[p], Q[p])
    assert rel(Yp, Y[:, p]) < 1e-14 and rel(Zp, Z[:, p]) < 1e-14
