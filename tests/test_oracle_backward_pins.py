"""Pins of the fp64 backward oracle (FLARE++ paper, App. B.5 "Local backward",
and the derivative of the decoder's softmax over the latents, App. A.1).

None of these re-types the oracle's formulas.  They check it against
  - central finite differences of the oracle's forward, which is pinned on
    its own (test_oracle_pins.py): a dropped term, a wrong sign, a wrong
    scale or a transposed operand changes a directional derivative;
  - an independent library routine: PyTorch's CPU autograd in float64
    through torch.softmax;
  - closed forms of degenerate cases (one latent, one token) and the
    invariants that follow from the shift invariance of each softmax.
"""
import numpy as np
import pytest


def _rand(seed, *shape, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _inner(a, b):
    return float(np.sum(np.asarray(a) * np.asarray(b)))


def _problem(seed, B=2, H=2, N=9, M=5, D=4, q_batched=False):
    Q = _rand(seed, *((B, H, M, D) if q_batched else (H, M, D)), std=0.8)
    K = _rand(seed + 1, B, H, N, D)
    V = _rand(seed + 2, B, H, N, D)
    return Q, K, V


# --- finite differences of the pinned forward ------------------------------

EPS = 1e-5


def _fd(f, x, u):
    return (f(x + EPS * u) - f(x - EPS * u)) / (2 * EPS)


@pytest.mark.parametrize("q_batched", [False, True])
@pytest.mark.parametrize("scale", [0.0, 0.9])
def test_flare_backward_matches_finite_differences(orc, q_batched, scale):
    Q, K, V = _problem(11, q_batched=q_batched)
    dY = _rand(14, *K.shape)
    dQ, dK, dV = orc.flare_backward(Q, K, V, dY, scale=scale)

    def loss(Q_, K_, V_):
        return _inner(dY, orc.flare_forward(Q_, K_, V_, scale)[0])

    for i, (x, g) in enumerate(((Q, dQ), (K, dK), (V, dV))):
        u = _rand(20 + i, *x.shape)
        args = [Q, K, V]

        def f(y, i=i):
            a = list(args)
            a[i] = y
            return loss(*a)

        assert abs(_fd(f, x, u) - _inner(g, u)) <= 1e-7 * max(1.0, abs(_inner(g, u)))


@pytest.mark.parametrize("with_dL", [False, True])
def test_encode_backward_matches_finite_differences(orc, with_dL):
    # loss = <dZ, Z> + <dL, L>: both encoder outputs carry a cotangent (App. B.5)
    Q, K, V = _problem(31, N=11, M=6, D=3)
    dZ = _rand(34, 2, 2, 6, 3)
    dL = _rand(35, 2, 2, 6) if with_dL else None
    dQ, dK, dV = orc.encode_backward(Q, K, V, dZ, dL)

    def loss(Q_, K_, V_):
        Z, L = orc.encode(Q_, K_, V_)
        return _inner(dZ, Z) + (_inner(dL, L) if with_dL else 0.0)

    for i, (x, g) in enumerate(((Q, dQ), (K, dK), (V, dV))):
        u = _rand(40 + i, *x.shape)
        args = [Q, K, V]

        def f(y, i=i):
            a = list(args)
            a[i] = y
            return loss(*a)

        assert abs(_fd(f, x, u) - _inner(g, u)) <= 1e-7 * max(1.0, abs(_inner(g, u)))


def test_decode_backward_matches_finite_differences(orc):
    Q, K, _ = _problem(51, N=8, M=7, D=4, q_batched=True)
    Z = _rand(53, 2, 2, 7, 4)
    dY = _rand(54, *K.shape)
    dQ, dK, dZ = orc.decode_backward(Q, K, Z, dY)

    def loss(Q_, K_, Z_):
        return _inner(dY, orc.decode(Q_, K_, Z_))

    for i, (x, g) in enumerate(((Q, dQ), (K, dK), (Z, dZ))):
        u = _rand(60 + i, *x.shape)
        args = [Q, K, Z]

        def f(y, i=i):
            a = list(args)
            a[i] = y
            return loss(*a)

        assert abs(_fd(f, x, u) - _inner(g, u)) <= 1e-7 * max(1.0, abs(_inner(g, u)))


# --- an independent library routine -----------------------------------------

def test_flare_backward_matches_torch_autograd(orc):
    torch = pytest.importorskip("torch")
    Q, K, V = _problem(71, B=2, H=3, N=40, M=12, D=8)
    dY = _rand(74, *K.shape)
    s = 0.7
    q = torch.tensor(Q, requires_grad=True)
    k = torch.tensor(K, requires_grad=True)
    v = torch.tensor(V, requires_grad=True)
    enc = torch.softmax(s * torch.matmul(q.unsqueeze(0), k.transpose(-1, -2)), dim=-1)   # [B,H,M,N]
    z = torch.matmul(enc, v)
    dec = torch.softmax(s * torch.matmul(k, q.unsqueeze(0).transpose(-1, -2)), dim=-1)   # [B,H,N,M]
    y = torch.matmul(dec, z)
    y.backward(torch.tensor(dY))
    dQ, dK, dV, dZ = orc.flare_backward(Q, K, V, dY, scale=s, return_dZ=True)
    np.testing.assert_allclose(dQ, q.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, k.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, v.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_encode_backward_with_dL_matches_torch_autograd(orc):
    torch = pytest.importorskip("torch")
    Q, K, V = _problem(81, B=1, H=2, N=33, M=10, D=8, q_batched=True)
    dZ = _rand(84, 1, 2, 10, 8)
    dL = _rand(85, 1, 2, 10)
    q = torch.tensor(Q, requires_grad=True)
    k = torch.tensor(K, requires_grad=True)
    v = torch.tensor(V, requires_grad=True)
    sc = torch.matmul(q, k.transpose(-1, -2)) / np.sqrt(8.0)
    z = torch.matmul(torch.softmax(sc, dim=-1), v)
    lse = torch.logsumexp(sc, dim=-1)
    (torch.sum(z * torch.tensor(dZ)) + torch.sum(lse * torch.tensor(dL))).backward()
    dQ, dK, dV = orc.encode_backward(Q, K, V, dZ, dL)
    np.testing.assert_allclose(dQ, q.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, k.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, v.grad.numpy(), rtol=1e-10, atol=1e-12)


# --- closed forms and invariants -------------------------------------------

def test_one_latent_decoder_passes_dY_straight_to_Z(orc):
    # with M = 1 the decoder's softmax is identically 1, so Y_n = Z for every
    # token: dZ = sum_n dY_n and the decoder gives Q and K no gradient
    Q, K, _ = _problem(91, N=13, M=1, D=4)
    Z = _rand(93, 2, 2, 1, 4)
    dY = _rand(94, *K.shape)
    dQ, dK, dZ = orc.decode_backward(Q, K, Z, dY)
    np.testing.assert_allclose(dZ[:, :, 0], dY.sum(axis=2), rtol=1e-13, atol=1e-13)
    assert np.abs(dQ).max() < 1e-13 and np.abs(dK).max() < 1e-13


def test_one_token_encoder_closed_form(orc):
    # with N = 1 every encoder weight is 1 and Z_m = V_1, L_m = s q_m.k_1:
    # dV_1 = sum_m dZ_m, dS_m = dL_m, so dK_1 = s sum_m dL_m q_m and dQ_m = s dL_m k_1
    s = 0.5
    Q, K, V = _problem(101, B=1, H=1, N=1, M=4, D=3, q_batched=True)
    dZ = _rand(104, 1, 1, 4, 3)
    dL = _rand(105, 1, 1, 4)
    dQ, dK, dV = orc.encode_backward(Q, K, V, dZ, dL, scale=s)
    np.testing.assert_allclose(dV[0, 0, 0], dZ[0, 0].sum(axis=0), rtol=1e-13)
    np.testing.assert_allclose(dK[0, 0, 0], s * dL[0, 0] @ Q[0, 0], rtol=1e-12)
    np.testing.assert_allclose(dQ[0, 0], s * dL[0, 0][:, None] * K[0, 0, 0][None, :], rtol=1e-12)


def test_shift_invariance_of_the_softmaxes(orc):
    # Adding one vector to every key shifts each encoder score row by a
    # constant, which the softmax over tokens ignores, while L_m moves by
    # s q_m.u: so sum_n dK_enc,n = s sum_m dL_m q_m.  Adding one vector to
    # every latent query shifts each decoder row by a constant: the decoder
    # queries' gradients sum to zero.
    s = 0.6
    Q, K, V = _problem(111, B=2, H=2, N=17, M=6, D=4, q_batched=True)
    dZ = _rand(114, 2, 2, 6, 4)
    dL = _rand(115, 2, 2, 6)
    _, dK, _ = orc.encode_backward(Q, K, V, dZ, dL, scale=s)
    np.testing.assert_allclose(dK.sum(axis=2), s * np.einsum("bhm,bhmd->bhd", dL, Q), rtol=1e-10, atol=1e-12)
    Z = _rand(116, 2, 2, 6, 4)
    dY = _rand(117, *K.shape)
    dQ, _, _ = orc.decode_backward(Q, K, Z, dY, scale=s)
    assert np.abs(dQ.sum(axis=2)).max() < 1e-12


def test_shared_queries_sum_the_batch(orc):
    # Q shared over the batch ([H,M,D]): its cotangent is the sum over b of
    # the cotangents of per-batch copies
    Q, K, V = _problem(121, B=3, H=2, N=10, M=5, D=4)
    dY = _rand(124, *K.shape)
    dQ, dK, dV = orc.flare_backward(Q, K, V, dY)
    Qb = np.broadcast_to(Q, (3,) + Q.shape).copy()
    dQb, dKb, dVb = orc.flare_backward(Qb, K, V, dY)
    np.testing.assert_allclose(dQ, dQb.sum(axis=0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dK, dKb, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dV, dVb, rtol=1e-13, atol=1e-15)


# --- FLARE++ (App. B.5: the synthesis encoder receives the reduced query cotangent) ---

def _pp_problem(seed, B=2, H=2, N=9, M=5, D=4):
    r = [_rand(seed + i, *s) for i, s in enumerate([(H, M, D), (B, H, N, D), (B, H, N, D), (H, M, D), (B, H, N, D),
                                                     (B, H, N, D)])]
    Qs, Ks, Vs, Qf, K, V = r
    gate = 0.3 + 0.5 * np.abs(_rand(seed + 9, H))
    return Qs, Ks, Vs, Qf, gate, K, V


@pytest.mark.parametrize("shared", [True, False])
def test_pp_backward_matches_finite_differences(orc, shared):
    Qs, Ks, Vs, Qf, gate, K, V = _pp_problem(131)
    if shared:
        Vs = Ks
    dY = _rand(140, *K.shape)
    dQs, dKs, dVs, dQf, dg, dK, dV = orc.flare_pp_backward(Qs, Ks, Vs, Qf, gate, K, V, dY)
    names = ["Qs", "Ks", "Vs", "Qf", "gate", "K", "V"]
    grads = {"Qs": dQs, "Ks": dKs, "Vs": dVs, "Qf": dQf, "gate": dg, "K": dK, "V": dV}
    base = dict(Qs=Qs, Ks=Ks, Vs=Vs, Qf=Qf, gate=gate, K=K, V=V)

    def loss(**a):
        vs = a["Ks"] if shared else a["Vs"]
        return _inner(dY, orc.flare_pp_forward(a["Qs"], a["Ks"], vs, a["Qf"], a["gate"], a["K"], a["V"])[0])

    for i, n in enumerate(names):
        if shared and n == "Vs":
            assert dVs is None
            continue
        u = _rand(150 + i, *base[n].shape)

        def f(y, n=n):
            a = dict(base)
            a[n] = y
            return loss(**a)

        g = grads[n]
        assert abs(_fd(f, base[n], u) - _inner(g, u)) <= 1e-7 * max(1.0, abs(_inner(g, u))), n


def test_pp_backward_matches_torch_autograd(orc):
    torch = pytest.importorskip("torch")
    Qs, Ks, Vs, Qf, gate, K, V = _pp_problem(161, B=2, H=2, N=30, M=8, D=8)
    dY = _rand(170, *K.shape)
    s = 1.0 / np.sqrt(8.0)
    t = {n: torch.tensor(x, requires_grad=True) for n, x in dict(Qs=Qs, Ks=Ks, Qf=Qf, gate=gate, K=K, V=V).items()}

    def sdpa(q, k, v):
        return torch.matmul(torch.softmax(s * torch.matmul(q, k.transpose(-1, -2)), dim=-1), v)

    qd = sdpa(t["Qs"].unsqueeze(0), t["Ks"], t["Ks"])                       # shared keys and values
    q = t["Qf"].unsqueeze(0) + t["gate"][None, :, None, None] * qd
    z = sdpa(q, t["K"], t["V"])
    y = sdpa(t["K"], q, z)
    y.backward(torch.tensor(dY))
    dQs, dKs, dVs, dQf, dg, dK, dV = orc.flare_pp_backward(Qs, Ks, Ks, Qf, gate, K, V, dY)
    assert dVs is None
    for n, g in dict(Qs=dQs, Ks=dKs, Qf=dQf, gate=dg, K=dK, V=dV).items():
        np.testing.assert_allclose(g, t[n].grad.numpy(), rtol=1e-9, atol=1e-12, err_msg=n)
