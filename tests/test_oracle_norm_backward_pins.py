"""Pins of the oracle's backward through the FLARE++ input norms
(oracle.rms_norm_backward, oracle.flare_pp_backward_normed; FLARE++ paper,
App. A.3, A.4 and Table 2 in A.7 for the norms, App. B.5 for the backward).

None re-types the oracle's formulas.  They check it against
  - PyTorch's own RMS norm (torch.nn.functional.rms_norm) differentiated by
    CPU autograd in float64, an independent library routine;
  - central finite differences of the oracle's normalised FLARE++ forward,
    itself pinned in test_oracle_norm_pins.py, along random directions in
    every raw input and every learned channel scale, for the FLARE++ and the
    simplified variants of Table 2.
"""
import numpy as np
import pytest
import torch


def _rand(seed, *shape, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _inner(a, b):
    return float(np.sum(np.asarray(a) * np.asarray(b)))


@pytest.mark.parametrize("with_alpha", [False, True])
@pytest.mark.parametrize("shape", [(3, 7, 4), (2, 3, 5, 8)])
def test_rms_norm_backward_matches_torch_autograd(orc, shape, with_alpha):
    H, D = shape[-3], shape[-1]
    # spread row magnitudes so the norm's Jacobian differs between rows
    x = _rand(1, *shape) * np.exp(_rand(2, *shape[:-1], 1, std=0.7))
    dy = _rand(3, *shape)
    alpha = 1.0 + _rand(4, H, D, std=0.2) if with_alpha else None
    eps = 1e-3  # large enough that a dropped eps term shows
    dx, da = orc.rms_norm_backward(x, dy, alpha, eps)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    at = torch.tensor(alpha, dtype=torch.float64, requires_grad=True) if with_alpha else None
    # torch normalises the last axis; the per-head channel scale broadcasts over rows
    y = torch.nn.functional.rms_norm(xt, (D,), None, eps)
    if with_alpha:
        y = y * at[:, None, :]
    y.backward(torch.tensor(dy))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-12)
    if with_alpha:
        np.testing.assert_allclose(da, at.grad.numpy(), rtol=1e-11, atol=1e-12)
    else:
        assert da is None


def _raw_problem(seed, variant, B=2, H=2, N=11, M=5, D=4):
    mag = lambda s, *sh: np.exp(_rand(s, *sh[:-1], 1, std=0.5))  # noqa: E731
    Qs = _rand(seed, H, M, D) * mag(seed + 10, H, M, D)
    Ks = _rand(seed + 1, B, H, N, D) * mag(seed + 11, B, H, N, D)
    Qf = _rand(seed + 2, H, M, D, std=0.5)
    K = _rand(seed + 3, B, H, N, D) * mag(seed + 12, B, H, N, D)
    V = _rand(seed + 4, B, H, N, D)
    gate = 1.0 / (1.0 + np.exp(-_rand(seed + 5, H)))
    a_qs = 1.0 + _rand(seed + 6, H, D, std=0.2)
    a_ks = 1.0 + _rand(seed + 7, H, D, std=0.2)
    a_k = 1.0 + _rand(seed + 8, H, D, std=0.2)
    if variant == "flarepp":  # Table 2: N_a(Qs), N_0(Ks) = Vs, N_0(Qf), N_a(K)
        return dict(Qs=Qs, Ks=Ks, Vs=Ks, Qf=Qf, gate=gate, K=K, V=V), \
            dict(norm_qs=True, norm_ks=True, norm_qf=True, norm_k=True, alpha_qs=a_qs, alpha_k=a_k)
    Vs = _rand(seed + 9, B, H, N, D)      # simplified: N_a(Qs), N_a(Ks), separate Vs, no blend
    return dict(Qs=Qs, Ks=Ks, Vs=Vs, Qf=np.zeros_like(Qf), gate=np.ones(H), K=K, V=V), \
        dict(norm_qs=True, norm_ks=True, alpha_qs=a_qs, alpha_ks=a_ks)


@pytest.mark.parametrize("variant", ["flarepp", "simplified"])
def test_normed_pp_backward_matches_finite_differences(orc, variant):
    x, fl = _raw_problem(31, variant)
    shared = x["Vs"] is x["Ks"]
    dY = _rand(41, *x["K"].shape)
    eps = 1e-4
    grads = orc.flare_pp_backward_normed(x["Qs"], x["Ks"], x["Vs"], x["Qf"], x["gate"], x["K"], x["V"], dY,
                                         eps=eps, **fl)
    dQs, dKs, dVs, dQf, dgate, dK, dV, da_qs, da_ks, da_k = grads
    if shared:
        assert dVs is None

    def loss(**over):
        args = dict(x)
        f = dict(fl)
        for k, v in over.items():
            if k.startswith("alpha_"):
                f[k] = v
            else:
                args[k] = v
        if shared:
            args["Vs"] = args["Ks"]   # one array: keys and values move together
        Y, _, _, _ = orc.flare_pp_forward_normed(args["Qs"], args["Ks"], args["Vs"], args["Qf"], args["gate"],
                                                 args["K"], args["V"], eps=eps, **f)
        return _inner(Y, dY)

    h = 1e-5
    checks = [("Qs", dQs), ("Ks", dKs), ("Qf", dQf), ("gate", dgate), ("K", dK), ("V", dV)]
    if not shared:
        checks.append(("Vs", dVs))
    checks += [(k, g) for k, g in (("alpha_qs", da_qs), ("alpha_ks", da_ks), ("alpha_k", da_k)) if k in fl]
    rng = np.random.default_rng(5)
    for name, g in checks:
        base = fl[name] if name.startswith("alpha_") else x[name]
        assert g is not None and g.shape == np.shape(base), name
        for _ in range(2):
            u = rng.standard_normal(np.shape(base))
            fd = (loss(**{name: base + h * u}) - loss(**{name: base - h * u})) / (2 * h)
            an = _inner(g, u)
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)
