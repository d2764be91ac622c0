"""GPU parity of the float32 backward (flare_backward, flare_encode_backward
and flare_pp_backward with FLARE_F32 through the C ABI) against the fp64
oracle's flare_backward, encode_backward and flare_pp_backward.

The float32 forward runs on the GPU first and its Z, L (and, for FLARE++,
routing queries) are what the backward takes; the oracle recomputes
everything from the same float32 inputs in fp64.  Bars: rel-L2 1e-5 on every
gradient (float32 inputs) and, per row (a token of dK / dV, a latent of dQ /
dZ), ROW_FACTOR times that relative to the row's norm floored at the RMS row
norm.
"""
import math
import sys

import numpy as np
import pytest

from helpers import ROW_FACTOR, TOL, dev, host, rel_l2, row_err

pytestmark = pytest.mark.gpu
BAR = TOL["f32"]


@pytest.fixture(scope="module")
def flare():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_attention_amd as r
    r.load()
    return r


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(name, got, ref, tol=BAR):
    assert np.all(np.isfinite(got)), name
    e, r = rel_l2(got, ref), row_err(got, ref)
    say(f"  {name}: rel-L2 {e:.3e}, worst row {r:.3e} (bars {tol:g}, {ROW_FACTOR * tol:g})")
    assert e <= tol, f"{name}: rel-L2 {e:.3e} > {tol:g}"
    assert r <= ROW_FACTOR * tol, f"{name}: worst row {r:.3e} > {ROW_FACTOR * tol:g}"


def gpu_backward(flare, Q, K, V, dY, scale=0.0):
    """float32 forward then backward on the GPU; host (dQ, dK, dV, dZ)."""
    import torch
    Qd, Kd, Vd, dYd = dev(Q, "f32"), dev(K, "f32"), dev(V, "f32"), dev(dY, "f32")
    B, H, N, D = K.shape
    M = Q.shape[-2]
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=Kd.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=Kd.device)
    flare.flare_forward(Qd, Kd, Vd, scale=scale, Z=Z, L=L)
    dZ = torch.empty_like(Z)
    dQ, dK, dV, _ = flare.flare_backward(Qd, Kd, Vd, Z, L, dYd, scale=scale, dZ=dZ)
    torch.cuda.synchronize()
    assert dK.dtype == torch.float32 and dV.dtype == torch.float32
    return host(dQ), host(dK), host(dV), host(dZ)


def compare(orc, flare, Q, K, V, dY, scale=0.0):
    got = gpu_backward(flare, Q, K, V, dY, scale)
    ref = orc.flare_backward(Q, K, V, dY, scale=scale, return_dZ=True)
    for n, g, r in zip(("dQ", "dK", "dV", "dZ"), got, ref):
        check(n, g, r)


# shared and per-batch queries, both head sizes, ragged token counts that
# span several tiles and splits, latent counts that are not multiples of 32
# or 64, and M = 256 with D = 32 (the largest row-pass LDS)
SHAPES = [  # B, H, N, M, D, q_batched
    (1, 2, 3001, 64, 32, False), (2, 3, 1000, 48, 16, True), (1, 1, 5, 3, 16, False),
    (1, 1, 777, 33, 32, True), (1, 2, 2100, 256, 32, False), (2, 2, 4097, 100, 16, False),
]


def test_backward_f32_single_token(flare, orc):
    """N = 1: dQ = dK = 0 exactly (see the bf16 test of the same case); their
    computed values are rounding noise, bounded against dV; dV and dZ match
    the oracle at the float32 bar."""
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    w = make_gaussian(1, 3, 1, 28, 32, "f32", seed=95)
    dY = cotangent(96, "dy", w.K.shape, dtype="f32")
    say("[backward f32] B1 H3 N1 M28 D32")
    dQ, dK, dV, dZ = gpu_backward(flare, w.Q, w.K, w.V, dY)
    ref = orc.flare_backward(w.Q, w.K, w.V, dY, return_dZ=True)
    check("dV", dV, ref[2])
    check("dZ", dZ, ref[3])
    big = np.linalg.norm(dV)
    say(f"  |dQ| {np.linalg.norm(dQ):.2e}, |dK| {np.linalg.norm(dK):.2e}, |dV| {big:.2e}")
    assert np.all(np.isfinite(dQ)) and np.all(np.isfinite(dK))
    assert np.linalg.norm(dQ) <= 1e-5 * big and np.linalg.norm(dK) <= 1e-5 * big


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}N{}M{}D{}qb{}".format(*s))
def test_backward_f32_gaussian(flare, orc, shape):
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    B, H, N, M, D, qb = shape
    w = make_gaussian(B, H, N, M, D, "f32", seed=191)
    Q = np.broadcast_to(w.Q, (B,) + w.Q.shape).copy() if qb else w.Q
    dY = cotangent(192, "dy", w.K.shape, "f32")
    say(f"[backward f32] B{B} H{H} N{N} M{M} D{D} q_batched {qb}")
    compare(orc, flare, Q, w.K, w.V, dY)


def test_backward_f32_single_head_workload(flare, orc):
    # the single-head float32 workload (B1 H1 N1024 M32 D16), whole
    from rank_latent_attention_amd.inputs import config1, cotangent
    w = config1()
    say(f"[backward f32] {w.name}")
    compare(orc, flare, w.Q, w.K, w.V, cotangent(193, "dy", w.K.shape, "f32"))


def test_backward_f32_pde_mesh_workload(flare, orc):
    # the PDE-mesh float32 workload (B4 H8 N16641 M128 D16), whole: latents
    # with a large common part, the case the decoder side centres them for
    from rank_latent_attention_amd.inputs import config2, cotangent
    w = config2("f32")
    say(f"[backward f32] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D}")
    compare(orc, flare, w.Q, w.K, w.V, cotangent(194, "dy", w.K.shape, "f32"))


def test_backward_f32_explicit_scale(flare, orc):
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    w = make_gaussian(1, 2, 2500, 64, 32, "f32", seed=195)
    say("[backward f32] explicit scale 0.4")
    compare(orc, flare, w.Q, w.K, w.V, cotangent(196, "dy", w.K.shape, "f32"), scale=0.4)


def test_backward_f32_large_scores(flare, orc):
    # log2 scores up to 160 (sign keys, queries 1..5 x a key, scale
    # 1 / log2 e): every weight keeps its exact shift, none overflows
    from rank_latent_attention_amd.inputs import cotangent
    rng = np.random.default_rng(197)
    N, M, D = 900, 36, 32
    K = (rng.integers(0, 2, size=(1, 1, N, D)) * 2 - 1).astype(np.float32)
    V = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    Q = np.zeros((1, M, D), np.float32)
    pick = rng.choice(N, size=M, replace=False)
    Q[0] = K[0, 0, pick] * rng.integers(1, 6, size=(M, 1))
    say("[backward f32] log2 scores up to 160")
    compare(orc, flare, Q, K, V, cotangent(198, "dy", K.shape, "f32"), scale=1.0 / math.log2(math.e))


@pytest.mark.parametrize("with_dL", [False, True])
def test_encode_backward_f32(flare, orc, with_dL):
    import torch
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    B, H, N, M, D = 2, 2, 3000, 96, 32
    w = make_gaussian(B, H, N, M, D, "f32", seed=199)
    dZ = cotangent(200, "dz", (B, H, M, D), "f32")
    dL = cotangent(201, "dl", (B, H, M), "f32") if with_dL else None
    Qd, Kd, Vd = dev(w.Q, "f32"), dev(w.K, "f32"), dev(w.V, "f32")
    Z, L = flare.flare_encode(Qd, Kd, Vd)
    dQ, dK, dV = flare.flare_encode_backward(Qd, Kd, Vd, Z, L, dev(dZ, "f32"), None if dL is None else dev(dL, "f32"))
    torch.cuda.synchronize()
    ref = orc.encode_backward(w.Q, w.K, w.V, dZ, dL)
    say(f"[encode backward f32] dL {with_dL}")
    for n, g, r in zip(("dQ", "dK", "dV"), (host(dQ), host(dK), host(dV)), ref):
        check(n, g, r)


def test_backward_f32_is_deterministic(flare):
    import torch
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    w = make_gaussian(1, 2, 9000, 128, 32, "f32", seed=202)
    Qd, Kd, Vd = dev(w.Q, "f32"), dev(w.K, "f32"), dev(w.V, "f32")
    dYd = dev(cotangent(203, "dy", w.K.shape, "f32"), "f32")
    Z = torch.empty((1, 2, 128, 32), dtype=torch.float32, device=Kd.device)
    L = torch.empty((1, 2, 128), dtype=torch.float32, device=Kd.device)
    flare.flare_forward(Qd, Kd, Vd, Z=Z, L=L)
    a = flare.flare_backward(Qd, Kd, Vd, Z, L, dYd)
    b = flare.flare_backward(Qd, Kd, Vd, Z, L, dYd)
    torch.cuda.synchronize()
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


def test_backward_f32_without_tokens(flare):
    # N = 0: the forward gives Z = 0 and L = -inf; the query and latent
    # cotangents are zero
    import torch
    Q = torch.randn(2, 16, 16, device="cuda:0")
    K = torch.empty((1, 2, 0, 16), dtype=torch.float32, device="cuda:0")
    Z = torch.zeros((1, 2, 16, 16), device="cuda:0")
    L = torch.full((1, 2, 16), -float("inf"), device="cuda:0")
    dQ = torch.full((2, 16, 16), 7.0, device="cuda:0")
    dZ = torch.full((1, 2, 16, 16), 7.0, device="cuda:0")
    flare.flare_backward(Q, K, K, Z, L, K, dQ=dQ, dZ=dZ)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dQ).item() == 0 and torch.count_nonzero(dZ).item() == 0


def test_backward_f32_workspace_too_small(flare):
    import torch
    Q = torch.zeros(1, 32, 16, device="cuda:0")
    K = torch.zeros(1, 1, 64, 16, device="cuda:0")
    Z = torch.zeros(1, 1, 32, 16, device="cuda:0")
    L = torch.zeros(1, 1, 32, device="cuda:0")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(flare.FlareError) as e:
        flare.flare_backward(Q, K, K, Z, L, K, ws=ws)
    assert e.value.status == 3


# --- FLARE++ in float32 ---

PP_NAMES = ("dQs", "dKs", "dVs", "dQf", "dgate", "dK", "dV")


@pytest.mark.parametrize("shape", [(2, 2, 3000, 64, 32, True), (2, 2, 3000, 64, 32, False),
                                   (1, 3, 1000, 48, 16, True), (2, 1, 777, 33, 32, False)],
                         ids=lambda s: "B{}H{}N{}M{}D{}shared{}".format(*s))
def test_pp_backward_f32(flare, orc, shape):
    import torch
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian_pp
    B, H, N, M, D, shared = shape
    w = make_gaussian_pp(B, H, N, M, D, "f32", seed=211, share_vs=shared)
    dY = cotangent(212, "dy", w.K.shape, "f32")
    say(f"[pp backward f32] B{B} H{H} N{N} M{M} D{D} shared {shared}")
    d = "f32"
    Qs, Ks, Qf, K, V = dev(w.Qs, d), dev(w.Ks, d), dev(w.Qf, d), dev(w.K, d), dev(w.V, d)
    Vs = Ks if shared else dev(w.Vs, d)
    gate = dev(w.gate, "f32")
    Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    flare.flare_pp_forward(Qs, Ks, Vs, Qf, gate, K, V, Q_out=Qo, Z=Z, L=L)
    out = flare.flare_pp_backward(Qs, Ks, Vs, Qf, gate, K, V, Qo, Z, L, dev(dY, d))
    torch.cuda.synchronize()
    got = tuple(None if x is None else host(x) for x in out[:7])
    ref = orc.flare_pp_backward(w.Qs, w.Ks, w.Ks if shared else w.Vs, w.Qf, w.gate, w.K, w.V, dY, shared_vs=shared)
    for n, g, r in zip(PP_NAMES, got, ref):
        if r is None:
            assert g is None, n
            continue
        if n == "dgate":  # one value per head: the rel-L2 bar alone
            e = rel_l2(g, r)
            say(f"  dgate: rel-L2 {e:.3e} (bar {BAR:g})")
            assert e <= BAR
            continue
        check(n, g, r)


@pytest.mark.parametrize("shape", [(2, 3, 5221, 93, 32, True, 0.0), (1, 5, 12000, 64, 16, False, 0.3),
                                   (3, 2, 777, 256, 32, False, 0.11), (1, 1, 2, 7, 16, True, 0.0)],
                         ids=lambda s: "B{}H{}N{}M{}D{}qb{}s{}".format(*s))
def test_backward_f32_more_shapes(flare, orc, shape):
    """Irregular M, an explicit scale 1.2 times the default (D = 16), two
    tokens, per-batch queries: the float32 bar on every gradient."""
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    B, H, N, M, D, qb, scale = shape
    w = make_gaussian(B, H, N, M, D, "f32", seed=N + M)
    Q = np.broadcast_to(w.Q, (B,) + w.Q.shape).copy() if qb else w.Q
    dY = cotangent(N + M + 1, "dy", w.K.shape, dtype="f32")
    say(f"[backward f32] B{B} H{H} N{N} M{M} D{D} q_batched {qb} scale {scale}")
    compare(orc, flare, Q, w.K, w.V, dY, scale=scale)
