"""GPU parity of the backward (flare_backward, flare_encode_backward and
flare_pp_backward through the C ABI) against the fp64 oracle's
flare_backward, encode_backward and flare_pp_backward.

The forward runs on the GPU first (its Z, L and, for FLARE++, routing
queries are what the backward takes, as in training); the oracle recomputes
everything from the same bf16 inputs in fp64.  Bar: rel-L2 1e-2 on every
gradient (bf16 inputs, float32 accumulation, bf16 matrix-core operands).
"""
import sys

import numpy as np
import pytest

from helpers import TOL, dev, host, rel_l2

pytestmark = pytest.mark.gpu


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


def check(name, got, ref, tol=TOL["bf16"]):
    e = rel_l2(got, ref)
    say(f"  {name}: rel-L2 {e:.3e} (bar {tol:g})")
    assert e <= tol, f"{name}: rel-L2 {e:.3e} > {tol:g}"


def gpu_backward(flare, Q, K, V, dY, scale=0.0):
    """Forward then backward on the GPU; returns host (dQ, dK, dV, dZ)."""
    import torch
    Qd, Kd, Vd, dYd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), dev(dY, "bf16")
    B, H, N, D = K.shape
    M = Q.shape[-2]
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=Kd.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=Kd.device)
    flare.flare_forward(Qd, Kd, Vd, scale=scale, Z=Z, L=L)
    dZ = torch.empty_like(Z)
    dQ, dK, dV, _ = flare.flare_backward(Qd, Kd, Vd, Z, L, dYd, scale=scale, dZ=dZ)
    torch.cuda.synchronize()
    return host(dQ), host(dK), host(dV), host(dZ)


def compare(orc, flare, Q, K, V, dY, scale=0.0):
    got = gpu_backward(flare, Q, K, V, dY, scale)
    ref = orc.flare_backward(Q, K, V, dY, scale=scale, return_dZ=True)
    for n, g, r in zip(("dQ", "dK", "dV", "dZ"), got, ref):
        assert np.all(np.isfinite(g)), n
        check(n, g, r)


# shared and per-batch queries, both head sizes, ragged token counts that
# span several tiles and splits, latent counts with a partial last block
SHAPES = [  # B, H, N, M, D, q_batched
    (1, 2, 3001, 64, 32, False), (2, 3, 1000, 48, 16, True), (1, 1, 5, 3, 16, False),
    (2, 2, 20000, 256, 32, False), (1, 1, 777, 33, 32, True), (1, 4, 4096, 128, 16, False),
]


def test_backward_single_token(flare, orc):
    """N = 1: every latent is the one value row and so is every output, for
    any queries and key (the encode's softmax over one token is 1, and the
    decode's weights sum to one over equal latents), so dQ = dK = 0 exactly.
    A relative error against that zero is meaningless: their computed values
    are rounding noise, bounded against dV (= dY here); dV and dZ match the
    oracle."""
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    w = make_gaussian(2, 3, 1, 64, 16, "bf16", seed=93)
    dY = cotangent(94, "dy", w.K.shape)
    say("[backward] B2 H3 N1 M64 D16")
    dQ, dK, dV, dZ = gpu_backward(flare, w.Q, w.K, w.V, dY)
    ref = orc.flare_backward(w.Q, w.K, w.V, dY, return_dZ=True)
    check("dV", dV, ref[2])
    check("dZ", dZ, ref[3])
    big = np.linalg.norm(dV)
    say(f"  |dQ| {np.linalg.norm(dQ):.2e}, |dK| {np.linalg.norm(dK):.2e}, |dV| {big:.2e}")
    assert np.all(np.isfinite(dQ)) and np.all(np.isfinite(dK))
    assert np.linalg.norm(dQ) <= 1e-5 * big and np.linalg.norm(dK) <= 1e-5 * big


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}N{}M{}D{}qb{}".format(*s))
def test_backward_gaussian(flare, orc, shape):
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    B, H, N, M, D, qb = shape
    w = make_gaussian(B, H, N, M, D, "bf16", seed=91)
    Q = np.broadcast_to(w.Q, (B,) + w.Q.shape).copy() if qb else w.Q
    dY = cotangent(92, "dy", w.K.shape)
    say(f"[backward] B{B} H{H} N{N} M{M} D{D} q_batched {qb}")
    compare(orc, flare, Q, w.K, w.V, dY)


def test_backward_explicit_scale(flare, orc):
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    w = make_gaussian(1, 2, 2500, 64, 32, "bf16", seed=93)
    say("[backward] explicit scale 0.4")
    compare(orc, flare, w.Q, w.K, w.V, cotangent(94, "dy", w.K.shape), scale=0.4)


def test_backward_structured_mesh(flare, orc):
    # keys and values from random Fourier features of a point cloud (the
    # irregular-mesh workload, a few batches): latents with a large common part
    from rank_latent_attention_amd.inputs import config3, cotangent
    w = config3(256)
    sl = slice(0, 2)
    Q, K, V = w.Q[:2], w.K[sl, :2], w.V[sl, :2]
    say(f"[backward] {w.name} B2 H2 N{w.N} M{w.M} D{w.D}")
    compare(orc, flare, Q, K, V, cotangent(95, "dy", K.shape))


@pytest.mark.parametrize("with_dL", [False, True])
def test_encode_backward(flare, orc, with_dL):
    import torch
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    B, H, N, M, D = 2, 2, 3000, 96, 32
    w = make_gaussian(B, H, N, M, D, "bf16", seed=96)
    dZ = cotangent(97, "dz", (B, H, M, D), "f32")
    dL = cotangent(98, "dl", (B, H, M), "f32") if with_dL else None
    Qd, Kd, Vd = dev(w.Q, "bf16"), dev(w.K, "bf16"), dev(w.V, "bf16")
    Z, L = flare.flare_encode(Qd, Kd, Vd)
    dQ, dK, dV = flare.flare_encode_backward(Qd, Kd, Vd, Z, L, dev(dZ, "f32"),
                                             None if dL is None else dev(dL, "f32"))
    torch.cuda.synchronize()
    ref = orc.encode_backward(w.Q, w.K, w.V, dZ, dL)
    say(f"[encode backward] dL {with_dL}")
    for n, g, r in zip(("dQ", "dK", "dV"), (host(dQ), host(dK), host(dV)), ref):
        check(n, g, r)


def test_backward_is_deterministic(flare):
    import torch
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    w = make_gaussian(1, 2, 9000, 128, 32, "bf16", seed=99)
    Qd, Kd, Vd = dev(w.Q, "bf16"), dev(w.K, "bf16"), dev(w.V, "bf16")
    dYd = dev(cotangent(100, "dy", w.K.shape), "bf16")
    Z = torch.empty((1, 2, 128, 32), dtype=torch.float32, device=Kd.device)
    L = torch.empty((1, 2, 128), dtype=torch.float32, device=Kd.device)
    flare.flare_forward(Qd, Kd, Vd, Z=Z, L=L)
    a = flare.flare_backward(Qd, Kd, Vd, Z, L, dYd)
    b = flare.flare_backward(Qd, Kd, Vd, Z, L, dYd)
    torch.cuda.synchronize()
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)


def test_backward_without_tokens(flare):
    # N = 0: the forward gives Z = 0 and L = -inf; nothing reaches the queries
    import torch
    Q = torch.randn(2, 16, 16, device="cuda:0").to(torch.bfloat16)
    K = torch.empty((1, 2, 0, 16), dtype=torch.bfloat16, device="cuda:0")
    Z = torch.zeros((1, 2, 16, 16), device="cuda:0")
    L = torch.full((1, 2, 16), -float("inf"), device="cuda:0")
    dQ = torch.full((2, 16, 16), 7.0, device="cuda:0")
    flare.flare_backward(Q, K, K, Z, L, K, dQ=dQ)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dQ).item() == 0


def test_backward_workspace_too_small(flare):
    import torch
    Q = torch.zeros(1, 32, 16, dtype=torch.bfloat16, device="cuda:0")
    K = torch.zeros(1, 1, 64, 16, dtype=torch.bfloat16, device="cuda:0")
    Z = torch.zeros(1, 1, 32, 16, device="cuda:0")
    L = torch.zeros(1, 1, 32, device="cuda:0")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(flare.FlareError) as e:
        flare.flare_backward(Q, K, K, Z, L, K, ws=ws)
    assert e.value.status == 3


def test_million_token_backward_one_head(flare, orc):
    # the million-point surface-mesh workload launched whole (all eight
    # heads, the benchmark's launch configuration); one head is checked in
    # full against the oracle (dQ and dZ reduce over all 2^20 tokens)
    import torch
    from rank_latent_attention_amd.inputs import config5, cotangent
    w = config5(False)
    dY = cotangent(101, "dy", w.K.shape)
    say(f"[c5 backward] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D}")
    dQ, dK, dV, dZ = gpu_backward(flare, w.Q, w.K, w.V, dY)
    for n, x in (("dQ", dQ), ("dK", dK), ("dV", dV), ("dZ", dZ)):
        assert np.all(np.isfinite(x)), n
    h = 3
    sl = slice(h, h + 1)
    ref = orc.flare_backward(w.Q[sl], w.K[:, sl], w.V[:, sl], dY[:, sl], return_dZ=True)
    for n, g, r in zip(("dQ", "dK", "dV", "dZ"), (dQ[sl], dK[:, sl], dV[:, sl], dZ[:, sl]), ref):
        check(f"head {h} {n}", g, r)


# --- FLARE++ (App. B.5: the synthesis encoder receives the reduced query cotangent) ---

def gpu_pp_backward(flare, w, dY, shared=True):
    """GPU FLARE++ forward then backward; returns the host gradients in the
    oracle's order (dQs, dKs, dVs or None, dQf, dgate, dK, dV)."""
    import torch
    d = "bf16"
    Qs, Ks, Qf, K, V = dev(w.Qs, d), dev(w.Ks, d), dev(w.Qf, d), dev(w.K, d), dev(w.V, d)
    Vs = Ks if shared else dev(w.Vs, d)
    gate = dev(w.gate, "f32")
    B, H, N, D = K.shape
    M = Qs.shape[1]
    Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    flare.flare_pp_forward(Qs, Ks, Vs, Qf, gate, K, V, Q_out=Qo, Z=Z, L=L)
    out = flare.flare_pp_backward(Qs, Ks, Vs, Qf, gate, K, V, Qo, Z, L, dev(dY, d))
    torch.cuda.synchronize()
    return tuple(None if x is None else host(x) for x in out[:7])


PP_NAMES = ("dQs", "dKs", "dVs", "dQf", "dgate", "dK", "dV")


def compare_pp(got, ref, prefix=""):
    for n, g, r in zip(PP_NAMES, got, ref):
        if r is None:
            assert g is None, n
            continue
        assert np.all(np.isfinite(g)), n
        check(prefix + n, g, r)


@pytest.mark.parametrize("shape", [(2, 2, 3000, 64, 32, True), (2, 2, 3000, 64, 32, False),
                                   (1, 3, 1000, 48, 16, True), (2, 1, 777, 33, 32, False)],
                         ids=lambda s: "B{}H{}N{}M{}D{}shared{}".format(*s))
def test_pp_backward(flare, orc, shape):
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian_pp
    B, H, N, M, D, shared = shape
    w = make_gaussian_pp(B, H, N, M, D, "bf16", seed=111, share_vs=shared)
    dY = cotangent(112, "dy", w.K.shape)
    say(f"[pp backward] B{B} H{H} N{N} M{M} D{D} shared {shared}")
    got = gpu_pp_backward(flare, w, dY, shared)
    ref = orc.flare_pp_backward(w.Qs, w.Ks, w.Ks if shared else w.Vs, w.Qf, w.gate, w.K, w.V, dY, shared_vs=shared)
    compare_pp(got, ref)


def test_pp_backward_long_sequence_workload(flare, orc):
    # the long-sequence classification workload (B32 H4 N4096 M64 D32), whole
    from rank_latent_attention_amd.inputs import config4, cotangent
    w = config4()
    dY = cotangent(113, "dy", w.K.shape)
    say(f"[pp backward] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D}")
    got = gpu_pp_backward(flare, w, dY, True)
    ref = orc.flare_pp_backward(w.Qs, w.Ks, w.Ks, w.Qf, w.gate, w.K, w.V, dY, shared_vs=True)
    compare_pp(got, ref)


def test_pp_million_token_backward_one_head(flare, orc):
    # the million-point FLARE++ workload launched whole; one head checked in
    # full (dQs, dQf, dgate and dZ-like reductions run over all 2^20 tokens)
    from rank_latent_attention_amd.inputs import config5, cotangent
    w = config5(True)
    dY = cotangent(114, "dy", w.K.shape)
    say(f"[c5pp backward] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D}")
    got = gpu_pp_backward(flare, w, dY, True)
    h = 6
    sl = slice(h, h + 1)
    ref = orc.flare_pp_backward(w.Qs[sl], w.Ks[:, sl], w.Ks[:, sl], w.Qf[sl], w.gate[sl], w.K[:, sl], w.V[:, sl],
                                dY[:, sl], shared_vs=True)
    heads = (got[0][sl], got[1][:, sl], None, got[3][sl], got[4][sl], got[5][:, sl], got[6][:, sl])
    compare_pp(heads, ref, prefix=f"head {h} ")


def _spread_inputs(seed, N=700, M=40, D=32):
    """Two heads.  Head 0: four latent queries are 3 x a token's sign key, the
    others zero; with scale 1/log2(e) its log2 scores are exact integers up to
    96, so the latents' log-normalisers spread by more than 64 (log2) and
    the row pass leaves that head to its exact-weight kernel.  Head 1:
    ordinary Gaussian inputs (the factored kernel).  Every input is exact in
    bf16."""
    rng = np.random.default_rng(seed)
    K = np.empty((1, 2, N, D), np.float32)
    K[0, 0] = rng.integers(0, 2, size=(N, D)) * 2 - 1
    K[0, 1] = np.round(rng.standard_normal((N, D)) * 8) / 8
    V = (np.round(rng.standard_normal((1, 2, N, D)) * 8) / 8).astype(np.float32)
    Q = np.zeros((2, M, D), np.float32)
    pick = rng.choice(N, size=4, replace=False)
    Q[0, :4] = 3 * K[0, 0, pick]
    Q[1] = np.round(rng.standard_normal((M, D)) * 2) / 16
    return Q, K, V


def test_backward_wide_log_normaliser_spread(flare, orc):
    import math
    from rank_latent_attention_amd.inputs import cotangent
    Q, K, V = _spread_inputs(121)
    dY = cotangent(122, "dy", K.shape)
    scale = 1.0 / math.log2(math.e)
    _, _, L = orc.flare_forward(Q, K, V, scale)
    spread = (L.max(axis=-1) - L.min(axis=-1)) / math.log(2)
    say(f"[backward spread] log2 spread of L per head {spread.ravel()}")
    assert spread[0, 0] > 64 and spread[0, 1] < 64
    compare(orc, flare, Q, K, V, dY, scale=scale)


def test_encode_backward_wide_log_normaliser_spread(flare, orc):
    import math
    import torch
    from rank_latent_attention_amd.inputs import cotangent
    Q, K, V = _spread_inputs(123)
    scale = 1.0 / math.log2(math.e)
    dZ = cotangent(124, "dz", (1, 2, Q.shape[1], Q.shape[2]), "f32")
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    Z, L = flare.flare_encode(Qd, Kd, Vd, scale=scale)
    dQ, dK, dV = flare.flare_encode_backward(Qd, Kd, Vd, Z, L, dev(dZ, "f32"), None, scale=scale)
    torch.cuda.synchronize()
    ref = orc.encode_backward(Q, K, V, dZ, None, scale)
    say("[encode backward spread]")
    for n, g, r in zip(("dQ", "dK", "dV"), (host(dQ), host(dK), host(dV)), ref):
        check(n, g, r)


def test_backward_scores_beyond_the_unshifted_range(flare, orc):
    # log2 scores up to 160 (exact integers: sign keys, queries 5 x a key,
    # scale 1/log2(e)): the forward's encode and decode and the backward's
    # statistics pass overflow their unshifted weights and recompute with the
    # exact maxima, and the row pass leaves the head to its exact-weight kernel
    import math
    from rank_latent_attention_amd.inputs import cotangent
    rng = np.random.default_rng(141)
    N, M, D = 900, 36, 32
    K = (rng.integers(0, 2, size=(1, 1, N, D)) * 2 - 1).astype(np.float32)
    V = (np.round(rng.standard_normal((1, 1, N, D)) * 8) / 8).astype(np.float32)
    Q = np.zeros((1, M, D), np.float32)
    pick = rng.choice(N, size=M, replace=False)
    Q[0] = K[0, 0, pick] * rng.integers(1, 6, size=(M, 1))
    dY = cotangent(142, "dy", K.shape)
    say("[backward] log2 scores up to 160")
    compare(orc, flare, Q, K, V, dY, scale=1.0 / math.log2(math.e))


# --------------------------------------------------------------------------
# Backward through the fused input norms (flare_pp_backward_norm) against
# oracle.flare_pp_backward_normed, pinned in test_oracle_norm_backward_pins.py
# --------------------------------------------------------------------------

NORM_EPS = 1e-6


def gpu_pp_backward_norm(flare, w, dY, flags):
    """GPU fused-norm FLARE++ forward, then its backward; host gradients in the
    oracle's order (dQs, dKs, dVs or None, dQf, dgate, dK, dV, dalpha_qs,
    dalpha_ks, dalpha_k)."""
    import torch
    d = "bf16"
    Qs, Ks, Qf, K, V = dev(w.Qs, d), dev(w.Ks, d), dev(w.Qf, d), dev(w.K, d), dev(w.V, d)
    Vs = Ks if w.Vs is w.Ks else dev(w.Vs, d)
    gate = dev(w.gate, "f32")

    def a(x, bit):
        return dev(x, "f32") if x is not None and flags & bit else None
    aqs, aks, ak = a(w.alpha_qs, 1), a(w.alpha_ks, 2), a(w.alpha_k, 8)
    B, H, N, D = K.shape
    M = Qs.shape[1]
    Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    flare.flare_pp_forward_norm(Qs, Ks, Vs, Qf, gate, K, V, flags, aqs, aks, ak, eps=NORM_EPS, Q_out=Qo, Z=Z, L=L)
    out = flare.flare_pp_backward_norm(Qs, Ks, Vs, Qf, gate, K, V, Qo, Z, L, dev(dY, d), flags, aqs, aks, ak,
                                       eps=NORM_EPS)
    torch.cuda.synchronize()
    return tuple(None if x is None else host(x) for x in out[:10])


def oracle_pp_backward_norm(orc, w, dY, flags):
    f = dict(norm_qs=bool(flags & 1), norm_ks=bool(flags & 2), norm_qf=bool(flags & 4), norm_k=bool(flags & 8),
             alpha_qs=w.alpha_qs if flags & 1 else None, alpha_ks=w.alpha_ks if flags & 2 else None,
             alpha_k=w.alpha_k if flags & 8 else None, eps=NORM_EPS)
    return orc.flare_pp_backward_normed(w.Qs, w.Ks, w.Vs, w.Qf, w.gate, w.K, w.V, dY, **f)


PPN_NAMES = PP_NAMES + ("dalpha_qs", "dalpha_ks", "dalpha_k")


@pytest.mark.parametrize("variant,B,H,N,M,D", [
    ("flarepp", 2, 2, 1500, 64, 32), ("flarepp", 1, 3, 777, 33, 16),
    ("simplified", 2, 2, 1000, 64, 32), ("simplified", 1, 2, 700, 48, 16),
])
def test_pp_backward_norm(flare, orc, variant, B, H, N, M, D):
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian_pp_raw
    w = make_gaussian_pp_raw(B, H, N, M, D, "bf16", seed=121, variant=variant)
    dY = cotangent(122, "dy", w.K.shape)
    flags = w.norm_flags
    say(f"[pp backward, norms {flags}] {variant} B{B} H{H} N{N} M{M} D{D}")
    got = gpu_pp_backward_norm(flare, w, dY, flags)
    ref = oracle_pp_backward_norm(orc, w, dY, flags)
    for n, g, r in zip(PPN_NAMES, got, ref):
        if r is None:
            assert g is None, n
            continue
        assert np.all(np.isfinite(g)), n
        check(n, g, r)


def test_pp_backward_norm_flags_zero_is_pp_backward(flare):
    # norm_flags = 0 makes the call flare_pp_backward, bit for bit
    import torch
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian_pp
    w = make_gaussian_pp(1, 2, 900, 32, 32, "bf16", seed=123, share_vs=True)
    dY = cotangent(124, "dy", w.K.shape)
    d = "bf16"
    Qs, Ks, Qf, K, V = dev(w.Qs, d), dev(w.Ks, d), dev(w.Qf, d), dev(w.K, d), dev(w.V, d)
    gate = dev(w.gate, "f32")
    B, H, N, D = K.shape
    M = Qs.shape[1]
    Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    flare.flare_pp_forward(Qs, Ks, Ks, Qf, gate, K, V, Q_out=Qo, Z=Z, L=L)
    dy = dev(dY, d)
    a = flare.flare_pp_backward(Qs, Ks, Ks, Qf, gate, K, V, Qo, Z, L, dy)
    b = flare.flare_pp_backward_norm(Qs, Ks, Ks, Qf, gate, K, V, Qo, Z, L, dy, 0)
    torch.cuda.synchronize()
    for x, y in zip(a[:7], b[:7]):
        assert (x is None) == (y is None)
        if x is not None:
            assert torch.equal(x, y)


def test_pp_norm_million_token_backward_one_head(flare, orc):
    # the million-point FLARE++ workload before its norms (flags 15), forward
    # and backward launched whole as the benchmark runs them; one head checked
    # in full against the oracle (the channel-scale cotangents sum over all
    # 2^20 tokens of that head)
    from rank_latent_attention_amd.inputs import config5_raw, cotangent
    w = config5_raw()
    dY = cotangent(115, "dy", w.K.shape)
    say(f"[c5pp norm backward] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D} flags {w.norm_flags}")
    got = gpu_pp_backward_norm(flare, w, dY, w.norm_flags)
    h = 3
    sl = slice(h, h + 1)

    def a(x):
        return None if x is None else x[sl]
    Ks = w.Ks[:, sl]
    ref = orc.flare_pp_backward_normed(w.Qs[sl], Ks, Ks, w.Qf[sl], w.gate[sl], w.K[:, sl], w.V[:, sl], dY[:, sl],
                                       norm_qs=True, norm_ks=True, norm_qf=True, norm_k=True, alpha_qs=a(w.alpha_qs),
                                       alpha_ks=None, alpha_k=a(w.alpha_k), eps=NORM_EPS)
    heads = (got[0][sl], got[1][:, sl], None, got[3][sl], got[4][sl], got[5][:, sl], got[6][:, sl], got[7][sl],
             None, got[9][sl])
    for n, g, r in zip(PPN_NAMES, heads, ref):
        if r is None:
            assert g is None, n
            continue
        assert np.all(np.isfinite(g)), n
        check(f"head {h} {n}", g, r)


@pytest.mark.parametrize("seed", range(6))
def test_backward_random_shapes(flare, orc, seed):
    # seeded random shapes: ragged token counts, latent counts off the 32-grid,
    # both widths, shared and per-batch queries
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    rng = np.random.default_rng(300 + seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    N, M, D = int(rng.integers(1, 2500)), int(rng.integers(1, 257)), int(rng.choice([16, 32]))
    qb = bool(rng.integers(0, 2))
    w = make_gaussian(B, H, N, M, D, "bf16", seed=310 + seed)
    Q = np.broadcast_to(w.Q, (B,) + w.Q.shape).copy() if qb else w.Q
    dY = cotangent(320 + seed, "dy", w.K.shape)
    say(f"[backward random] B{B} H{H} N{N} M{M} D{D} q_batched {qb}")
    compare(orc, flare, Q, w.K, w.V, dY)


def test_pp_backward_norm_without_tokens(flare):
    # N = 0: the synthesised queries are 0, so the routing queries are N_0(Qf),
    # Z = 0 and L = -inf; every cotangent, the channel scales' included, is 0
    import torch
    B, H, M, D = 2, 2, 40, 32
    dev_ = "cuda:0"
    Qs = torch.randn(H, M, D, device=dev_).to(torch.bfloat16)
    Qf = torch.randn(H, M, D, device=dev_).to(torch.bfloat16)
    K = torch.empty((B, H, 0, D), dtype=torch.bfloat16, device=dev_)
    gate = torch.full((H,), 0.5, device=dev_)
    aqs = 1.0 + 0.1 * torch.randn(H, D, device=dev_)
    ak = 1.0 + 0.1 * torch.randn(H, D, device=dev_)
    Qo = torch.empty((B, H, M, D), device=dev_)
    Z = torch.empty((B, H, M, D), device=dev_)
    L = torch.empty((B, H, M), device=dev_)
    flare.flare_pp_forward_norm(Qs, K, K, Qf, gate, K, K, 15, aqs, None, ak, eps=NORM_EPS, Q_out=Qo, Z=Z, L=L)
    out = flare.flare_pp_backward_norm(Qs, K, K, Qf, gate, K, K, Qo, Z, L, K, 15, aqs, None, ak, eps=NORM_EPS)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(L)) and torch.count_nonzero(Z).item() == 0
    dQs, dKs, dVs, dQf, dgate, dK, dV, da_qs, da_ks, da_k, _ = out
    assert dVs is None and da_ks is None
    for t in (dQs, dQf, dgate, da_qs, da_k):
        assert torch.all(torch.isfinite(t)) and torch.count_nonzero(t).item() == 0
    assert dKs.numel() == 0 and dK.numel() == 0 and dV.numel() == 0


def _random_backward_shapes(seed, count):
    """Seeded shapes (B, H, N, M, D, q_batched, scale) for the FLARE backward:
    token counts from 2 to 40,000, any M up to 256, both head sizes, shared
    and per-batch queries, the default scale or an explicit one up to 1.2
    times it; B H N M stays under 6e6 so that the oracle ends in seconds."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 9))
        M = int(rng.choice([int(rng.integers(1, 257)), 64, 128, 256]))
        D = int(rng.choice([16, 32]))
        N = int(rng.integers(2, 40001))
        N = max(2, min(N, 6_000_000 // (B * H * M)))
        scale = float(rng.choice([0.0, 0.0, 0.11, 0.3]))
        out.append((B, H, N, M, D, bool(rng.integers(0, 2)), scale))
    return out


@pytest.mark.parametrize("shape", _random_backward_shapes(404, 8),
                         ids=lambda s: "B{}H{}N{}M{}D{}qb{}s{}".format(*s))
def test_random_backward_shapes(flare, orc, shape):
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian
    B, H, N, M, D, qb, scale = shape
    w = make_gaussian(B, H, N, M, D, "bf16", seed=N + M)
    Q = np.broadcast_to(w.Q, (B,) + w.Q.shape).copy() if qb else w.Q
    dY = cotangent(N + M + 1, "dy", w.K.shape)
    say(f"[backward, random] B{B} H{H} N{N} M{M} D{D} q_batched {qb} scale {scale}")
    compare(orc, flare, Q, w.K, w.V, dY, scale=scale)


def _random_pp_backward_shapes(seed, count):
    """Seeded FLARE++ backward shapes (B, H, N, M, D, shared values)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        M = int(rng.choice([int(rng.integers(1, 257)), 64, 128]))
        D = int(rng.choice([16, 32]))
        N = max(2, min(int(rng.integers(2, 30001)), 3_000_000 // (B * H * M)))
        out.append((B, H, N, M, D, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("shape", _random_pp_backward_shapes(7, 6),
                         ids=lambda s: "B{}H{}N{}M{}D{}shared{}".format(*s))
def test_random_pp_backward_shapes(flare, orc, shape):
    """The FLARE++ backward at seeded shapes.  Every gradient but the gate's
    meets the bf16 bar as a rel-L2.  The gate's, dg_h = sum over b, m, d of
    dQ * Qd, is one sum per head of terms of both signs, so its relative error
    is the error of dQ amplified by cancellation: it is bounded against the
    sum of the terms' magnitudes instead (computed from the oracle's routing
    cotangent and synthesis latents)."""
    from rank_latent_attention_amd.inputs import cotangent, make_gaussian_pp
    B, H, N, M, D, shared = shape
    w = make_gaussian_pp(B, H, N, M, D, "bf16", seed=N + M, share_vs=shared)
    dY = cotangent(N + M + 2, "dy", w.K.shape)
    say(f"[pp backward, random] B{B} H{H} N{N} M{M} D{D} shared {shared}")
    got = gpu_pp_backward(flare, w, dY, shared)
    Vs = w.Ks if shared else w.Vs
    ref = orc.flare_pp_backward(w.Qs, w.Ks, Vs, w.Qf, w.gate, w.K, w.V, dY, shared_vs=shared)
    for n, g, r in zip(PP_NAMES, got, ref):
        if r is None:
            assert g is None, n
            continue
        assert np.all(np.isfinite(g)), n
        if n != "dgate":
            check(n, g, r)
    Qb = orc.pp_queries(w.Qs, w.Ks, Vs, w.Qf, w.gate)
    Qd = (Qb - np.asarray(w.Qf, np.float64)[None]) / np.asarray(w.gate, np.float64)[None, :, None, None]
    dQ = orc.flare_backward(Qb, w.K, w.V, dY)[0]
    mass = np.abs(dQ * Qd).sum(axis=(0, 2, 3))  # per head
    e = np.abs(np.asarray(got[4], np.float64) - np.asarray(ref[4], np.float64)) / mass
    say(f"  dgate: error / sum |dQ Qd| up to {e.max():.2e} (bar {TOL['bf16']:g}); "
        f"conditioning sum |terms| / |sum| up to {np.max(mass / np.abs(ref[4])):.1f}")
    assert np.all(e <= TOL["bf16"]), e
