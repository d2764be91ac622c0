"""GPU parity of the fused-projection forwards (flare_forward_proj,
flare_pp_forward_proj in include/flare.h) against the fp64 oracle: the per-head
projections K = X W_K, V = X W_V (FLARE++ paper, Sec. 3.1) are formed inside
the encode from the block input X, so the oracle projects X in fp64 and runs
the FLARE / FLARE++ pair.  The bars are those of bf16 inputs with float32
accumulation; the projected keys and values are rounded to bf16 inside, as
stored inputs are."""
import math
import sys

import numpy as np
import pytest

from helpers import ROW_FACTOR, TOL, dev, host, lse_err, rel_l2, row_err

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
    e, r = rel_l2(got, ref), row_err(got, ref)
    say(f"  {name}: rel-L2 {e:.3e} (bar {tol:g}), worst row {r:.3e} (bar {ROW_FACTOR * tol:g})")
    assert e <= tol and r <= ROW_FACTOR * tol


def check_lse(name, got, ref, tol=TOL["bf16"]):
    e = lse_err(got, ref)
    say(f"  {name}: RMS relative error of e^L {e:.3e} (bar {tol:g})")
    assert e <= tol


def run_proj(flare, w, Q=None):
    import torch
    X, WK, WV = dev(w.X, "bf16"), dev(w.WK, "bf16"), dev(w.WV, "bf16")
    Qd = dev(w.Q if Q is None else Q, "bf16")
    B, N, C = X.shape
    H, _, D = WK.shape
    M = Qd.shape[-2]
    Kt = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=X.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=X.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=X.device)
    Y, _, _, _ = flare.flare_forward_proj(X, WK, WV, Qd, K_out=Kt, Z=Z, L=L)
    torch.cuda.synchronize()
    return host(Y), host(Kt), host(Z), host(L)


def run_pp_proj(flare, w, flags):
    import torch
    X, WKs, WK, WV = (dev(a, "bf16") for a in (w.X, w.WKs, w.WK, w.WV))
    Qs, Qf = dev(w.Qs, "bf16"), dev(w.Qf, "bf16")
    gate = dev(w.gate, "f32")
    aqs = dev(w.alpha_qs, "f32") if flags & 1 else None
    ak = dev(w.alpha_k, "f32") if flags & 8 else None
    B, N, C = X.shape
    H, _, D = WK.shape
    M = Qs.shape[1]
    Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=X.device)
    Kt = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=X.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=X.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=X.device)
    Y, _, _, _, _ = flare.flare_pp_forward_proj(X, WKs, WK, WV, Qs, Qf, gate, flags, aqs, ak, Q_out=Qo, K_out=Kt,
                                                Z=Z, L=L)
    torch.cuda.synchronize()
    return host(Y), host(Qo), host(Kt), host(Z), host(L)


# B, H, N, M: ragged token counts, every workgroup shape of the encode plan
# (M = 16: 4 token lanes; 33, 64: 2; 128: 1; 256: 8 waves), one token
PROJ_SHAPES = [(1, 1, 1, 1), (1, 2, 100, 16), (2, 2, 777, 64), (1, 3, 1500, 33), (2, 1, 3000, 128),
               (1, 2, 5000, 256), (1, 1, 20000, 256)]


@pytest.mark.parametrize("shape", PROJ_SHAPES, ids=lambda s: "B{}H{}N{}M{}".format(*s))
def test_proj_shapes(flare, orc, shape):
    from rank_latent_attention_amd.inputs import make_gaussian_proj, round_bf16
    B, H, N, M = shape
    w = make_gaussian_proj(B, H, N, M, 32, seed=sum(shape))
    say(f"[proj] B{B} H{H} N{N} M{M} D32 C128")
    Y, Kt, Z, L = run_proj(flare, w)
    Yr, Zr, Lr = orc.flare_forward_proj(w.X, w.WK, w.WV, w.Q)
    check("K (projected, bf16)", Kt, round_bf16(orc.project(w.X, w.WK)))
    check("Z", Z, Zr)
    check_lse("L", L, Lr)
    check("Y", Y, Yr)


def test_proj_batched_queries(flare, orc):
    from rank_latent_attention_amd.inputs import make_gaussian_proj, to_dtype
    w = make_gaussian_proj(2, 3, 1200, 96, 32, seed=51)
    Qb = to_dtype(np.random.default_rng(52).standard_normal((2, 3, 96, 32)) / math.sqrt(32), "bf16")
    Y, _, Z, L = run_proj(flare, w, Q=Qb)
    Yr, Zr, Lr = orc.flare_forward_proj(w.X, w.WK, w.WV, Qb)
    check("Z", Z, Zr)
    check("Y", Y, Yr)


@pytest.mark.parametrize("flags", [15, 0])
@pytest.mark.parametrize("shape", [(2, 2, 900, 64), (1, 3, 4100, 256)], ids=lambda s: "B{}H{}N{}M{}".format(*s))
def test_pp_proj(flare, orc, shape, flags):
    from rank_latent_attention_amd.inputs import make_gaussian_proj
    B, H, N, M = shape
    w = make_gaussian_proj(B, H, N, M, 32, seed=sum(shape) + flags, pp=True)
    say(f"[pp proj] B{B} H{H} N{N} M{M} flags {flags}")
    Y, Qo, Kt, Z, L = run_pp_proj(flare, w, flags)
    f = flags
    Yr, Qr, Zr, Lr = orc.flare_pp_forward_proj(w.X, w.WKs, w.WK, w.WV, w.Qs, w.Qf, w.gate, norm_qs=bool(f & 1),
                                               norm_ks=bool(f & 2), norm_qf=bool(f & 4), norm_k=bool(f & 8),
                                               alpha_qs=w.alpha_qs if f & 1 else None,
                                               alpha_k=w.alpha_k if f & 8 else None)
    check("Q", Qo, Qr)
    check("Z", Z, Zr)
    check_lse("L", L, Lr)
    check("Y", Y, Yr)


@pytest.mark.parametrize("mult", [6.0, 40.0])
def test_proj_large_scores(flare, orc, mult):
    """Queries scaled up: the rounded queries fail the exactness bound (x6,
    largest log2 score about 20) or the weights leave the float range (x40);
    the workgroups project their tiles again and redo the scores exactly."""
    from rank_latent_attention_amd.inputs import make_gaussian_proj, to_dtype
    w = make_gaussian_proj(1, 2, 3000, 64, 32, seed=53)
    w.Q = to_dtype(w.Q.astype(np.float64) * mult, "bf16")
    say(f"[proj large scores] x{mult:g}")
    Y, _, Z, L = run_proj(flare, w)
    Yr, Zr, Lr = orc.flare_forward_proj(w.X, w.WK, w.WV, w.Q)
    check("Z", Z, Zr)
    check_lse("L", L, Lr)
    check("Y", Y, Yr)


def test_proj_million_tokens_sampled(flare, orc):
    """The million-point surface mesh from its block input, launched whole;
    heads 0 and 7 checked in full for Z and K, and on sampled tokens (both
    sides of every 8192-token seam) for Y."""
    from rank_latent_attention_amd.inputs import config5_proj, round_bf16
    w = config5_proj()
    say(f"[c5 proj] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D} C{w.X.shape[-1]} (full launch, sampled check)")
    Y, Kt, Z, L = run_proj(flare, w)
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(Z)) and np.all(np.isfinite(L))
    rng = np.random.default_rng(54)
    seams = np.arange(0, w.N + 1, 8192)
    idx = np.concatenate([seams - 1, seams, rng.choice(w.N, 1024, replace=False)])
    idx = np.unique(idx[(idx >= 0) & (idx < w.N)])
    for h in (0, 7):
        K = orc.project(w.X, w.WK[h:h + 1])
        V = orc.project(w.X, w.WV[h:h + 1])
        check(f"head {h} K", Kt[:, h:h + 1], round_bf16(K))
        Zr, Lr = orc.encode(w.Q[h:h + 1], K, V)
        check(f"head {h} Z", Z[:, h:h + 1], Zr)
        check_lse(f"head {h} L", L[:, h:h + 1], Lr)
        Yr = orc.decode(w.Q[h:h + 1], K, Zr, idx=idx)
        check(f"head {h} Y[{idx.size} tokens]", Y[:, h:h + 1][:, :, idx], Yr)
