"""GPU parity of the fused FLARE++ input normalisations.

flare_pp_forward_norm (through the C ABI) against the fp64 oracle's
flare_pp_forward_normed: per-head RMS norms N_0 / N_a of the FLARE++ paper
(App. A.3, A.4, A.6 and Table 2 in App. A.7) applied inside the kernels.
bf16 inputs, rel-L2 bar 1e-2 on Y, the routing queries, Z and L.
"""
import math
import sys

import numpy as np
import pytest

from helpers import TOL, dev, host, lse_err, rel_l2

pytestmark = pytest.mark.gpu

EPS = 1e-6


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


def run_norm(flare, w, flags, scale=0.0):
    import torch
    d = w.dtype
    Qs, Ks, Qf, K, V = dev(w.Qs, d), dev(w.Ks, d), dev(w.Qf, d), dev(w.K, d), dev(w.V, d)
    Vs = Ks if w.Vs is w.Ks else dev(w.Vs, d)
    gate = dev(w.gate, "f32")

    def a(x):
        return None if x is None else dev(x, "f32")

    B, H, N, D = K.shape
    M = Qs.shape[1]
    Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    Y, _, _, _ = flare.flare_pp_forward_norm(Qs, Ks, Vs, Qf, gate, K, V, flags, a(w.alpha_qs), a(w.alpha_ks),
                                             a(w.alpha_k), eps=EPS, scale=scale, Q_out=Qo, Z=Z, L=L)
    torch.cuda.synchronize()
    return host(Y), host(Qo), host(Z), host(L)


def oracle_norm(orc, w, flags, scale=0.0):
    return orc.flare_pp_forward_normed(
        w.Qs, w.Ks, w.Vs, w.Qf, w.gate, w.K, w.V, norm_qs=bool(flags & 1), norm_ks=bool(flags & 2),
        norm_qf=bool(flags & 4), norm_k=bool(flags & 8), alpha_qs=w.alpha_qs if flags & 1 else None,
        alpha_ks=w.alpha_ks if flags & 2 else None, alpha_k=w.alpha_k if flags & 8 else None, eps=EPS, scale=scale)


def check(name, got, ref, tol):
    e = rel_l2(got, ref)
    say(f"  {name}: rel-L2 {e:.3e} (bar {tol:g})")
    assert e <= tol, f"{name}: rel-L2 {e:.3e} > {tol:g}"


def check_lse(name, got, ref, tol):
    e = lse_err(got, ref)
    say(f"  {name}: RMS relative error of e^L {e:.3e} (bar {tol:g})")
    assert e <= tol, f"{name}: RMS relative error of e^L {e:.3e} > {tol:g}"


def compare(orc, flare, w, flags, scale=0.0, tol=TOL["bf16"]):
    Y, Q, Z, L = run_norm(flare, w, flags, scale)
    Yr, Qr, Zr, Lr = oracle_norm(orc, w, flags, scale)
    for n, g, r in (("Y", Y, Yr), ("Q", Q, Qr), ("Z", Z, Zr)):
        assert np.all(np.isfinite(g)), n
        check(n, g, r, tol)
    check_lse("L", L, Lr, tol)


# FLARE++ (shared synthesis keys and values, all four norms) and the
# simplified variant (separate values, norms on the seeds and keys only),
# at the long-sequence shape, ragged token counts and latent tails, both widths
SHAPES = [  # variant, B, H, N, M, D
    ("flarepp", 2, 4, 4096, 64, 32), ("flarepp", 1, 2, 3001, 48, 16), ("flarepp", 1, 1, 20000, 256, 32),
    ("simplified", 2, 2, 1000, 256, 32), ("simplified", 1, 3, 777, 33, 16), ("flarepp", 1, 1, 5, 3, 16),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "{}-B{}H{}N{}M{}D{}".format(*s))
def test_norm_variants(flare, orc, shape):
    from rank_latent_attention_amd.inputs import make_gaussian_pp_raw
    variant, B, H, N, M, D = shape
    w = make_gaussian_pp_raw(B, H, N, M, D, "bf16", seed=71, variant=variant)
    say(f"[norm {variant}] B{B} H{H} N{N} M{M} D{D} flags {w.norm_flags}")
    compare(orc, flare, w, w.norm_flags)


@pytest.mark.parametrize("flags", [1, 2, 4, 8, 6, 9])
def test_norm_flags_one_at_a_time(flare, orc, flags):
    from rank_latent_attention_amd.inputs import make_gaussian_pp_raw
    w = make_gaussian_pp_raw(1, 2, 1500, 64, 32, "bf16", seed=72)
    say(f"[norm flags {flags}]")
    compare(orc, flare, w, flags)


@pytest.mark.parametrize("flags", [8, 12])
@pytest.mark.parametrize("scale", [0.0, 0.3])
def test_normalised_routing_keys_at_a_sharper_scale(flare, orc, flags, scale):
    """N_0 routing keys (with and without N_0 on the fixed queries) at the
    default scale and at 1.2 times it (D = 16): the keys normalised on the fly
    and the queries they meet are rounded to fp16 for the score products, so
    the rounding of the normalised keys moves no score by more than 2^-11 of
    its terms.  With bf16 operands this shape reached rel-L2 1.1e-2 on Y at
    the sharper scale."""
    from rank_latent_attention_amd.inputs import make_gaussian_pp_raw
    w = make_gaussian_pp_raw(2, 7, 13392, 64, 16, "bf16", seed=2130, variant="flarepp")
    say(f"[norm flags {flags}, scale {scale}]")
    compare(orc, flare, w, flags, scale=scale)


def test_scaled_shared_keys_scale_the_latents(flare, orc):
    # N_a on keys that are also the values (App. A.6 with a learned scale):
    # the scale multiplies both the scores and the merged synthesis latents
    from rank_latent_attention_amd.inputs import channel_scales, make_gaussian_pp_raw
    w = make_gaussian_pp_raw(2, 3, 2000, 64, 32, "bf16", seed=73)
    w.alpha_ks = channel_scales(74, "alpha_ks", 3, 32)
    compare(orc, flare, w, 15)


def test_zero_flags_equal_the_plain_entry_point(flare):
    import torch
    from rank_latent_attention_amd.inputs import make_gaussian_pp_raw
    w = make_gaussian_pp_raw(1, 2, 3000, 64, 32, "bf16", seed=75)
    d = "bf16"
    Qs, Ks, Qf, K, V = dev(w.Qs, d), dev(w.Ks, d), dev(w.Qf, d), dev(w.K, d), dev(w.V, d)
    gate = dev(w.gate, "f32")
    Y1, _, _, _ = flare.flare_pp_forward(Qs, Ks, Ks, Qf, gate, K, V)
    Y2, _, _, _ = flare.flare_pp_forward_norm(Qs, Ks, Ks, Qf, gate, K, V, 0)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)


def _exact_inputs(B, H, N, M, D, seed):
    """Inputs that stay exact through every rounding of the path.  Every row
    that is normalised is a sign pattern times a power of two, so its N_0 row
    is the sign pattern itself (bf16-exact) while the row factors differ;
    values are multiples of 1/4; gate 1/2.  The synthesised queries are then
    sign rows and the routing queries N_0(Qf) + Qd / 2 lie in {+-1/2, +-3/2},
    so every score is exact in bf16 products and float32 sums."""
    from rank_latent_attention_amd.inputs import make_gaussian_pp_raw
    rng = np.random.default_rng(seed)
    w = make_gaussian_pp_raw(B, H, N, M, D, "bf16", seed=seed)

    def signs(shape, lo, hi):
        mag = np.exp2(rng.integers(lo, hi, size=shape[:-1] + (1,)))
        return ((rng.integers(0, 2, size=shape) * 2 - 1) * mag).astype(np.float32)

    w.Ks = signs((B, H, N, D), -1, 3)
    w.Vs = w.Ks
    w.K = signs((B, H, N, D), -1, 3)
    w.Qs = signs((H, M, D), 0, 2)
    w.Qf = signs((H, M, D), 0, 2)
    # each seed row gets one key with its own sign pattern (the largest
    # possible score, far above every random key), so the synthesis softmax
    # is one-hot to well below float32 resolution and Qd is a sign row
    for h in range(H):
        pick = rng.choice(N, size=M, replace=False)
        for b in range(B):
            w.Ks[b, h, pick] = np.sign(w.Qs[h]) * np.exp2(rng.integers(-1, 3, size=(M, 1)))
    w.V = (np.round(rng.standard_normal((B, H, N, D)) * 4) / 4).astype(np.float32)
    w.alpha_qs = w.alpha_ks = w.alpha_k = None
    w.gate = np.full((H,), 0.5, np.float32)
    return w


def test_norms_on_the_careful_path(flare, orc):
    # with s log2(e) = 8 the log2 scores reach several hundred, which
    # overflows the unshifted fast path in the synthesis encode, the routing
    # encode and the decode: waves take the exact-maximum recomputation, which
    # normalises the keys (and the shared values) itself
    w = _exact_inputs(1, 2, 700, 32, 32, seed=76)
    scale = 8.0 / math.log2(math.e)
    compare(orc, flare, w, 15, scale=scale)


def test_normalised_keys_with_queries_beyond_fp16(flare, orc):
    # s log2(e) = 2^16: the scaled routing queries (+-2^15, +-3 * 2^15) lie
    # beyond the fp16 range, so the fp16 score operands of the normalised
    # keys cannot hold them: their rounding error is infinite and every unit
    # of work takes the exact recomputation (hi + lo bf16 queries).  Scores
    # reach 3 * 10^6 (log2), where any relative error of a normalised key
    # would show, so every normalised row here is a sign row (its N_0 is
    # exact) and eps = 1e-30 leaves the row factors at exactly one; the
    # scores are then exact integers on both sides
    import torch
    w = _exact_inputs(1, 2, 700, 32, 32, seed=77)
    for name in ("Qs", "Ks", "K", "Qf"):
        setattr(w, name, np.sign(getattr(w, name)).astype(np.float32))
    w.Vs = w.Ks
    eps = 1e-30
    scale = 2.0 ** 16 / math.log2(math.e)
    d = "bf16"
    Qs, Ks, Qf, K, V = dev(w.Qs, d), dev(w.Ks, d), dev(w.Qf, d), dev(w.K, d), dev(w.V, d)
    B, H, N, D = K.shape
    M = Qs.shape[1]
    Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    Y, _, _, _ = flare.flare_pp_forward_norm(Qs, Ks, Ks, Qf, dev(w.gate, "f32"), K, V, 15, None, None, None, eps=eps,
                                            scale=scale, Q_out=Qo, Z=Z, L=L)
    torch.cuda.synchronize()
    Y, Q, Z, L = host(Y), host(Qo), host(Z), host(L)
    Yr, Qr, Zr, Lr = orc.flare_pp_forward_normed(w.Qs, w.Ks, w.Ks, w.Qf, w.gate, w.K, w.V, norm_qs=True, norm_ks=True,
                                                 norm_qf=True, norm_k=True, eps=eps, scale=scale)
    for n, g, r in (("Y", Y, Yr), ("Q", Q, Qr), ("Z", Z, Zr)):
        assert np.all(np.isfinite(g)), n
        check(n, g, r, TOL["bf16"])
    # L is of order 10^6 here: float32 holds it to about 0.1, so it is
    # compared to within a few units in its last place, not through e^L
    dL = np.abs(np.asarray(L, np.float64) - Lr)
    say(f"  L: largest |L - L_oracle| {dL.max():.3g} at |L| up to {np.abs(Lr).max():.3g}")
    assert np.all(dL <= 4 * 2.0 ** -23 * np.abs(Lr) + 1e-3)


@pytest.mark.parametrize("N", [1024, 2048], ids=lambda n: f"N{n}")
def test_short_heads_at_extreme_scores(flare, orc, N):
    # 128 heads of M = 64 with no norms take the one-workgroup-per-head
    # kernel (N 1024) or the per-latent-block kernel (N 2048); s log2(e) = 2^6
    # makes every unshifted weight overflow, so their encodes and decode must
    # all take the exact recomputation.  Scores are exact dyadic sums.
    w = _exact_inputs(32, 4, N, 64, 32, seed=78)
    scale = 2.0 ** 6 / math.log2(math.e)
    Y, Q, Z, L = run_norm(flare, w, 0, scale)
    Yr, Qr, Zr, Lr = oracle_norm(orc, w, 0, scale)
    for n, g, r in (("Y", Y, Yr), ("Q", Q, Qr), ("Z", Z, Zr)):
        assert np.all(np.isfinite(g)), n
        check(n, g, r, TOL["bf16"])
    # Without norms the routing queries are blends of tied synthesis keys,
    # not all bf16-exact: where the exact-score bound holds, a unit keeps its
    # fast scores, each within 2^-5 (log2) of the exact one, and L, set by the
    # largest scores, inherits up to that (ln 2 / 32 = 0.022), plus float32
    # rounding of L (of order 10^4 here)
    dL = np.abs(np.asarray(L, np.float64) - Lr)
    say(f"  L: largest |L - L_oracle| {dL.max():.3g} at |L| up to {np.abs(Lr).max():.3g}")
    assert np.all(dL <= math.log(2) / 32 + 8 * 2.0 ** -23 * np.abs(Lr) + 1e-3)


def test_million_token_raw_workload_sampled(flare, orc):
    # the million-point FLARE++ workload before its norms, launched whole and
    # checked on the routing queries, Z and L of two heads and on sampled rows of Y
    from rank_latent_attention_amd.inputs import config5_raw
    w = config5_raw()
    say(f"[c5 raw] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D} flags {w.norm_flags}")
    Y, Q, Z, L = run_norm(flare, w, w.norm_flags)
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(Z)) and np.all(np.isfinite(L))
    rng = np.random.default_rng(12)
    idx = np.unique(np.concatenate([[0, 1, w.N // 2, w.N - 1], rng.choice(w.N, size=2048, replace=False)]))
    tol = TOL["bf16"]
    for h in (0, 5):
        sl = slice(h, h + 1)
        Qs = orc.rms_norm(w.Qs[sl], w.alpha_qs[sl], EPS)
        Ks = orc.rms_norm(w.Ks[:, sl], None, EPS)
        Qf = orc.rms_norm(w.Qf[sl], None, EPS)
        K = orc.rms_norm(w.K[:, sl], w.alpha_k[sl], EPS)
        Qb = orc.pp_queries(Qs, Ks, Ks, Qf, w.gate[sl])
        check(f"head {h} Q", Q[:, sl], Qb, tol)
        Zr, Lr = orc.encode(Qb, K, w.V[:, sl])
        check(f"head {h} Z", Z[:, sl], Zr, tol)
        check_lse(f"head {h} L", L[:, sl], Lr, tol)
        Yr = orc.decode(Qb, K, Zr, idx=idx)
        check(f"head {h} Y[{idx.size} tokens]", Y[:, sl][:, :, idx], Yr, tol)


def test_million_token_simplified_workload_sampled(flare, orc):
    # the simplified FLARE++ bench workload (N_a on the seeds and synthesis
    # keys, separate synthesis values, no blend), launched whole and checked
    # on the routing queries, Z and L of two heads and on sampled rows of Y
    from rank_latent_attention_amd.inputs import config5_simplified
    w = config5_simplified()
    say(f"[c5 simplified] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D} flags {w.norm_flags}")
    Y, Q, Z, L = run_norm(flare, w, w.norm_flags)
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(Z)) and np.all(np.isfinite(L))
    rng = np.random.default_rng(13)
    idx = np.unique(np.concatenate([[0, 1, w.N // 2, w.N - 1], rng.choice(w.N, size=2048, replace=False)]))
    tol = TOL["bf16"]
    for h in (1, 6):
        sl = slice(h, h + 1)
        Qs = orc.rms_norm(w.Qs[sl], w.alpha_qs[sl], EPS)
        Ks = orc.rms_norm(w.Ks[:, sl], w.alpha_ks[sl], EPS)
        Qb = orc.pp_queries(Qs, Ks, w.Vs[:, sl], w.Qf[sl], w.gate[sl])
        check(f"head {h} Q", Q[:, sl], Qb, tol)
        Zr, Lr = orc.encode(Qb, w.K[:, sl], w.V[:, sl])
        check(f"head {h} Z", Z[:, sl], Zr, tol)
        check_lse(f"head {h} L", L[:, sl], Lr, tol)
        Yr = orc.decode(Qb, w.K[:, sl], Zr, idx=idx)
        check(f"head {h} Y[{idx.size} tokens]", Y[:, sl][:, :, idx], Yr, tol)
