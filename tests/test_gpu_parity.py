"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case draws seeded inputs from rank_latent_attention_amd.inputs, runs the
same arrays through both sides and compares element by element with the
rel-L2 bars: 1e-5 for float32 inputs, 1e-2 for bf16 inputs with float32
accumulation.  The million-token workload is launched exactly as the
benchmark launches it and checked on whole heads of Z and on sampled token
rows of Y, which the oracle computes one by one.
"""
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


def run_flare(flare, w, scale=0.0):
    import torch
    Q, K, V = dev(w.Q, w.dtype), dev(w.K, w.dtype), dev(w.V, w.dtype)
    B, H, N, D = K.shape
    M = Q.shape[-2]
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    Y, _, _ = flare.flare_forward(Q, K, V, scale=scale, Z=Z, L=L)
    torch.cuda.synchronize()
    return host(Y), host(Z), host(L)


def run_pp(flare, w, scale=0.0, alias=True):
    import torch
    d = w.dtype
    Qs, Ks, Qf, K, V = dev(w.Qs, d), dev(w.Ks, d), dev(w.Qf, d), dev(w.K, d), dev(w.V, d)
    Vs = Ks if (alias and w.Vs is w.Ks) else dev(w.Vs, d)
    gate = dev(w.gate, "f32")
    B, H, N, D = K.shape
    M = Qs.shape[1]
    Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    Y, _, _, _ = flare.flare_pp_forward(Qs, Ks, Vs, Qf, gate, K, V, scale=scale, Q_out=Qo, Z=Z, L=L)
    torch.cuda.synchronize()
    return host(Y), host(Qo), host(Z), host(L)


def check(name, got, ref, tol):
    """rel-L2 over the whole tensor within tol, and every row (last axis)
    within ROW_FACTOR * tol of its own norm (see helpers.row_err)."""
    e = rel_l2(got, ref)
    r = row_err(got, ref)
    say(f"  {name}: rel-L2 {e:.3e} (bar {tol:g}), worst row {r:.3e} (bar {ROW_FACTOR * tol:g})")
    assert e <= tol, f"{name}: rel-L2 {e:.3e} > {tol:g}"
    assert r <= ROW_FACTOR * tol, f"{name}: worst row error {r:.3e} > {ROW_FACTOR * tol:g}"


def check_lse(name, got, ref, tol):
    e = lse_err(got, ref)
    say(f"  {name}: RMS relative error of e^L {e:.3e} (bar {tol:g})")
    assert e <= tol, f"{name}: RMS relative error of e^L {e:.3e} > {tol:g}"


# --------------------------------------------------------------------------
# The five workloads (the million-token one is sampled, below)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", ["c1", "c2f", "c2b", "c3a", "c3b"])
def test_config_flare(flare, orc, cfg):
    from rank_latent_attention_amd.inputs import CONFIGS
    w = CONFIGS[cfg]()
    say(f"[{cfg}] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D} {w.dtype}")
    Y, Z, L = run_flare(flare, w)
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    tol = TOL[w.dtype]
    check("Z", Z, Zr, tol)
    check_lse("L", L, Lr, tol)
    check("Y", Y, Yr, tol)


def test_config4_flare_pp(flare, orc):
    from rank_latent_attention_amd.inputs import config4
    w = config4()
    say(f"[c4] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D} {w.dtype}")
    Y, Qo, Z, L = run_pp(flare, w)
    Yr, Qr, Zr, Lr = orc.flare_pp_forward(w.Qs, w.Ks, w.Vs, w.Qf, w.gate, w.K, w.V)
    tol = TOL[w.dtype]
    check("Q", Qo, Qr, tol)
    check("Z", Z, Zr, tol)
    check_lse("L", L, Lr, tol)
    check("Y", Y, Yr, tol)


def _sample_tokens(N, seed, count=2048, seam=8192):
    """Random tokens plus the ends and both sides of every multiple of `seam`
    (the boundaries of the decode's 8192-token and the encode's 16384-token
    workgroup pieces at the million-token shape)."""
    rng = np.random.default_rng(seed)
    seams = np.arange(0, N + 1, seam)
    around = np.concatenate([seams - 2, seams - 1, seams, seams + 1])
    idx = np.concatenate([[0, 1, N // 2, N - 2, N - 1], around, rng.choice(N, size=count, replace=False)])
    return np.unique(idx[(idx >= 0) & (idx < N)])


@pytest.mark.parametrize("pp", [False, True], ids=["c5", "c5pp"])
def test_config5_million_tokens_sampled(flare, orc, pp):
    import torch
    from rank_latent_attention_amd.inputs import config5
    w = config5(pp=pp)
    say(f"[{'c5pp' if pp else 'c5'}] {w.name} B{w.B} H{w.H} N{w.N} M{w.M} D{w.D} {w.dtype} (full launch, sampled check)")
    if pp:
        Y, Qo, Z, L = run_pp(flare, w)
    else:
        Y, Z, L = run_flare(flare, w)
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(Z)) and np.all(np.isfinite(L))
    idx = _sample_tokens(w.N, 11)
    tol = TOL[w.dtype]
    for h in range(w.H):
        sl = slice(h, h + 1)
        K, V = w.K[:, sl], w.V[:, sl]
        if pp:
            Qb = orc.pp_queries(w.Qs[sl], w.Ks[:, sl], w.Vs[:, sl], w.Qf[sl], w.gate[sl])
            check(f"head {h} Q", Qo[:, sl], Qb, tol)
            Zr, Lr = orc.encode(Qb, K, V)
            Yr = orc.decode(Qb, K, Zr, idx=idx)
        else:
            Zr, Lr = orc.encode(w.Q[sl], K, V)
            Yr = orc.decode(w.Q[sl], K, Zr, idx=idx)
        check(f"head {h} Z", Z[:, sl], Zr, tol)
        check_lse(f"head {h} L", L[:, sl], Lr, tol)
        check(f"head {h} Y[{idx.size} tokens]", Y[:, sl][:, :, idx], Yr, tol)
    del torch


# --------------------------------------------------------------------------
# Shapes: ragged tails, tiny and maximal latent counts, both widths and dtypes
# --------------------------------------------------------------------------

SHAPES = [  # B, H, N, M, D
    (1, 1, 1, 1, 16), (1, 1, 5, 3, 16), (1, 2, 31, 32, 32), (2, 3, 100, 33, 32), (1, 2, 300, 65, 16),
    (1, 1, 1000, 200, 32), (2, 2, 257, 256, 16), (1, 1, 129, 96, 32), (3, 1, 4099, 128, 16),
    (1, 1, 20000, 256, 32), (1, 1, 640, 17, 16),
    # every compile-time latent block count of the bf16 decode (2, 4, 8) at both widths
    (2, 1, 1500, 64, 32), (1, 2, 777, 128, 32), (1, 1, 2050, 64, 16),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}H{}N{}M{}D{}".format(*s))
def test_shapes(flare, orc, shape, dtype):
    from rank_latent_attention_amd.inputs import make_gaussian
    B, H, N, M, D = shape
    w = make_gaussian(B, H, N, M, D, dtype, seed=sum(shape))
    say(f"[shape] {shape} {dtype}")
    Y, Z, L = run_flare(flare, w)
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    tol = TOL[dtype]
    check("Z", Z, Zr, tol)
    check_lse("L", L, Lr, tol)
    check("Y", Y, Yr, tol)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batched_queries(flare, orc, dtype):
    from rank_latent_attention_amd.inputs import make_gaussian
    w = make_gaussian(2, 3, 700, 48, 32, dtype, seed=5)
    rng = np.random.default_rng(6)
    from rank_latent_attention_amd.inputs import to_dtype
    w.Q = to_dtype(rng.standard_normal((2, 3, 48, 32)) / math.sqrt(32), dtype)
    Y, Z, L = run_flare(flare, w)
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    check("Z", Z, Zr, TOL[dtype])
    check("Y", Y, Yr, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pp_shapes_and_unshared_values(flare, orc, dtype):
    from rank_latent_attention_amd.inputs import make_gaussian_pp
    for shape, share in [((2, 2, 333, 40, 16), True), ((1, 3, 1500, 64, 32), False)]:
        w = make_gaussian_pp(*shape, dtype=dtype, seed=7, share_vs=share)
        say(f"[pp] {shape} {dtype} shared={share}")
        Y, Qo, Z, L = run_pp(flare, w)
        Yr, Qr, Zr, Lr = orc.flare_pp_forward(w.Qs, w.Ks, w.Vs, w.Qf, w.gate, w.K, w.V)
        check("Q", Qo, Qr, TOL[dtype])
        check("Z", Z, Zr, TOL[dtype])
        check("Y", Y, Yr, TOL[dtype])


def _head_batch(H, fill):
    """A batch size for the forwards that run each head in its own workgroup
    (D = 32, M = 64 or 128, bf16, short heads) once B H reaches half of the
    compute units: "half" gives B H = half of them, "more" one step of H
    past that, "all" every compute unit, and "quarter" a quarter of them (the
    launch sequence, for comparison).  FLARE++ heads of 2048 tokens or more
    at "half" with M = 64 take one workgroup per (head, latent block)
    instead."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if fill == "quarter":
        return -(-cus // (4 * H))
    if fill == "all":
        return -(-cus // H)
    if fill == "half":
        return -(-cus // (2 * H))
    return -(-cus // (2 * H)) + 1


@pytest.mark.parametrize("N,M,H,share,mult,fill", [
    (1, 64, 4, True, 1.0, "half"),        # one token per head
    (100, 64, 4, False, 1.0, "more"),     # less than one tile, unshared synthesis values
    (1000, 128, 2, True, 1.0, "half"),
    (4097, 128, 4, False, 1.0, "more"),   # one token past 16 tiles
    (8192, 64, 8, True, 1.0, "half"),     # the longest heads it takes
    (3000, 64, 4, False, 1.0, "quarter"), # below half of the compute units: the launch sequence
    (3000, 64, 4, True, 8.0, "half"),     # keys x8: exact-score redo in both encodes and the decode
    (2500, 64, 4, False, 8.0, "more"),
])
def test_pp_one_workgroup_per_head(flare, orc, N, M, H, share, mult, fill):
    from rank_latent_attention_amd.inputs import make_gaussian_pp, to_dtype
    B = _head_batch(H, fill)
    w = make_gaussian_pp(B, H, N, M, 32, dtype="bf16", seed=31 + N, share_vs=share)
    if mult != 1.0:
        w.Ks = to_dtype(w.Ks.astype(np.float64) * mult, "bf16")
        w.Vs = w.Ks if share else w.Vs
        w.K = to_dtype(w.K.astype(np.float64) * mult, "bf16")
    say(f"[pp per head] B{B} H{H} N{N} M{M} D32 bf16 shared={share} keys x{mult:g} ({fill})")
    Y, Qo, Z, L = run_pp(flare, w)
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(Z)) and np.all(np.isfinite(L))
    tol = TOL["bf16"]
    Yr, Qr, Zr, Lr = orc.flare_pp_forward(w.Qs, w.Ks, w.Vs, w.Qf, w.gate, w.K, w.V)
    check("Q", Qo, Qr, tol)
    if mult == 1.0:
        check("Z", Z, Zr, tol)
        check_lse("L", L, Lr, tol)
        check("Y", Y, Yr, tol)
    # The routing half against the oracle at the queries this call formed:
    # with scores of a hundred or more, the synthesis's bf16 rounding of the
    # queries (rel. about 1e-3) alone moves L by more than its bar.
    say("  routing from the formed queries:")
    Yq, Zq, Lq = orc.flare_forward(Qo, w.K, w.V)
    check("Z", Z, Zq, tol)
    check_lse("L", L, Lq, tol)
    check("Y", Y, Yq, tol)


@pytest.mark.parametrize("N,M,H,batched,mult,fill", [
    (1, 64, 4, False, 1.0, "half"),       # one token per head
    (100, 128, 4, True, 1.0, "more"),     # less than one tile, per-batch queries
    (4097, 64, 2, False, 1.0, "half"),    # one token past 8 tiles
    (4096, 128, 8, True, 1.0, "half"),    # the longest heads it takes below every compute unit
    (8192, 64, 4, False, 1.0, "all"),     # the longest heads it takes
    (3000, 64, 4, False, 1.0, "quarter"), # below half of the compute units: the launch sequence
    (3000, 64, 4, False, 8.0, "more"),    # queries x8: exact-score redo in the encode and the decode
])
def test_forward_one_workgroup_per_head(flare, orc, N, M, H, batched, mult, fill):
    """The FLARE forward runs each head in its own workgroup under the same
    conditions as FLARE++ (bf16, D = 32, M = 64 or 128, up to 8192 tokens,
    B H at least half the compute units).  Against the oracle, and against
    the standalone decode (which checks every block's key norms) on the
    forward's own Z: bit for bit where no block needs the exact-score redo.
    With the redo the two differ in rounding, because a redone 32-token block
    is one of the decode's pieces' blocks, and the per-head decode cuts the
    tokens into blocks from each head's start."""
    import torch
    from rank_latent_attention_amd.inputs import make_gaussian, to_dtype
    B = _head_batch(H, fill)
    w = make_gaussian(B, H, N, M, 32, "bf16", seed=57 + N)
    if batched:
        rng = np.random.default_rng(58 + N)
        w.Q = to_dtype(rng.standard_normal((B, H, M, 32)) / math.sqrt(32), "bf16")
    if mult != 1.0:
        w.Q = to_dtype(w.Q.astype(np.float64) * mult, "bf16")
    say(f"[forward per head] B{B} H{H} N{N} M{M} D32 bf16 batched={batched} queries x{mult:g} ({fill})")
    Q, K, V = dev(w.Q, "bf16"), dev(w.K, "bf16"), dev(w.V, "bf16")
    Z = torch.empty((B, H, M, 32), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    Y, _, _ = flare.flare_forward(Q, K, V, Z=Z, L=L)
    Yd = flare.flare_decode(Q, K, Z)
    torch.cuda.synchronize()
    tol = TOL["bf16"]
    if mult == 1.0:
        assert torch.equal(Y, Yd), "forward and standalone decode differ"
    else:
        check("Y against the standalone decode", host(Y), host(Yd), tol)
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    check("Z", host(Z), Zr, tol)
    check_lse("L", host(L), Lr, tol)
    check("Y", host(Y), Yr, tol)


@pytest.mark.parametrize("D,mult", [(32, 1.0), (16, 1.0), (32, 8.0)])
def test_decode_merges_the_splits(flare, orc, D, mult):
    """bf16 at M = 256 with at least 16384 (head, latent) pairs and few
    splits per head: the decode merges the encode's splits as it stages the
    latents (no merge launch), and the first workgroup of each head writes Z
    and L.  Against the oracle; Y bit for bit against the standalone decode
    on the forward's Z where no block needs the exact-score redo; and the
    FLARE++ forward, whose routing decode takes float32 queries."""
    import torch
    from rank_latent_attention_amd.inputs import make_gaussian, make_gaussian_pp, to_dtype
    w = make_gaussian(16, 4, 3000, 256, D, "bf16", seed=61 + D)
    if mult != 1.0:
        w.Q = to_dtype(w.Q.astype(np.float64) * mult, "bf16")
    say(f"[decode merges] B16 H4 N3000 M256 D{D} bf16 queries x{mult:g}")
    Q, K, V = dev(w.Q, "bf16"), dev(w.K, "bf16"), dev(w.V, "bf16")
    Z = torch.empty((16, 4, 256, D), dtype=torch.float32, device=K.device)
    L = torch.empty((16, 4, 256), dtype=torch.float32, device=K.device)
    Y, _, _ = flare.flare_forward(Q, K, V, Z=Z, L=L)
    Yd = flare.flare_decode(Q, K, Z)
    torch.cuda.synchronize()
    tol = TOL["bf16"]
    if mult == 1.0:
        assert torch.equal(Y, Yd), "forward and standalone decode differ"
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    check("Z", host(Z), Zr, tol)
    check_lse("L", host(L), Lr, tol)
    check("Y", host(Y), Yr, tol)
    if D == 32 and mult == 1.0:
        wp = make_gaussian_pp(16, 4, 3000, 256, 32, dtype="bf16", seed=63)
        Yp, Qo, Zp, Lp = run_pp(flare, wp)
        Ypr, Qpr, Zpr, Lpr = orc.flare_pp_forward(wp.Qs, wp.Ks, wp.Vs, wp.Qf, wp.gate, wp.K, wp.V)
        check("FLARE++ Q", Qo, Qpr, tol)
        check("FLARE++ Z", Zp, Zpr, tol)
        check_lse("FLARE++ L", Lp, Lpr, tol)
        check("FLARE++ Y", Yp, Ypr, tol)


@pytest.mark.parametrize("B,H,N,M,share,mult", [
    (16, 4, 4096, 128, True, 1.0),
    (8, 3, 2048, 256, False, 1.0),   # the shortest heads it takes, unshared synthesis values
    (16, 5, 3001, 96, True, 1.0),    # three latent blocks (the decode's generic latent loop)
    (16, 4, 3000, 128, True, 8.0),   # keys x8: exact-score redo in both encodes and the decode
])
def test_latent_blocks_per_workgroup(flare, orc, B, H, N, M, share, mult):
    """FLARE++, bf16, D = 32, heads of 2048 to 8192 tokens whose latent
    blocks B H M / 32 fill more than half of the compute units and at most
    all of them (on MI355X): every (head, latent block) runs its synthesis
    encode, blend and routing encode in its own workgroup over all of the
    head's tokens, then the decode runs as its own launch."""
    from rank_latent_attention_amd.inputs import make_gaussian_pp, to_dtype
    say(f"[latent blocks] B{B} H{H} N{N} M{M} D32 bf16 shared={share} keys x{mult:g}")
    tol = TOL["bf16"]
    w = make_gaussian_pp(B, H, N, M, 32, dtype="bf16", seed=71 + N, share_vs=share)
    if mult != 1.0:
        w.Ks = to_dtype(w.Ks.astype(np.float64) * mult, "bf16")
        w.Vs = w.Ks if share else w.Vs
        w.K = to_dtype(w.K.astype(np.float64) * mult, "bf16")
    Y, Qo, Z, L = run_pp(flare, w)
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(Z)) and np.all(np.isfinite(L))
    Yr, Qr, Zr, Lr = orc.flare_pp_forward(w.Qs, w.Ks, w.Vs, w.Qf, w.gate, w.K, w.V)
    check("Q", Qo, Qr, tol)
    if mult == 1.0:
        check("Z", Z, Zr, tol)
        check_lse("L", L, Lr, tol)
        check("Y", Y, Yr, tol)
    say("  routing from the formed queries:")
    Yq, Zq, Lq = orc.flare_forward(Qo, w.K, w.V)
    check("Z", Z, Zq, tol)
    check_lse("L", L, Lq, tol)
    check("Y", Y, Yq, tol)


def test_encode_and_decode_entry_points(flare, orc):
    import torch
    from rank_latent_attention_amd.inputs import make_gaussian
    w = make_gaussian(2, 2, 777, 64, 16, "f32", seed=8)
    Q, K, V = dev(w.Q, "f32"), dev(w.K, "f32"), dev(w.V, "f32")
    Z, L = flare.flare_encode(Q, K, V)
    Zr, Lr = orc.encode(w.Q, w.K, w.V)
    check("encode Z", host(Z), Zr, 1e-5)
    check_lse("encode L", host(L), Lr, 1e-5)
    Zin = dev(Zr, "f32")                      # decode on the oracle's latents
    Y = flare.flare_decode(Q, K, Zin)
    torch.cuda.synchronize()
    check("decode Y", host(Y), orc.decode(w.Q, w.K, Zr), 1e-5)


# --------------------------------------------------------------------------
# Closed forms and properties
# --------------------------------------------------------------------------

def test_hand_example_embedded(flare):
    """Worked example (s = 1, D = 1) padded to D = 16 with zeros: exact values."""
    import torch
    D = 16
    Q = np.zeros((1, 2, D), np.float32); Q[0, 1, 0] = 1.0
    K = np.zeros((1, 1, 2, D), np.float32); K[0, 0, 1, 0] = math.log(3.0)
    V = np.zeros((1, 1, 2, D), np.float32); V[0, 0, 0, 0] = 1.0; V[0, 0, 1, 0] = 5.0
    Zt = torch.empty((1, 1, 2, D), dtype=torch.float32, device="cuda:0")
    Lt = torch.empty((1, 1, 2), dtype=torch.float32, device="cuda:0")
    Y, _, _ = flare.flare_forward(dev(Q, "f32"), dev(K, "f32"), dev(V, "f32"), scale=1.0, Z=Zt, L=Lt)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(Zt)[0, 0, :, 0], [3.0, 4.0], rtol=2e-6)
    np.testing.assert_allclose(host(Lt)[0, 0], [math.log(2), math.log(4)], rtol=2e-6)
    np.testing.assert_allclose(host(Y)[0, 0, :, 0], [3.5, 3.75], rtol=2e-6)
    assert np.all(host(Zt)[..., 1:] == 0) and np.all(host(Y)[..., 1:] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identical_keys_give_mean(flare, dtype):
    from rank_latent_attention_amd.inputs import make_gaussian
    w = make_gaussian(1, 2, 3000, 64, 32, dtype, seed=9)
    w.K = np.ascontiguousarray(np.broadcast_to(w.K[:, :, :1], w.K.shape))
    Y, Z, L = run_flare(flare, w)
    mean = w.V.astype(np.float64).mean(axis=2, keepdims=True)
    check("Z vs mean(V)", Z, np.broadcast_to(mean, Z.shape), TOL[dtype])
    check("Y vs mean(V)", Y, np.broadcast_to(mean, Y.shape), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_token_permutation_equivariance(flare, dtype):
    from rank_latent_attention_amd.inputs import make_gaussian
    w = make_gaussian(1, 2, 2000, 64, 16, dtype, seed=10)
    perm = np.random.default_rng(11).permutation(w.N)
    Y, Z, L = run_flare(flare, w)
    w.K, w.V = np.ascontiguousarray(w.K[:, :, perm]), np.ascontiguousarray(w.V[:, :, perm])
    Yp, Zp, Lp = run_flare(flare, w)
    tol = TOL[dtype]
    check("Z permuted", Zp, Z, tol)
    check_lse("L permuted", Lp, L, tol)
    check("Y permuted", Yp, Y[:, :, perm], tol)


def test_bitwise_reproducible(flare):
    """Repeated calls give identical bits: the split launch sequence, the
    one-workgroup-per-head forwards (FLARE and FLARE++) and the decode that
    merges the splits itself."""
    from rank_latent_attention_amd.inputs import make_gaussian, make_gaussian_pp
    B = _head_batch(4, "half")
    for w in (make_gaussian(2, 4, 50000, 128, 32, "bf16", seed=12), make_gaussian(B, 4, 2000, 64, 32, "bf16", seed=13),
              make_gaussian(16, 4, 3000, 256, 16, "bf16", seed=14)):
        say(f"[reproducible] B{w.B} H{w.H} N{w.N} M{w.M} D{w.D}")
        a = run_flare(flare, w)
        b = run_flare(flare, w)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    wp = make_gaussian_pp(B, 4, 2000, 64, 32, dtype="bf16", seed=16)
    a = run_pp(flare, wp)
    b = run_pp(flare, wp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_shared_values_path_equals_copy(flare):
    from rank_latent_attention_amd.inputs import make_gaussian_pp
    w = make_gaussian_pp(2, 2, 5000, 64, 32, dtype="bf16", seed=13, share_vs=True)
    a = run_pp(flare, w, alias=True)
    b = run_pp(flare, w, alias=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mult", [10.0, 60.0])
def test_large_scores_do_not_overflow(flare, orc, dtype, mult):
    """Queries scaled by 10 (largest log2 score about 21) and by 60 (about
    130): the rounded queries of the fast loops would move these scores by
    more than their bound, and at x60 the weights leave the float range, so
    the work is redone with exact scores and the exact maximum; both meet the
    workloads' bars."""
    from rank_latent_attention_amd.inputs import make_gaussian, to_dtype
    w = make_gaussian(1, 2, 4000, 64, 16, dtype, seed=14)
    w.Q = to_dtype(w.Q.astype(np.float64) * mult, dtype)
    smax = np.max(np.einsum("hmd,bhnd->bhmn", w.Q.astype(np.float64), w.K.astype(np.float64))) * math.log2(math.e) / 4
    say(f"[large scores] x{mult:g} {dtype}: largest log2 score {smax:.1f}")
    Y, Z, L = run_flare(flare, w)
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    assert np.all(np.isfinite(Y)) and np.all(np.isfinite(Z)) and np.all(np.isfinite(L))
    tol = TOL[dtype]
    check("Z", Z, Zr, tol)
    check_lse("L", L, Lr, tol)
    check("Y", Y, Yr, tol)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("e", [6, 12])
def test_extreme_scores_stay_finite(flare, orc, dtype, e):
    """Scores of order 10^4 and 10^6 in log2 units (s log2(e) = 2^e, sign
    keys, queries of one or two times a sign row), exact in every product:
    every unshifted weight overflows, so the fast loops' sums are Inf or NaN
    (an Inf weight times a zero selector), and every unit of work must take
    the exact recomputation.  L is of order 10^5 to 10^7 here and float32
    holds it to a few units in its last place."""
    rng = np.random.default_rng(11)

    def signs(shape, lo, hi):
        mag = np.exp2(rng.integers(lo, hi, size=shape[:-1] + (1,)))
        return ((rng.integers(0, 2, size=shape) * 2 - 1) * mag).astype(np.float32)
    B, H, N, M, D = 1, 2, 700, 64, 32
    Q, K = signs((H, M, D), 0, 2), signs((B, H, N, D), -1, 3)
    V = (np.round(rng.standard_normal((B, H, N, D)) * 4) / 4).astype(np.float32)
    scale = 2.0 ** e / math.log2(math.e)
    say(f"[extreme scores] s log2 e = 2^{e}, {dtype}")
    import torch
    Qd, Kd, Vd = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=Kd.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=Kd.device)
    Y, _, _ = flare.flare_forward(Qd, Kd, Vd, scale=scale, Z=Z, L=L)
    torch.cuda.synchronize()
    Y, Z, L = host(Y), host(Z), host(L)
    Yr, Zr, Lr = orc.flare_forward(Q, K, V, scale=scale)
    check("Z", Z, Zr, TOL[dtype])
    check("Y", Y, Yr, TOL[dtype])
    dL = np.abs(np.asarray(L, np.float64) - Lr)
    say(f"  L: largest |L - L_oracle| {dL.max():.3g} at |L| up to {np.abs(Lr).max():.3g}")
    assert np.all(dL <= 4 * 2.0 ** -23 * np.abs(Lr) + 1e-3)


def test_split_sums_beyond_float_range(flare, orc):
    """All keys identical with log2 scores of about 115, over 2^16 tokens cut
    into hundreds of workgroup splits: every split's weight sum is finite
    (about 2^122) but their total is not, so the splits must be merged in
    shifted form (Sec. 3.3).  Each latent then averages V (the weights are
    equal), and L = ln N + s q.k."""
    from rank_latent_attention_amd.inputs import make_gaussian, to_dtype
    N, M, D = 1 << 16, 64, 32
    w = make_gaussian(1, 1, N, M, D, "bf16", seed=31)
    c = math.log2(math.e) / math.sqrt(D)
    k = w.Q[0, 0].astype(np.float64)
    k = k / np.linalg.norm(k) * 115.0 / (c * np.linalg.norm(w.Q[0, 0]))  # the log2 score of latent 0 is ~115
    w.K = np.ascontiguousarray(np.broadcast_to(to_dtype(k, "bf16"), (1, 1, N, D)))
    S2 = c * w.Q[0].astype(np.float64) @ w.K[0, 0, 0].astype(np.float64)
    say(f"[split sums] largest log2 score {S2.max():.1f}, {N} tokens")
    assert S2.max() > 110
    Y, Z, L = run_flare(flare, w)
    mean = w.V.astype(np.float64).mean(axis=2, keepdims=True)
    check("Z vs mean(V)", Z, np.broadcast_to(mean, Z.shape), TOL["bf16"])
    Lr = np.log(N) + S2 / math.log2(math.e)
    check_lse("L", L, Lr[None, None], TOL["bf16"])
    Yr, Zr, Lr2 = orc.flare_forward(w.Q, w.K, w.V)
    check("Y", Y, Yr, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_key_shift_leaves_latents(flare, orc, dtype):
    """K -> K + 1 c^T adds q_m . c to every score of latent m, which the
    softmax over the tokens removes (App. B.3): Z and the oracle's Z of the
    unshifted keys agree.  Keys on a grid of 1/16 and integer shifts keep
    every shifted key exact in bf16."""
    from rank_latent_attention_amd.inputs import make_gaussian
    w = make_gaussian(1, 2, 3000, 64, 32, dtype, seed=32)
    rng = np.random.default_rng(33)
    w.K = (np.clip(np.round(w.K.astype(np.float64) * 8), -100, 100) / 16).astype(np.float32)
    shift = rng.integers(-3, 4, size=(1, 2, 1, 32)).astype(np.float32)
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    w.K = (w.K + shift).astype(np.float32)
    Y, Z, L = run_flare(flare, w)
    check("Z of shifted keys vs Z", Z, Zr, TOL[dtype])
    Zs, _ = orc.encode(w.Q, w.K, w.V)
    check("oracle Z of shifted keys vs Z", Zs, Zr, 1e-12)


def test_head_key_bound_matches_per_block_checks(flare, orc):
    """flare_forward hands the decode each head's largest key norm from the
    encode, and the decode skips its per-block key-norm check for heads
    where that bound already rules out a score error beyond the limit.  One
    head here has a few keys 60 times longer than the others (its blocks with
    them take the exact recomputation), the others none.  The forward's Y must
    equal, bit for bit, the standalone decode's (which checks every block)
    on the forward's own Z, and match the oracle."""
    import torch
    from rank_latent_attention_amd.inputs import make_gaussian
    w = make_gaussian(1, 3, 5000, 64, 32, "bf16", seed=41)
    rng = np.random.default_rng(42)
    big = rng.choice(5000, size=5, replace=False)
    K = w.K.astype(np.float32).copy()
    K[0, 1, big] *= 60.0
    w.K = dev(K, "bf16").float().cpu().numpy()  # both sides take the bf16-rounded keys
    Q, Kd, V = dev(w.Q, "bf16"), dev(w.K, "bf16"), dev(w.V, "bf16")
    Z = torch.empty((1, 3, 64, 32), dtype=torch.float32, device=Kd.device)
    L = torch.empty((1, 3, 64), dtype=torch.float32, device=Kd.device)
    Y, _, _ = flare.flare_forward(Q, Kd, V, Z=Z, L=L)
    Yd = flare.flare_decode(Q, Kd, Z)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yd), "forward and standalone decode differ"
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    check("Y", host(Y), Yr, TOL["bf16"])
    check("Z", host(Z), Zr, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_query_shift_leaves_decode(flare, orc, dtype):
    """Q -> Q + 1 c^T adds k_n . c to every decode score of token n, which the
    softmax over the latents removes: flare_decode of the shifted queries on
    the same latents gives the same Y (queries on a grid of 1/64 and shifts
    on a grid of 1/8 keep them exact in bf16)."""
    import torch
    from rank_latent_attention_amd.inputs import make_gaussian
    w = make_gaussian(2, 2, 2500, 64, 32, dtype, seed=34)
    rng = np.random.default_rng(35)
    w.Q = (np.clip(np.round(w.Q.astype(np.float64) * 64), -120, 120) / 64).astype(np.float32)
    Zr, _ = orc.encode(w.Q, w.K, w.V)
    Yr = orc.decode(w.Q, w.K, Zr)
    Qs = (w.Q + rng.integers(-4, 5, size=(2, 1, 32)) / 8).astype(np.float32)
    Y = flare.flare_decode(dev(Qs, dtype), dev(w.K, dtype), dev(Zr, "f32"))
    torch.cuda.synchronize()
    check("Y of shifted queries vs Y", host(Y), Yr, TOL[dtype])


def test_explicit_scale(flare, orc):
    from rank_latent_attention_amd.inputs import make_gaussian, make_gaussian_pp
    w = make_gaussian(1, 2, 900, 32, 16, "f32", seed=15)
    Y, Z, L = run_flare(flare, w, scale=0.37)
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V, scale=0.37)
    check("Z", Z, Zr, 1e-5)
    check("Y", Y, Yr, 1e-5)
    # the one-workgroup-per-head FLARE++ forward with the same override
    wp = make_gaussian_pp(_head_batch(4, "half"), 4, 700, 64, 32, dtype="bf16", seed=17)
    Y, Qo, Z, L = run_pp(flare, wp, scale=0.37)
    Yr, Qr, Zr, Lr = orc.flare_pp_forward(wp.Qs, wp.Ks, wp.Vs, wp.Qf, wp.gate, wp.K, wp.V, scale=0.37)
    check("Q", Qo, Qr, TOL["bf16"])
    check("Z", Z, Zr, TOL["bf16"])
    check("Y", Y, Yr, TOL["bf16"])


def test_empty_token_axis(flare):
    """N = 0: every latent is an empty row, Z = 0 and L = -inf (App. B.3)."""
    import torch
    Q = torch.randn(2, 8, 16, device="cuda:0")
    K = torch.empty(1, 2, 0, 16, device="cuda:0")
    Z = torch.full((1, 2, 8, 16), 7.0, device="cuda:0")
    L = torch.zeros((1, 2, 8), device="cuda:0")
    flare.flare_forward(Q, K, K.clone(), Z=Z, L=L)
    torch.cuda.synchronize()
    assert torch.all(Z == 0) and torch.all(torch.isneginf(L))


def test_workspace_too_small_is_rejected(flare):
    import torch
    from rank_latent_attention_amd.flare import FlareError, OP_FORWARD, workspace_size
    Q = torch.randn(1, 64, 16, device="cuda:0")
    K = torch.randn(1, 1, 4096, 16, device="cuda:0")
    need = workspace_size(OP_FORWARD, 1, 1, 4096, 64, 16, 0)
    assert need > 0
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(FlareError) as e:
        flare.flare_forward(Q, K, K, ws=ws)
    assert e.value.status == 3


def _random_shapes(seed, count):
    """Seeded random (B, H, N, M, D): ragged token counts (including fewer
    tokens than a tile or a workgroup piece), latent counts off the 32-grid
    and both widths."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 3000)),
                    int(rng.integers(1, 257)), int(rng.choice([16, 32]))))
    return out


@pytest.mark.parametrize("shape", _random_shapes(2024, 12), ids=lambda s: "B{}H{}N{}M{}D{}".format(*s))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_random_shapes(flare, orc, shape, dtype):
    from rank_latent_attention_amd.inputs import make_gaussian
    B, H, N, M, D = shape
    w = make_gaussian(B, H, N, M, D, dtype, seed=7 * N + M)
    say(f"[random shape] {shape} {dtype}")
    Y, Z, L = run_flare(flare, w)
    Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    tol = TOL[dtype]
    check("Z", Z, Zr, tol)
    check_lse("L", L, Lr, tol)
    check("Y", Y, Yr, tol)


def _random_short_heads(seed, count):
    """Seeded shapes (B, H, N, M, FLARE++) for the many-short-heads forwards,
    drawn in turn from four regimes of a 256-unit chip: latent blocks per
    workgroup (FLARE++, B H M / 32 between half and all of the units, 2048 to
    8192 tokens), one workgroup per head (M of 64 or 128, B H of half the
    units or more), the decode that merges the splits (FLARE, M = 256, many
    heads), and shapes just outside these (M not a power of two, heads longer
    than the per-head bound).  B H N M stays under 8e7 so that the oracle
    ends in seconds."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        H = int(rng.choice([2, 4, 8]))
        regime = i % 4
        if regime == 0:
            MB = int(rng.integers(2, 9))
            lo, hi = 128 // MB + 1, 256 // MB
            BH = int(rng.integers(lo, hi + 1))
            N, M, pp = int(rng.integers(2048, 8193)), 32 * MB, True
        elif regime == 1:
            M, pp = int(rng.choice([64, 128])), bool(rng.integers(0, 2))
            BH = int(rng.integers(128, 321))
            N = int(rng.integers(1, (8192 if pp or BH >= 256 else 4096) + 1))
        elif regime == 2:
            BH, M, pp = int(rng.integers(64, 161)), 256, False
            N = int(rng.integers(1, 8193))
        else:
            M, pp = int(rng.choice([96, 160, 192])), bool(rng.integers(0, 2))
            BH = int(rng.integers(32, 257))
            N = int(rng.integers(4097, 9001))
        N = max(1, min(N, 80_000_000 // (BH * M)))
        out.append((max(1, BH // H), H, N, M, pp))
    return out


@pytest.mark.parametrize("shape", _random_short_heads(77, 8),
                         ids=lambda s: "B{}H{}N{}M{}{}".format(*s[:4], "pp" if s[4] else ""))
def test_random_short_head_shapes(flare, orc, shape):
    from rank_latent_attention_amd.inputs import make_gaussian, make_gaussian_pp
    B, H, N, M, pp = shape
    say(f"[short heads] B{B} H{H} N{N} M{M} D32 bf16 {'FLARE++' if pp else 'FLARE'}")
    tol = TOL["bf16"]
    if pp:
        w = make_gaussian_pp(B, H, N, M, 32, dtype="bf16", seed=N + M, share_vs=bool(N % 2))
        Y, Qo, Z, L = run_pp(flare, w)
        Yr, Qr, Zr, Lr = orc.flare_pp_forward(w.Qs, w.Ks, w.Vs, w.Qf, w.gate, w.K, w.V)
        check("Q", Qo, Qr, tol)
    else:
        w = make_gaussian(B, H, N, M, 32, "bf16", seed=N + M)
        Y, Z, L = run_flare(flare, w)
        Yr, Zr, Lr = orc.flare_forward(w.Q, w.K, w.V)
    check("Z", Z, Zr, tol)
    check_lse("L", L, Lr, tol)
    check("Y", Y, Yr, tol)
