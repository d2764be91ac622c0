"""The allocation-free entry point flare_forward_noalloc (include/flare.h)
against flare_forward on the same inputs, through the C ABI: two calls in a
row on the same GPU's scratch array, the second on a smaller problem, each
bitwise equal to flare_forward's result (same kernels, same split plan) and
so within the workloads' bars; and a problem whose scratch exceeds the
array is refused before anything runs."""
import numpy as np
import pytest

from helpers import TOL, dev, host, lse_err, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def flare():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_latent_attention_amd as r
    r.load()
    return r


def _run(flare, w, noalloc):
    import torch
    Q, K, V = dev(w.Q, w.dtype), dev(w.K, w.dtype), dev(w.V, w.dtype)
    B, H, N, D = K.shape
    M = Q.shape[-2]
    Y = torch.empty_like(K)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device)
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device)
    if noalloc:
        flare.flare_forward_noalloc(Q, K, V, Y=Y, Z=Z, L=L)
    else:
        flare.flare_forward(Q, K, V, Y=Y, Z=Z, L=L)
    torch.cuda.synchronize()
    return host(Y), host(Z), host(L)


def test_noalloc_matches_forward_twice_second_smaller(flare):
    from rank_latent_attention_amd.inputs import make_gaussian
    # the second shape has enough short heads for one workgroup per head
    for shape, dtype in [((2, 4, 40000, 256, 32), "bf16"), ((32, 4, 2000, 64, 32), "bf16"), ((1, 3, 5000, 64, 16), "bf16"),
                         ((1, 2, 3000, 48, 16), "f32")]:
        w = make_gaussian(*shape, dtype=dtype, seed=sum(shape))
        print(f"[noalloc] {shape} {dtype}", flush=True)
        ref = _run(flare, w, noalloc=False)
        got = _run(flare, w, noalloc=True)
        for name, g, r in zip("YZ", got[:2], ref[:2]):
            e = rel_l2(g, r)
            print(f"  {name}: rel-L2 vs flare_forward {e:.3e}, bitwise equal {np.array_equal(g, r)}", flush=True)
            assert e <= TOL[dtype]
            assert np.array_equal(g, r)
        assert lse_err(got[2], ref[2]) <= TOL[dtype]
        assert np.array_equal(got[2], ref[2])


def test_noalloc_without_latent_outputs(flare):
    """Z and L not requested: they live in the scratch array too."""
    import torch
    from rank_latent_attention_amd.inputs import make_gaussian
    w = make_gaussian(1, 2, 3333, 128, 32, "bf16", seed=41)
    Yr = _run(flare, w, noalloc=False)[0]
    Q, K, V = dev(w.Q, "bf16"), dev(w.K, "bf16"), dev(w.V, "bf16")
    Y = torch.empty_like(K)
    flare.flare_forward_noalloc(Q, K, V, Y=Y)
    torch.cuda.synchronize()
    assert np.array_equal(host(Y), Yr)


def test_noalloc_refuses_problems_beyond_its_scratch(flare):
    """B*H*M*D float32 latents alone beyond 32 MiB (here 64 MiB, with Z and L
    left to the scratch): refused with the workspace status, nothing run
    (the outputs keep their fill)."""
    import torch
    from rank_latent_attention_amd.flare import FlareError, OP_FORWARD, workspace_size
    B, H, N, M, D = 256, 8, 16, 256, 32
    assert workspace_size(OP_FORWARD, B, H, N, M, D, 1) > (32 << 20)
    Q = torch.zeros((H, M, D), dtype=torch.bfloat16, device="cuda:0")
    K = torch.zeros((B, H, N, D), dtype=torch.bfloat16, device="cuda:0")
    Y = torch.full_like(K, 3.0)
    with pytest.raises(FlareError) as e:
        flare.flare_forward_noalloc(Q, K, K, Y=Y)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert torch.all(Y == 3.0)
