"""Host-side checks of the C ABI: the library loads, exports every function
that include/flare.h declares, and rejects bad arguments before touching the
GPU (these calls return before any HIP runtime call, so they run without one)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flare.h")


@pytest.fixture(scope="module")
def lib():
    from rank_latent_attention_amd import flare
    if not os.path.exists(flare.LIB_PATH):
        from rank_latent_attention_amd import build
        build.build()
    return flare.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(flare_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["flare_workspace_size", "flare_encode", "flare_decode", "flare_forward",
                                           "flare_pp_forward", "flare_pp_forward_norm", "flare_backward",
                                           "flare_encode_backward", "flare_pp_backward", "flare_pp_backward_norm",
                                           "flare_status_string", "flare_forward_noalloc", "flare_forward_proj",
                                           "flare_pp_forward_proj"])


def test_library_exports_every_declared_symbol(lib):
    from rank_latent_attention_amd import flare
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(flare.SYMBOLS) == set(declared_functions())


def test_status_strings(lib):
    for code, word in [(0, b"ok"), (1, b"invalid"), (2, b"unsupported"), (3, b"workspace"), (4, b"HIP")]:
        assert word in lib.flare_status_string(code)
    assert lib.flare_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(1 << 20)        # 16-byte aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)


def enc(lib, B=1, H=1, N=64, M=32, D=16, dt=1, qb=0, Q=FAKE, K=FAKE, V=FAKE, Z=FAKE):
    return lib.flare_encode(Q, qb, K, V, Z, None, B, H, N, M, D, dt, 0.0, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=24), 2), (dict(D=64), 2), (dict(M=257), 2), (dict(dt=7), 2),
    (dict(M=0), 1), (dict(B=0), 1), (dict(H=-1), 1), (dict(N=-5), 1), (dict(qb=2), 1),
    (dict(Q=None), 1), (dict(Z=None), 1), (dict(K=None), 1), (dict(V=None), 1),
    (dict(Q=MISALIGNED), 1), (dict(K=MISALIGNED), 1),
    (dict(B=1 << 16, H=1 << 8, N=1 << 8), 2),
])
def test_encode_rejects_bad_arguments(lib, kw, status):
    assert enc(lib, **kw) == status


def test_other_entry_points_reject_bad_arguments(lib):
    assert lib.flare_decode(FAKE, 0, FAKE, FAKE, FAKE, 1, 1, 8, 8, 48, 1, 0.0, None, 0, None) == 2
    assert lib.flare_decode(None, 0, FAKE, FAKE, FAKE, 1, 1, 8, 8, 16, 1, 0.0, None, 0, None) == 1
    assert lib.flare_forward(FAKE, 0, FAKE, FAKE, None, None, None, 1, 1, 8, 8, 16, 1, 0.0, None, 0, None) == 1
    assert lib.flare_forward(FAKE, 0, FAKE, FAKE, FAKE, None, None, 1, 1, 8, 300, 16, 1, 0.0, None, 0, None) == 2
    assert lib.flare_pp_forward(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None,
                                1, 1, 8, 8, 16, 1, 0.0, None, 0, None) == 1
    assert lib.flare_pp_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                                1, 1, 8, 8, 20, 1, 0.0, None, 0, None) == 2
    assert lib.flare_workspace_size(9, 1, 1, 8, 8, 16, 1) == 0
    assert lib.flare_workspace_size(0, 1, 1, 8, 8, 24, 1) == 0
    assert lib.flare_workspace_size(1, 1, 1, 8, 8, 16, 1) == 0   # the decode needs no workspace


def ppn(lib, flags=15, eps=1e-6, dt=1, D=16, aqs=None, aks=None, ak=None):
    return lib.flare_pp_forward_norm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                                     1, 1, 8, 8, D, dt, 0.0, flags, aqs, aks, ak, eps, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=16), 1), (dict(flags=-1), 1),                       # unknown flag bits
    (dict(eps=0.0), 1), (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1),
    (dict(dt=0), 2),                                                 # float32 inputs cannot be normalised
    (dict(aqs=MISALIGNED), 1), (dict(ak=MISALIGNED), 1),
    (dict(D=20), 2),
])
def test_pp_forward_norm_rejects_bad_arguments(lib, kw, status):
    assert ppn(lib, **kw) == status


def bwd(lib, dt=1, D=16, M=8, Q=FAKE, Z=FAKE, L=FAKE, dY=FAKE, dQ=FAKE, dK=FAKE, dZo=None):
    return lib.flare_backward(Q, 0, FAKE, FAKE, Z, L, dY, dQ, dK, FAKE, dZo, 1, 1, 8, M, D, dt, 0.0, FAKE, 1 << 30,
                              None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=3), 2), (dict(D=24), 2), (dict(M=300), 2),              # unknown dtype, head size, latent count
    (dict(dt=0, Q=None), 1), (dict(dt=0, dQ=MISALIGNED), 1),         # float32: the same argument checks
    (dict(Q=None), 1), (dict(Z=None), 1), (dict(L=None), 1), (dict(dY=None), 1), (dict(dQ=None), 1),
    (dict(dK=None), 1), (dict(dQ=MISALIGNED), 1), (dict(dZo=MISALIGNED), 1),
])
def test_backward_rejects_bad_arguments(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_encode_backward_rejects_bad_arguments(lib):
    eb = lib.flare_encode_backward
    assert eb(FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 1, 1, 8, 8, 16, 1, 0.0, FAKE, 1 << 30,
              None) == 1   # dZ is required
    assert eb(FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE, 1, 1, 8, 8, 16, 1, 0.0, FAKE,
              1 << 30, None) == 1
    assert eb(FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1, 1, 8, 8, 16, 3, 0.0, FAKE, 1 << 30,
              None) == 2   # unknown dtype
    assert eb(FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 1, 1, 8, 8, 16, 0, 0.0, FAKE, 1 << 30,
              None) == 1   # float32: dZ is required too
    assert lib.flare_workspace_size(7, 1, 1, 8, 8, 16, 0) == 0   # the backward through the norms is bf16 only


def ppb(lib, dt=1, D=16, Vs=FAKE, dVs=FAKE, Q=FAKE, dgate=FAKE, dQo=None):
    return lib.flare_pp_backward(FAKE, FAKE, Vs, FAKE, FAKE, FAKE, FAKE, Q, FAKE, FAKE, FAKE, FAKE, FAKE, dVs, FAKE,
                                 dgate, dQo, FAKE, FAKE, 1, 1, 8, 8, D, dt, 0.0, FAKE, 1 << 30, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=3), 2), (dict(D=20), 2), (dict(Q=None), 1), (dict(dgate=None), 1), (dict(dt=0, Q=None), 1),
    (dict(Vs=ctypes.c_void_p(2 << 20), dVs=None), 1),   # separate synthesis values need their cotangent
    (dict(dQo=MISALIGNED), 1),
])
def test_pp_backward_rejects_bad_arguments(lib, kw, status):
    assert ppb(lib, **kw) == status


def ppbn(lib, dt=1, D=16, flags=15, eps=1e-6, aqs=FAKE, daqs=FAKE, ak=FAKE, dak=FAKE, Q=FAKE):
    return lib.flare_pp_backward_norm(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, Q, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None, FAKE, FAKE, None, FAKE, FAKE, daqs, None, dak, 1, 1, 8, 8, D, dt, 0.0,
                                      flags, aqs, None, ak, eps, FAKE, 1 << 30, None)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=16), 1), (dict(dt=0), 2), (dict(D=20), 2), (dict(eps=0.0), 1), (dict(eps=-1.0), 1),
    (dict(daqs=None), 1),                 # a scale given with its flag set needs its cotangent
    (dict(dak=None), 1), (dict(aqs=MISALIGNED), 1), (dict(dak=MISALIGNED), 1),
    (dict(flags=0, Q=None), 1),           # no norms: the call is flare_pp_backward, with its checks
])
def test_pp_backward_norm_rejects_bad_arguments(lib, kw, status):
    assert ppbn(lib, **kw) == status


def test_pp_backward_norm_workspace_holds_the_normalised_inputs(lib):
    # no device here: the size query fails closed (0) rather than guessing
    assert lib.flare_workspace_size(7, 1, 1, 8, 8, 16, 0) == 0   # bf16 only
    assert lib.flare_workspace_size(8, 1, 1, 8, 8, 16, 1) == 0   # unknown op


# --------------------------------------------------------------------------
# The Python binding validates caller-supplied outputs and the device before
# any library call (CPU tensors here: the checks fire before anything runs).
# --------------------------------------------------------------------------

def _cpu(shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("bad", ["Z_shape", "Z_dtype", "L_shape", "Y_shape", "Y_dtype", "ws_type"])
def test_binding_rejects_wrong_outputs(bad):
    import torch
    from rank_latent_attention_amd import flare
    B, H, N, M, D = 1, 2, 100, 32, 16
    Q, K, V = _cpu((H, M, D)), _cpu((B, H, N, D)), _cpu((B, H, N, D))
    kw = {"Z": torch.zeros((B, H, M, D)), "L": torch.zeros((B, H, M)), "Y": _cpu((B, H, N, D))}
    if bad == "Z_shape":
        kw["Z"] = torch.zeros((B, H, M - 1, D))
    elif bad == "Z_dtype":
        kw["Z"] = _cpu((B, H, M, D))
    elif bad == "L_shape":
        kw["L"] = torch.zeros((B, H, M, 1))
    elif bad == "Y_shape":
        kw["Y"] = _cpu((B, H, N - 1, D))
    elif bad == "Y_dtype":
        kw["Y"] = torch.zeros((B, H, N, D))
    with pytest.raises((ValueError, TypeError)):
        if bad == "ws_type":
            flare.flare_forward(Q, K, V, ws=bytearray(16), **kw)
        else:
            flare.flare_forward(Q, K, V, **kw)


def test_binding_rejects_wrong_outputs_of_every_entry_point():
    import torch
    from rank_latent_attention_amd import flare
    B, H, N, M, D = 2, 2, 64, 16, 16
    Q, K, V = _cpu((H, M, D)), _cpu((B, H, N, D)), _cpu((B, H, N, D))
    gate = torch.zeros(H)
    small = torch.zeros((B, H, M - 1, D))
    with pytest.raises(ValueError):
        flare.flare_encode(Q, K, V, Z=small)
    with pytest.raises(ValueError):
        flare.flare_decode(Q, K, torch.zeros((B, H, M, D)), Y=_cpu((B, H, N, D // 2)))
    with pytest.raises(ValueError):
        flare.flare_pp_forward(Q, K, K, Q, gate, K, V, Q_out=small)
    with pytest.raises(ValueError):
        flare.flare_pp_forward_norm(Q, K, K, Q, gate, K, V, flare.NORM_FLAREPP, Z=small)
    Z, L = torch.zeros((B, H, M, D)), torch.zeros((B, H, M))
    with pytest.raises(ValueError):
        flare.flare_backward(Q, K, V, Z, L, K, dK=_cpu((B, H, N - 1, D)))
    with pytest.raises(ValueError):
        flare.flare_backward(Q, K, V, Z, L, K, dQ=_cpu((H, M, D)))
    with pytest.raises(ValueError):
        flare.flare_encode_backward(Q, K, V, Z, L, Z, dV=torch.zeros((B, H, N, D)))
    Qb = torch.zeros((B, H, M, D))
    with pytest.raises(ValueError):
        flare.flare_pp_backward(Q, K, K, Q, gate, K, V, Qb, Z, L, K, dQ_out=small)


def test_binding_rejects_host_tensors():
    """Well-formed arguments that live in host memory are refused: the
    kernels would dereference their addresses on the GPU."""
    from rank_latent_attention_amd import flare
    Q, K, V = _cpu((2, 32, 16)), _cpu((1, 2, 100, 16)), _cpu((1, 2, 100, 16))
    with pytest.raises(ValueError, match="GPU"):
        flare.flare_forward(Q, K, V)
    with pytest.raises(ValueError, match="GPU"):
        flare.flare_decode(Q, K, _cpu((1, 2, 32, 16)).float())
