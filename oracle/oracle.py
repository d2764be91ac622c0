"""ctypes front end of the fp64 C oracle (oracle/flare_oracle.c).

TEST INFRASTRUCTURE: imported by tests, by the smoke check and by the
benchmark's CPU-baseline leg only.  It shares no code with the GPU library.

All arrays are converted to contiguous float64; outputs are float64.
Shapes: K, V [B,H,N,D]; Q [H,M,D] (shared over the batch) or [B,H,M,D];
Z [B,H,M,D]; L [B,H,M]; Y [B,H,N,D].  ``scale <= 0`` selects 1/sqrt(D).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flare_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

__all__ = ["build", "lib", "threads", "encode", "decode", "flare_forward", "pp_queries",
           "flare_pp_forward", "materialize", "rms_norm", "flare_pp_forward_normed", "encode_backward",
           "decode_backward", "flare_backward", "flare_pp_backward", "rms_norm_backward",
           "flare_pp_backward_normed", "project", "flare_forward_proj", "flare_pp_forward_proj"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) into oracle/liboracle.so
    (without force, only when the library is missing or older than its source)."""
    global _lib
    stale = not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        L.oracle_encode.argtypes = [dp, i, dp, dp, i, i, i, i, i, ctypes.c_double, dp, dp]
        L.oracle_decode_rows.argtypes = [dp, i, dp, dp, i, i, i, i, i, ctypes.c_double,
                                         ctypes.POINTER(ctypes.c_long), ctypes.c_long, dp]
        L.oracle_flare_forward.argtypes = [dp, i, dp, dp, i, i, i, i, i, ctypes.c_double, dp, dp, dp]
        L.oracle_pp_queries.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, ctypes.c_double, dp]
        L.oracle_flare_pp_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, ctypes.c_double,
                                              dp, dp, dp, dp]
        L.oracle_materialize.argtypes = [dp, dp, i, i, i, ctypes.c_double, dp, dp]
        L.oracle_threads.argtypes = [i]
        L.oracle_encode_backward.argtypes = [dp, i, dp, dp, dp, dp, i, i, i, i, i, ctypes.c_double, dp, dp, dp]
        L.oracle_decode_backward.argtypes = [dp, i, dp, dp, dp, i, i, i, i, i, ctypes.c_double, dp, dp, dp]
        for fn in (L.oracle_encode, L.oracle_decode_rows, L.oracle_flare_forward, L.oracle_pp_queries,
                   L.oracle_flare_pp_forward, L.oracle_materialize, L.oracle_threads, L.oracle_encode_backward,
                   L.oracle_decode_backward):
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def threads(n: int = 0) -> int:
    """Set (n > 0) and return the OpenMP thread count the oracle uses."""
    return int(lib().oracle_threads(int(n)))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x: Optional[np.ndarray]):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _q_batched(Q: np.ndarray, B: int) -> int:
    if Q.ndim == 3:
        return 0
    if Q.ndim == 4 and Q.shape[0] == B:
        return 1
    raise ValueError(f"Q must be [H,M,D] or [B,H,M,D], got {Q.shape}")


def encode(Q, K, V, scale: float = 0.0) -> Tuple[np.ndarray, np.ndarray]:
    """Z = SDPA(Q, K, V) per (b, h) and its log-normaliser L."""
    K, V, Q = _f64(K), _f64(V), _f64(Q)
    B, H, N, D = K.shape
    M = Q.shape[-2]
    if V.shape != K.shape or Q.shape[-1] != D:
        raise ValueError("shape mismatch")
    Z = np.empty((B, H, M, D))
    L = np.empty((B, H, M))
    rc = lib().oracle_encode(_p(Q), _q_batched(Q, B), _p(K), _p(V), B, H, N, M, D, float(scale), _p(Z), _p(L))
    if rc:
        raise RuntimeError(f"oracle_encode failed ({rc})")
    return Z, L


def decode(Q, K, Z, scale: float = 0.0, idx=None) -> np.ndarray:
    """Y = SDPA(K, Q, Z) per (b, h); with ``idx`` only those token rows ([B,H,len(idx),D])."""
    K, Q, Z = _f64(K), _f64(Q), _f64(Z)
    B, H, N, D = K.shape
    M = Q.shape[-2]
    if idx is None:
        count, ip = N, None
    else:
        idx_arr = np.ascontiguousarray(np.asarray(idx, dtype=np.int64))
        count = int(idx_arr.size)
        ip = idx_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_long))
    Y = np.empty((B, H, count, D))
    rc = lib().oracle_decode_rows(_p(Q), _q_batched(Q, B), _p(K), _p(Z), B, H, N, M, D, float(scale), ip,
                                  count, _p(Y))
    if rc:
        raise RuntimeError(f"oracle_decode_rows failed ({rc})")
    return Y


def flare_forward(Q, K, V, scale: float = 0.0):
    """FLARE routing forward: returns (Y, Z, L)."""
    K, V, Q = _f64(K), _f64(V), _f64(Q)
    B, H, N, D = K.shape
    M = Q.shape[-2]
    Y = np.empty((B, H, N, D))
    Z = np.empty((B, H, M, D))
    L = np.empty((B, H, M))
    rc = lib().oracle_flare_forward(_p(Q), _q_batched(Q, B), _p(K), _p(V), B, H, N, M, D, float(scale),
                                    _p(Y), _p(Z), _p(L))
    if rc:
        raise RuntimeError(f"oracle_flare_forward failed ({rc})")
    return Y, Z, L


def pp_queries(Qs, Ks, Vs, Qf, gate, scale: float = 0.0) -> np.ndarray:
    """FLARE++ routing queries Q[b,h] = Qf[h] + gate[h] * SDPA(Qs[h], Ks[b,h], Vs[b,h])."""
    Qs, Ks, Vs, Qf, gate = _f64(Qs), _f64(Ks), _f64(Vs), _f64(Qf), _f64(gate)
    B, H, N, D = Ks.shape
    M = Qs.shape[-2]
    Qout = np.empty((B, H, M, D))
    rc = lib().oracle_pp_queries(_p(Qs), _p(Ks), _p(Vs), _p(Qf), _p(gate), B, H, N, M, D, float(scale),
                                 _p(Qout))
    if rc:
        raise RuntimeError(f"oracle_pp_queries failed ({rc})")
    return Qout


def flare_pp_forward(Qs, Ks, Vs, Qf, gate, K, V, scale: float = 0.0):
    """FLARE++ routing forward: returns (Y, Q, Z, L) with Q the per-batch routing queries."""
    Qs, Ks, Vs, Qf, gate = _f64(Qs), _f64(Ks), _f64(Vs), _f64(Qf), _f64(gate)
    K, V = _f64(K), _f64(V)
    B, H, N, D = K.shape
    M = Qs.shape[-2]
    Y = np.empty((B, H, N, D))
    Qout = np.empty((B, H, M, D))
    Z = np.empty((B, H, M, D))
    L = np.empty((B, H, M))
    rc = lib().oracle_flare_pp_forward(_p(Qs), _p(Ks), _p(Vs), _p(Qf), _p(gate), _p(K), _p(V), B, H, N, M, D,
                                       float(scale), _p(Y), _p(Qout), _p(Z), _p(L))
    if rc:
        raise RuntimeError(f"oracle_flare_pp_forward failed ({rc})")
    return Y, Qout, Z, L


def rms_norm(x, alpha=None, eps: float = 1e-6) -> np.ndarray:
    """Per-head RMS normalisation over the head dimension D (the last axis).

    FLARE++ paper, App. A.3 and A.4 and Table 2 in A.7: N_0 divides each row
    by its root mean square, and N_a additionally multiplies by a learned
    per-channel scale.  Written out in fp64:
        y[..., h, r, d] = x[..., h, r, d] / sqrt(mean_d x[..., h, r, :]^2 + eps) * alpha[h, d]
    ``x`` has the head axis third from last ([H, rows, D] or [B, H, rows, D]);
    ``alpha`` is [H, D], or None for N_0.  The pages do not state eps; the
    default 1e-6 is a reading of them, not a value they give.
    """
    x = _f64(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if alpha is not None:
        a = _f64(alpha)
        if a.shape != (x.shape[-3], x.shape[-1]):
            raise ValueError(f"alpha must be [H, D] = {(x.shape[-3], x.shape[-1])}, got {a.shape}")
        y = y * a[:, None, :]
    return y


def flare_pp_forward_normed(Qs, Ks, Vs, Qf, gate, K, V, *, norm_qs=False, norm_ks=False, norm_qf=False,
                            norm_k=False, alpha_qs=None, alpha_ks=None, alpha_k=None, eps: float = 1e-6,
                            scale: float = 0.0):
    """FLARE++ routing forward with its per-head input normalisations applied
    first, in the order of Table 2 (FLARE++ paper, App. A.7):
      seeds Q~ -> N(Q~; alpha_qs)     (FLARE++ and the simplified variant: N_a)
      keys  K~ -> N(K~; alpha_ks)     (FLARE++: N_0; simplified: N_a)
      V~ is the normalised K~ when it is the same array as K~ (App. A.6),
      otherwise it is used as given (simplified variant: no norm)
      Q^f   -> N_0(Q^f)               (FLARE++, App. A.4)
      K     -> N(K; alpha_k)          (FLARE++: N_a)
    then the plain FLARE++ forward.  Returns (Y, Q, Z, L).
    """
    shared = Vs is Ks
    Qs_n = rms_norm(Qs, alpha_qs, eps) if norm_qs else Qs
    Ks_n = rms_norm(Ks, alpha_ks, eps) if norm_ks else Ks
    Vs_n = Ks_n if shared else Vs
    Qf_n = rms_norm(Qf, None, eps) if norm_qf else Qf
    K_n = rms_norm(K, alpha_k, eps) if norm_k else K
    return flare_pp_forward(Qs_n, Ks_n, Vs_n, Qf_n, gate, K_n, V, scale)


def project(X, W) -> np.ndarray:
    """Per-head input projection of FLARE (FLARE++ paper, Sec. 3.1: K_h = X W_K,h
    and V_h = X W_V,h), in fp64.  X [B, N, C] (the block's input tokens,
    shared by every head), W [H, C, D]; returns [B, H, N, D] with
    out[b, h, n, :] = X[b, n, :] @ W[h]."""
    X, W = _f64(X), _f64(W)
    if X.ndim != 3 or W.ndim != 3 or W.shape[1] != X.shape[2]:
        raise ValueError(f"X must be [B,N,C] and W [H,C,D], got {X.shape}, {W.shape}")
    return np.ascontiguousarray(np.matmul(X[:, None], W[None]))


def flare_forward_proj(X, WK, WV, Q, scale: float = 0.0):
    """FLARE routing forward from the block input: K = X W_K, V = X W_V per head
    (Sec. 3.1), then the FLARE pair.  Returns (Y, Z, L)."""
    return flare_forward(Q, project(X, WK), project(X, WV), scale)


def flare_pp_forward_proj(X, WKs, WK, WV, Qs, Qf, gate, *, norm_qs=False, norm_ks=False, norm_qf=False,
                          norm_k=False, alpha_qs=None, alpha_k=None, eps: float = 1e-6, scale: float = 0.0):
    """FLARE++ routing forward from the block input: the synthesis keys
    K~ = X W~_K (also the synthesis values, App. A.6), the routing keys
    K = X W_K and values V = X W_V per head, then the per-head norms of the
    flags and the FLARE++ forward (flare_pp_forward_normed).  Returns (Y, Q, Z, L)."""
    Ks = project(X, WKs)
    return flare_pp_forward_normed(Qs, Ks, Ks, Qf, gate, project(X, WK), project(X, WV), norm_qs=norm_qs,
                                   norm_ks=norm_ks, norm_qf=norm_qf, norm_k=norm_k, alpha_qs=alpha_qs,
                                   alpha_k=alpha_k, eps=eps, scale=scale)


def materialize(Q, K, scale: float = 0.0):
    """One head: (Wenc [M,N], Wdec [N,M]) with Z = Wenc V and Y = Wdec Z."""
    Q, K = _f64(Q), _f64(K)
    M, D = Q.shape
    N = K.shape[0]
    Wenc = np.empty((M, N))
    Wdec = np.empty((N, M))
    rc = lib().oracle_materialize(_p(Q), _p(K), N, M, D, float(scale), _p(Wenc), _p(Wdec))
    if rc:
        raise RuntimeError(f"oracle_materialize failed ({rc})")
    return Wenc, Wdec


def encode_backward(Q, K, V, dZ, dL=None, scale: float = 0.0):
    """Reverse mode of the encoder (Z, L) = Enc(Q, K, V): FLARE++ paper, App.
    B.5, local backward with one shard.  Given the cotangents dZ [B,H,M,D] and
    dL [B,H,M] (None = 0) returns (dQ, dK, dV); dQ has Q's layout (summed
    over the batch when Q is [H,M,D])."""
    K, V, Q, dZ = _f64(K), _f64(V), _f64(Q), _f64(dZ)
    B, H, N, D = K.shape
    M = Q.shape[-2]
    dL = None if dL is None else _f64(dL)
    if V.shape != K.shape or dZ.shape != (B, H, M, D) or (dL is not None and dL.shape != (B, H, M)):
        raise ValueError("shape mismatch")
    dQ = np.empty(Q.shape)
    dK = np.empty(K.shape)
    dV = np.empty(V.shape)
    rc = lib().oracle_encode_backward(_p(Q), _q_batched(Q, B), _p(K), _p(V), _p(dZ), _p(dL), B, H, N, M, D,
                                      float(scale), _p(dQ), _p(dK), _p(dV))
    if rc:
        raise RuntimeError(f"oracle_encode_backward failed ({rc})")
    return dQ, dK, dV


def decode_backward(Q, K, Z, dY, scale: float = 0.0):
    """Reverse mode of the decoder Y = SDPA(K, Q, Z) (softmax over the latents,
    App. A.1): given dY [B,H,N,D] returns (dQ, dK, dZ)."""
    K, Q, Z, dY = _f64(K), _f64(Q), _f64(Z), _f64(dY)
    B, H, N, D = K.shape
    M = Q.shape[-2]
    if dY.shape != K.shape or Z.shape != (B, H, M, D):
        raise ValueError("shape mismatch")
    dQ = np.empty(Q.shape)
    dK = np.empty(K.shape)
    dZ = np.empty(Z.shape)
    rc = lib().oracle_decode_backward(_p(Q), _q_batched(Q, B), _p(K), _p(Z), _p(dY), B, H, N, M, D, float(scale),
                                      _p(dQ), _p(dK), _p(dZ))
    if rc:
        raise RuntimeError(f"oracle_decode_backward failed ({rc})")
    return dQ, dK, dZ


def flare_backward(Q, K, V, dY, scale: float = 0.0, return_dZ: bool = False):
    """Reverse mode of the FLARE pair Y = Dec(Q, K, Enc(Q, K, V)): the decoder's
    backward gives dZ and its shares of dQ and dK; the encoder's backward
    (App. B.5, dL = 0) takes that dZ and gives dV and the other shares.
    Returns (dQ, dK, dV), plus dZ when ``return_dZ``."""
    _, Z, _ = flare_forward(Q, K, V, scale)
    dQd, dKd, dZ = decode_backward(Q, K, Z, dY, scale)
    dQe, dKe, dV = encode_backward(Q, K, V, dZ, None, scale)
    out = (dQd + dQe, dKd + dKe, dV)
    return out + (dZ,) if return_dZ else out


def flare_pp_backward(Qs, Ks, Vs, Qf, gate, K, V, dY, scale: float = 0.0, shared_vs=None):
    """Reverse mode of the FLARE++ forward (FLARE++ paper, App. B.5, last
    paragraph): the routing pair's backward gives the cotangent dQ of the
    per-batch routing queries (plus dK, dV); the blend Q = Qf + g Qd passes
    dQf = sum_b dQ, dg_h = sum_{b,m,d} dQ Qd and dQd = g dQ; dQd is handed
    once to the synthesis encoder's backward (dL = 0), which gives dQs (summed
    over the batch), dKs and dVs.  With shared synthesis keys and values
    (``shared_vs``, default: Vs is Ks) the value cotangent is added to the
    key cotangent and dVs is returned as None.
    Returns (dQs, dKs, dVs, dQf, dgate, dK, dV)."""
    shared = (Vs is Ks) if shared_vs is None else bool(shared_vs)
    Qs, Ks, Vs, Qf, gate = _f64(Qs), _f64(Ks), _f64(Vs), _f64(Qf), _f64(gate)
    Qd, _ = encode(Qs, Ks, Vs, scale)                       # [B,H,M,D]
    Q = Qf[None] + gate[None, :, None, None] * Qd
    dQ, dK, dV = flare_backward(Q, K, V, dY, scale)
    dQf = dQ.sum(axis=0)
    dgate = np.einsum("bhmd,bhmd->h", dQ, Qd)
    dQd = gate[None, :, None, None] * dQ
    dQs, dKs, dVs = encode_backward(Qs, Ks, Vs, dQd, None, scale)
    if shared:
        return dQs, dKs + dVs, None, dQf, dgate, dK, dV
    return dQs, dKs, dVs, dQf, dgate, dK, dV


def rms_norm_backward(x, dy, alpha=None, eps: float = 1e-6):
    """Reverse mode of rms_norm: given dy, the cotangent of N(x), returns
    (dx, dalpha) (dalpha is None for N_0).  With r = (mean_d x^2 + eps)^(-1/2)
    per row and xh = r x, the forward is N(x) = xh * alpha (App. A.3/A.4), so
        dalpha[h, d] = sum over the rows of head h of dy * xh,
        g = dy * alpha,   dx = r * (g - xh * mean_d(g * xh)),
    the last from d r / d x_j = -r^3 x_j / D.  Written out in fp64."""
    x, dy = _f64(x), _f64(dy)
    if x.shape != dy.shape:
        raise ValueError("x and dy must have one shape")
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xh = x * r
    dalpha = None
    g = dy
    if alpha is not None:
        a = _f64(alpha)
        g = dy * a[:, None, :]
        t = dy * xh                                     # [..., H, rows, D]
        dalpha = t.reshape((-1,) + t.shape[-3:]).sum(axis=(0, 2))
    dx = r * (g - xh * np.mean(g * xh, axis=-1, keepdims=True))
    return dx, dalpha


def flare_pp_backward_normed(Qs, Ks, Vs, Qf, gate, K, V, dY, *, norm_qs=False, norm_ks=False, norm_qf=False,
                             norm_k=False, alpha_qs=None, alpha_ks=None, alpha_k=None, eps: float = 1e-6,
                             scale: float = 0.0):
    """Reverse mode of flare_pp_forward_normed: the FLARE++ backward on the
    normalised inputs (flare_pp_backward), then each norm's backward
    (rms_norm_backward) on the cotangent of its output.  With shared synthesis
    keys and values (Vs is Ks) the values are the normalised keys, so their
    cotangent joins the keys' before the norm's backward.
    Returns (dQs, dKs, dVs, dQf, dgate, dK, dV, dalpha_qs, dalpha_ks, dalpha_k);
    dVs is None when shared, each dalpha is None when its norm has no scale
    or is off."""
    shared = Vs is Ks
    Qs_n = rms_norm(Qs, alpha_qs, eps) if norm_qs else _f64(Qs)
    Ks_n = rms_norm(Ks, alpha_ks, eps) if norm_ks else _f64(Ks)
    Vs_n = Ks_n if shared else _f64(Vs)
    Qf_n = rms_norm(Qf, None, eps) if norm_qf else _f64(Qf)
    K_n = rms_norm(K, alpha_k, eps) if norm_k else _f64(K)
    dQs, dKs, dVs, dQf, dgate, dK, dV = flare_pp_backward(Qs_n, Ks_n, Vs_n, Qf_n, gate, K_n, V, dY, scale,
                                                          shared_vs=shared)
    da_qs = da_ks = da_k = None
    if norm_qs:
        dQs, da_qs = rms_norm_backward(Qs, dQs, alpha_qs, eps)
    if norm_ks:
        dKs, da_ks = rms_norm_backward(Ks, dKs, alpha_ks, eps)
    if norm_qf:
        dQf, _ = rms_norm_backward(Qf, dQf, None, eps)
    if norm_k:
        dK, da_k = rms_norm_backward(K, dK, alpha_k, eps)
    return dQs, dKs, dVs, dQf, dgate, dK, dV, da_qs, da_ks, da_k
