"""ctypes binding of libflare.so (include/flare.h).

Argument marshalling only: every step of the routing forward runs in the HIP
kernels of csrc/flare.hip.  PyTorch supplies device memory (outputs and the
workspace are ``torch.empty`` tensors on the inputs' device) and the current
stream.  There is no fallback: without the built library every call raises.

Layouts (contiguous, D innermost):
  K, V, Ks, Vs, Y : [B, H, N, D]   float32 or bfloat16
  Q, Qs, Qf       : [H, M, D] (shared over the batch) or [B, H, M, D]
  Z               : [B, H, M, D] float32;  L : [B, H, M] float32
  gate            : [H] float32, g_h = sigmoid(gamma_h)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflare.so")

F32, BF16 = 0, 1
OP_ENCODE, OP_DECODE, OP_FORWARD, OP_PP_FORWARD, OP_BACKWARD, OP_ENCODE_BACKWARD, OP_PP_BACKWARD = 0, 1, 2, 3, 4, 5, 6
OP_PP_BACKWARD_NORM = 7
OP_FORWARD_PROJ, OP_PP_FORWARD_PROJ = 8, 9
#: input normalisation flags of flare_pp_forward_norm (include/flare.h)
NORM_QS, NORM_KS, NORM_QF, NORM_K = 1, 2, 4, 8
NORM_FLAREPP = NORM_QS | NORM_KS | NORM_QF | NORM_K  # FLARE++ (Table 2)
NORM_SIMPLIFIED = NORM_QS | NORM_KS                  # simplified FLARE++ (Table 2)
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}

#: every C entry point declared in include/flare.h
SYMBOLS = ("flare_workspace_size", "flare_encode", "flare_decode", "flare_forward", "flare_pp_forward",
           "flare_pp_forward_norm", "flare_backward", "flare_encode_backward", "flare_pp_backward",
           "flare_pp_backward_norm", "flare_status_string", "flare_forward_noalloc", "flare_forward_proj",
           "flare_pp_forward_proj")

_lib = None


class FlareError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libflare.so and declare the C signatures; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m rank_latent_attention_amd.build`")
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.flare_workspace_size.argtypes = [i, i, i, i, i, i, i]
    L.flare_workspace_size.restype = sz
    L.flare_encode.argtypes = [vp, i, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.flare_decode.argtypes = [vp, i, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.flare_forward.argtypes = [vp, i, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.flare_forward_noalloc.argtypes = [vp, i, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.flare_forward_proj.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz, vp]
    L.flare_pp_forward_proj.argtypes = [vp] * 12 + [i] * 7 + [f, i, vp, vp, f, vp, sz, vp]
    L.flare_pp_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.flare_pp_forward_norm.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, vp, vp, f,
                                        vp, sz, vp]
    L.flare_backward.argtypes = [vp, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.flare_encode_backward.argtypes = [vp, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.flare_pp_backward.argtypes = [vp] * 19 + [i, i, i, i, i, i, f, vp, sz, vp]
    L.flare_pp_backward_norm.argtypes = [vp] * 22 + [i, i, i, i, i, i, f, i, vp, vp, vp, f, vp, sz, vp]
    for fn in (L.flare_encode, L.flare_decode, L.flare_forward, L.flare_forward_noalloc, L.flare_forward_proj,
               L.flare_pp_forward_proj, L.flare_pp_forward, L.flare_pp_forward_norm,
               L.flare_backward, L.flare_encode_backward, L.flare_pp_backward, L.flare_pp_backward_norm):
        fn.restype = i
    L.flare_status_string.argtypes = [i]
    L.flare_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(fn: str, rc: int):
    if rc != 0:
        raise FlareError(fn, rc)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dims(Q: torch.Tensor, K: torch.Tensor) -> Tuple[int, int, int, int, int, int]:
    if K.dim() != 4:
        raise ValueError(f"K must be [B,H,N,D], got {tuple(K.shape)}")
    B, H, N, D = K.shape
    if Q.dim() == 3 and Q.shape[0] == H and Q.shape[2] == D:
        return B, H, N, Q.shape[1], D, 0
    if Q.dim() == 4 and Q.shape[0] == B and Q.shape[1] == H and Q.shape[3] == D:
        return B, H, N, Q.shape[2], D, 1
    raise ValueError(f"Q must be [H,M,D] or [B,H,M,D] matching K {tuple(K.shape)}, got {tuple(Q.shape)}")


def _same(ref: torch.Tensor, *ts):
    """Every given tensor is a contiguous GPU tensor on ref's device (the
    kernels take raw device pointers: a host or foreign-device pointer would
    be dereferenced on the GPU)."""
    for t in (ref,) + ts:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"expected a torch.Tensor, got {type(t).__name__}")
        if t.device != ref.device:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if ref.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {ref.device}")


def _out(name: str, t: Optional[torch.Tensor], shape, dtype: torch.dtype):
    """A caller-supplied output must have exactly the shape and dtype the
    kernels write (they get no sizes and would write past a smaller one)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _ws_bytes(ws: Optional[torch.Tensor]) -> int:
    """Byte size of a caller-supplied workspace (any dtype, contiguous)."""
    if ws is None:
        return 0
    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"ws must be a torch.Tensor, got {type(ws).__name__}")
    return ws.numel() * ws.element_size()


def _pp_outs(K: torch.Tensor, M: int, Y, Q_out, Z, L):
    B, H, N, D = K.shape
    _out("Y", Y, K.shape, K.dtype)
    _out("Q_out", Q_out, (B, H, M, D), torch.float32)
    _out("Z", Z, (B, H, M, D), torch.float32)
    _out("L", L, (B, H, M), torch.float32)


def workspace_size(op: int, B: int, H: int, N: int, M: int, D: int, dtype: int) -> int:
    return int(load().flare_workspace_size(op, B, H, N, M, D, dtype))


def workspace(op: int, B: int, H: int, N: int, M: int, D: int, dtype: int, device) -> Optional[torch.Tensor]:
    n = workspace_size(op, B, H, N, M, D, dtype)
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def flare_encode(Q, K, V, scale: float = 0.0, Z=None, L=None, ws=None):
    """Z = SDPA(Q, K, V) and its natural-log normaliser L; returns (Z, L)."""
    B, H, N, M, D, qb = _dims(Q, K)
    dt = _dtype_code(K)
    if Q.dtype != K.dtype or V.dtype != K.dtype or V.shape != K.shape:
        raise ValueError("Q, K, V must share dtype and K, V shape")
    _out("Z", Z, (B, H, M, D), torch.float32)
    _out("L", L, (B, H, M), torch.float32)
    _same(K, Q, V, Z, L, ws)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=K.device) if Z is None else Z
    L = torch.empty((B, H, M), dtype=torch.float32, device=K.device) if L is None else L
    ws = workspace(OP_ENCODE, B, H, N, M, D, dt, K.device) if ws is None else ws
    rc = load().flare_encode(_ptr(Q), qb, _ptr(K), _ptr(V), _ptr(Z), _ptr(L), B, H, N, M, D, dt, float(scale),
                             _ptr(ws), _ws_bytes(ws), _stream(K.device))
    _check("flare_encode", rc)
    return Z, L


def flare_decode(Q, K, Z, scale: float = 0.0, Y=None):
    """Y = SDPA(K, Q, Z): every token attends over the latents."""
    B, H, N, M, D, qb = _dims(Q, K)
    dt = _dtype_code(K)
    if Q.dtype != K.dtype or Z.dtype != torch.float32 or tuple(Z.shape) != (B, H, M, D):
        raise ValueError("Q must match K's dtype and Z must be float32 [B,H,M,D]")
    _out("Y", Y, K.shape, K.dtype)
    _same(K, Q, Z, Y)
    Y = torch.empty_like(K) if Y is None else Y
    rc = load().flare_decode(_ptr(Q), qb, _ptr(K), _ptr(Z), _ptr(Y), B, H, N, M, D, dt, float(scale), None, 0,
                             _stream(K.device))
    _check("flare_decode", rc)
    return Y


def flare_forward(Q, K, V, scale: float = 0.0, Y=None, Z=None, L=None, ws=None):
    """FLARE routing forward Y = SDPA(K, Q, SDPA(Q, K, V)); returns (Y, Z, L).

    Z and L are returned only when passed in (they are written into the given
    tensors); otherwise they live in the workspace and (Y, None, None) is returned.
    """
    B, H, N, M, D, qb = _dims(Q, K)
    dt = _dtype_code(K)
    if Q.dtype != K.dtype or V.dtype != K.dtype or V.shape != K.shape:
        raise ValueError("Q, K, V must share dtype and K, V shape")
    _out("Y", Y, K.shape, K.dtype)
    _out("Z", Z, (B, H, M, D), torch.float32)
    _out("L", L, (B, H, M), torch.float32)
    _same(K, Q, V, Y, Z, L, ws)
    Y = torch.empty_like(K) if Y is None else Y
    ws = workspace(OP_FORWARD, B, H, N, M, D, dt, K.device) if ws is None else ws
    rc = load().flare_forward(_ptr(Q), qb, _ptr(K), _ptr(V), _ptr(Y), _ptr(Z), _ptr(L), B, H, N, M, D, dt,
                              float(scale), _ptr(ws), _ws_bytes(ws), _stream(K.device))
    _check("flare_forward", rc)
    return Y, Z, L


def flare_forward_noalloc(Q, K, V, scale: float = 0.0, Y=None, Z=None, L=None):
    """flare_forward with the library's per-GPU scratch array instead of a
    workspace (flare_forward_noalloc in include/flare.h): the C call allocates
    nothing.  Pass Y (and Z, L) to keep this wrapper allocation-free too.
    Calls that overlap on one GPU race.  Returns (Y, Z, L)."""
    B, H, N, M, D, qb = _dims(Q, K)
    dt = _dtype_code(K)
    if Q.dtype != K.dtype or V.dtype != K.dtype or V.shape != K.shape:
        raise ValueError("Q, K, V must share dtype and K, V shape")
    _out("Y", Y, K.shape, K.dtype)
    _out("Z", Z, (B, H, M, D), torch.float32)
    _out("L", L, (B, H, M), torch.float32)
    _same(K, Q, V, Y, Z, L)
    Y = torch.empty_like(K) if Y is None else Y
    rc = load().flare_forward_noalloc(_ptr(Q), qb, _ptr(K), _ptr(V), _ptr(Y), _ptr(Z), _ptr(L), B, H, N, M, D, dt,
                                      float(scale), _stream(K.device))
    _check("flare_forward_noalloc", rc)
    return Y, Z, L


def _proj_dims(X, W, name="WK"):
    if X.dim() != 3:
        raise ValueError(f"X must be [B,N,C], got {tuple(X.shape)}")
    if W.dim() != 3 or W.shape[1] != X.shape[2]:
        raise ValueError(f"{name} must be [H,C,D] with C = {X.shape[2]}, got {tuple(W.shape)}")
    B, N, C = X.shape
    H, _, D = W.shape
    return B, H, N, D, C


def flare_forward_proj(X, WK, WV, Q, scale: float = 0.0, Y=None, K_out=None, Z=None, L=None, ws=None):
    """FLARE routing forward from the block input (flare_forward_proj in
    include/flare.h): K = X WK, V = X WV per head inside the encode, then the
    FLARE pair.  X [B,N,C], WK, WV [H,C,D], Q [H,M,D] or [B,H,M,D], all bf16.
    Returns (Y, K_out, Z, L); the last three only when passed in."""
    B, H, N, D, C = _proj_dims(X, WK)
    if WV.shape != WK.shape:
        raise ValueError("WV must have WK's shape")
    if Q.dim() == 3 and Q.shape[0] == H and Q.shape[2] == D:
        M, qb = Q.shape[1], 0
    elif Q.dim() == 4 and Q.shape[0] == B and Q.shape[1] == H and Q.shape[3] == D:
        M, qb = Q.shape[2], 1
    else:
        raise ValueError(f"Q must be [H,M,D] or [B,H,M,D] with H={H}, D={D}, got {tuple(Q.shape)}")
    for t in (X, WK, WV, Q):
        if t.dtype != torch.bfloat16:
            raise ValueError("X, WK, WV and Q must be bfloat16")
    _out("Y", Y, (B, H, N, D), torch.bfloat16)
    _out("K_out", K_out, (B, H, N, D), torch.bfloat16)
    _out("Z", Z, (B, H, M, D), torch.float32)
    _out("L", L, (B, H, M), torch.float32)
    _same(X, WK, WV, Q, Y, K_out, Z, L, ws)
    Y = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=X.device) if Y is None else Y
    ws = workspace(OP_FORWARD_PROJ, B, H, N, M, D, BF16, X.device) if ws is None else ws
    rc = load().flare_forward_proj(_ptr(X), _ptr(WK), _ptr(WV), _ptr(Q), qb, _ptr(Y), _ptr(K_out), _ptr(Z), _ptr(L),
                                   B, H, N, M, D, C, BF16, float(scale), _ptr(ws), _ws_bytes(ws), _stream(X.device))
    _check("flare_forward_proj", rc)
    return Y, K_out, Z, L


def flare_pp_forward_proj(X, WKs, WK, WV, Qs, Qf, gate, norm_flags: int, alpha_qs=None, alpha_k=None,
                          eps: float = 1e-6, scale: float = 0.0, Y=None, Q_out=None, K_out=None, Z=None, L=None,
                          ws=None):
    """FLARE++ routing forward from the block input (flare_pp_forward_proj in
    include/flare.h): synthesis keys (= values) X WKs, routing keys X WK and
    values X WV per head, the Table 2 norms of norm_flags (alpha_qs, alpha_k
    float32 [H,D] or None), then FLARE++.  Returns (Y, Q_out, K_out, Z, L)."""
    B, H, N, D, C = _proj_dims(X, WK)
    if WV.shape != WK.shape or WKs.shape != WK.shape:
        raise ValueError("WKs, WK, WV must share one shape [H,C,D]")
    if Qs.dim() != 3 or Qs.shape[0] != H or Qs.shape[2] != D or Qf.shape != Qs.shape:
        raise ValueError("Qs and Qf must be [H,M,D]")
    M = Qs.shape[1]
    for t in (X, WKs, WK, WV, Qs, Qf):
        if t.dtype != torch.bfloat16:
            raise ValueError("X, WKs, WK, WV, Qs and Qf must be bfloat16")
    if gate.dtype != torch.float32 or gate.numel() != H:
        raise ValueError("gate must be float32 [H]")
    for a in (alpha_qs, alpha_k):
        if a is not None and (a.dtype != torch.float32 or tuple(a.shape) != (H, D)):
            raise ValueError("alpha arrays must be float32 [H, D]")
    _out("Y", Y, (B, H, N, D), torch.bfloat16)
    _out("Q_out", Q_out, (B, H, M, D), torch.float32)
    _out("K_out", K_out, (B, H, N, D), torch.bfloat16)
    _out("Z", Z, (B, H, M, D), torch.float32)
    _out("L", L, (B, H, M), torch.float32)
    _same(X, WKs, WK, WV, Qs, Qf, gate, Y, Q_out, K_out, Z, L, alpha_qs, alpha_k, ws)
    Y = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=X.device) if Y is None else Y
    ws = workspace(OP_PP_FORWARD_PROJ, B, H, N, M, D, BF16, X.device) if ws is None else ws
    rc = load().flare_pp_forward_proj(_ptr(X), _ptr(WKs), _ptr(WK), _ptr(WV), _ptr(Qs), _ptr(Qf), _ptr(gate), _ptr(Y),
                                      _ptr(Q_out), _ptr(K_out), _ptr(Z), _ptr(L), B, H, N, M, D, C, BF16,
                                      float(scale), int(norm_flags), _ptr(alpha_qs), _ptr(alpha_k), float(eps),
                                      _ptr(ws), _ws_bytes(ws), _stream(X.device))
    _check("flare_pp_forward_proj", rc)
    return Y, Q_out, K_out, Z, L


def flare_pp_forward(Qs, Ks, Vs, Qf, gate, K, V, scale: float = 0.0, Y=None, Q_out=None, Z=None, L=None, ws=None):
    """FLARE++ routing forward; returns (Y, Q_out, Z, L) (the last three only when passed in)."""
    if K.dim() != 4:
        raise ValueError("K must be [B,H,N,D]")
    B, H, N, D = K.shape
    if Qs.dim() != 3 or Qs.shape[0] != H or Qs.shape[2] != D or Qf.shape != Qs.shape:
        raise ValueError("Qs and Qf must be [H,M,D]")
    M = Qs.shape[1]
    dt = _dtype_code(K)
    for t in (Qs, Ks, Vs, Qf, V):
        if t.dtype != K.dtype:
            raise ValueError("Qs, Ks, Vs, Qf, K, V must share one dtype")
    if Ks.shape != K.shape or Vs.shape != K.shape or V.shape != K.shape:
        raise ValueError("Ks, Vs, K, V must all be [B,H,N,D]")
    if gate.dtype != torch.float32 or gate.numel() != H:
        raise ValueError("gate must be float32 [H]")
    _pp_outs(K, M, Y, Q_out, Z, L)
    _same(K, Qs, Ks, Vs, Qf, gate, V, Y, Q_out, Z, L, ws)
    Y = torch.empty_like(K) if Y is None else Y
    ws = workspace(OP_PP_FORWARD, B, H, N, M, D, dt, K.device) if ws is None else ws
    rc = load().flare_pp_forward(_ptr(Qs), _ptr(Ks), _ptr(Vs), _ptr(Qf), _ptr(gate), _ptr(K), _ptr(V), _ptr(Y),
                                 _ptr(Q_out), _ptr(Z), _ptr(L), B, H, N, M, D, dt, float(scale), _ptr(ws),
                                 _ws_bytes(ws), _stream(K.device))
    _check("flare_pp_forward", rc)
    return Y, Q_out, Z, L


def flare_pp_forward_norm(Qs, Ks, Vs, Qf, gate, K, V, norm_flags: int, alpha_qs=None, alpha_ks=None, alpha_k=None,
                          eps: float = 1e-6, scale: float = 0.0, Y=None, Q_out=None, Z=None, L=None, ws=None):
    """FLARE++ routing forward with the per-head RMS norms of the flags fused
    into the kernels (flare_pp_forward_norm in include/flare.h); alpha_* are
    float32 [H, D] or None.  Returns (Y, Q_out, Z, L)."""
    if K.dim() != 4:
        raise ValueError("K must be [B,H,N,D]")
    B, H, N, D = K.shape
    if Qs.dim() != 3 or Qs.shape[0] != H or Qs.shape[2] != D or Qf.shape != Qs.shape:
        raise ValueError("Qs and Qf must be [H,M,D]")
    M = Qs.shape[1]
    dt = _dtype_code(K)
    for t in (Qs, Ks, Vs, Qf, V):
        if t.dtype != K.dtype:
            raise ValueError("Qs, Ks, Vs, Qf, K, V must share one dtype")
    if Ks.shape != K.shape or Vs.shape != K.shape or V.shape != K.shape:
        raise ValueError("Ks, Vs, K, V must all be [B,H,N,D]")
    if gate.dtype != torch.float32 or gate.numel() != H:
        raise ValueError("gate must be float32 [H]")
    for a in (alpha_qs, alpha_ks, alpha_k):
        if a is not None and (a.dtype != torch.float32 or tuple(a.shape) != (H, D)):
            raise ValueError("alpha arrays must be float32 [H, D]")
    _pp_outs(K, M, Y, Q_out, Z, L)
    _same(K, Qs, Ks, Vs, Qf, gate, V, Y, Q_out, Z, L, alpha_qs, alpha_ks, alpha_k, ws)
    Y = torch.empty_like(K) if Y is None else Y
    ws = workspace(OP_PP_FORWARD, B, H, N, M, D, dt, K.device) if ws is None else ws
    rc = load().flare_pp_forward_norm(_ptr(Qs), _ptr(Ks), _ptr(Vs), _ptr(Qf), _ptr(gate), _ptr(K), _ptr(V), _ptr(Y),
                                      _ptr(Q_out), _ptr(Z), _ptr(L), B, H, N, M, D, dt, float(scale), int(norm_flags),
                                      _ptr(alpha_qs), _ptr(alpha_ks), _ptr(alpha_k), float(eps), _ptr(ws),
                                      _ws_bytes(ws), _stream(K.device))
    _check("flare_pp_forward_norm", rc)
    return Y, Q_out, Z, L


def _grads(Q, K, dQ, dK, dV):
    _out("dQ", dQ, Q.shape, torch.float32)
    _out("dK", dK, K.shape, K.dtype)
    _out("dV", dV, K.shape, K.dtype)
    dQ = torch.empty(Q.shape, dtype=torch.float32, device=K.device) if dQ is None else dQ
    dK = torch.empty_like(K) if dK is None else dK
    dV = torch.empty_like(K) if dV is None else dV
    return dQ, dK, dV


def flare_backward(Q, K, V, Z, L, dY, scale: float = 0.0, dQ=None, dK=None, dV=None, dZ=None, ws=None):
    """Backward of the FLARE pair (flare_backward in include/flare.h): given
    the forward's Z [B,H,M,D] and L [B,H,M] (float32) and the output
    cotangent dY, returns (dQ, dK, dV, dZ); dQ is float32 in Q's layout,
    dK and dV in K's dtype (bf16 or float32); dZ only when passed in."""
    B, H, N, M, D, qb = _dims(Q, K)
    dt = _dtype_code(K)
    if Q.dtype != K.dtype or V.dtype != K.dtype or dY.dtype != K.dtype or V.shape != K.shape or dY.shape != K.shape:
        raise ValueError("Q, K, V, dY must share dtype and K, V, dY shape")
    if Z.dtype != torch.float32 or tuple(Z.shape) != (B, H, M, D) or L.dtype != torch.float32 or \
            tuple(L.shape) != (B, H, M):
        raise ValueError("Z must be float32 [B,H,M,D] and L float32 [B,H,M]")
    _out("dZ", dZ, (B, H, M, D), torch.float32)
    _same(K, Q, V, Z, L, dY, dQ, dK, dV, dZ, ws)
    dQ, dK, dV = _grads(Q, K, dQ, dK, dV)
    ws = workspace(OP_BACKWARD, B, H, N, M, D, dt, K.device) if ws is None else ws
    rc = load().flare_backward(_ptr(Q), qb, _ptr(K), _ptr(V), _ptr(Z), _ptr(L), _ptr(dY), _ptr(dQ), _ptr(dK),
                               _ptr(dV), _ptr(dZ), B, H, N, M, D, dt, float(scale), _ptr(ws),
                               _ws_bytes(ws), _stream(K.device))
    _check("flare_backward", rc)
    return dQ, dK, dV, dZ


def flare_encode_backward(Q, K, V, Z, L, dZ, dL=None, scale: float = 0.0, dQ=None, dK=None, dV=None, ws=None):
    """Backward of the encoder (flare_encode_backward in include/flare.h):
    given its outputs Z, L and their cotangents dZ, dL (float32; dL may be
    None), returns (dQ, dK, dV)."""
    B, H, N, M, D, qb = _dims(Q, K)
    dt = _dtype_code(K)
    if Q.dtype != K.dtype or V.dtype != K.dtype or V.shape != K.shape:
        raise ValueError("Q, K, V must share dtype and K, V shape")
    for t, shp in ((Z, (B, H, M, D)), (L, (B, H, M)), (dZ, (B, H, M, D)), (dL, (B, H, M))):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shp):
            raise ValueError("Z, dZ must be float32 [B,H,M,D]; L, dL float32 [B,H,M]")
    _same(K, Q, V, Z, L, dZ, dL, dQ, dK, dV, ws)
    dQ, dK, dV = _grads(Q, K, dQ, dK, dV)
    ws = workspace(OP_ENCODE_BACKWARD, B, H, N, M, D, dt, K.device) if ws is None else ws
    rc = load().flare_encode_backward(_ptr(Q), qb, _ptr(K), _ptr(V), _ptr(Z), _ptr(L), _ptr(dZ), _ptr(dL),
                                      _ptr(dQ), _ptr(dK), _ptr(dV), B, H, N, M, D, dt, float(scale), _ptr(ws),
                                      _ws_bytes(ws), _stream(K.device))
    _check("flare_encode_backward", rc)
    return dQ, dK, dV


def flare_pp_backward(Qs, Ks, Vs, Qf, gate, K, V, Q, Z, L, dY, scale: float = 0.0, dQ_out=None, ws=None):
    """Backward of the FLARE++ forward (flare_pp_backward in include/flare.h).
    Q, Z, L are the forward's routing queries (its Q_out), latents and
    log-normalisers for the same inputs.  Returns
    (dQs, dKs, dVs, dQf, dgate, dK, dV, dQ_out); dVs is None when Vs is Ks
    (its cotangent is then added into dKs), dQ_out only when passed in."""
    if K.dim() != 4:
        raise ValueError("K must be [B,H,N,D]")
    B, H, N, D = K.shape
    if Qs.dim() != 3 or Qs.shape[0] != H or Qs.shape[2] != D or Qf.shape != Qs.shape:
        raise ValueError("Qs and Qf must be [H,M,D]")
    M = Qs.shape[1]
    dt = _dtype_code(K)
    for t in (Qs, Ks, Vs, Qf, V, dY):
        if t.dtype != K.dtype:
            raise ValueError("Qs, Ks, Vs, Qf, K, V, dY must share one dtype")
    if Ks.shape != K.shape or Vs.shape != K.shape or V.shape != K.shape or dY.shape != K.shape:
        raise ValueError("Ks, Vs, K, V, dY must all be [B,H,N,D]")
    if gate.dtype != torch.float32 or gate.numel() != H:
        raise ValueError("gate must be float32 [H]")
    for t, shp in ((Q, (B, H, M, D)), (Z, (B, H, M, D)), (L, (B, H, M))):
        if t.dtype != torch.float32 or tuple(t.shape) != shp:
            raise ValueError("Q, Z must be float32 [B,H,M,D] and L float32 [B,H,M]")
    alias = Vs.data_ptr() == Ks.data_ptr()
    dev = K.device
    dQs = torch.empty((H, M, D), dtype=torch.float32, device=dev)
    dQf = torch.empty((H, M, D), dtype=torch.float32, device=dev)
    dgate = torch.empty((H,), dtype=torch.float32, device=dev)
    dKs, dK, dV = torch.empty_like(K), torch.empty_like(K), torch.empty_like(K)
    dVs = None if alias else torch.empty_like(K)
    _out("dQ_out", dQ_out, (B, H, M, D), torch.float32)
    _same(K, Qs, Ks, Vs, Qf, gate, V, Q, Z, L, dY, dQ_out, ws)
    ws = workspace(OP_PP_BACKWARD, B, H, N, M, D, dt, dev) if ws is None else ws
    rc = load().flare_pp_backward(_ptr(Qs), _ptr(Ks), _ptr(Vs), _ptr(Qf), _ptr(gate), _ptr(K), _ptr(V), _ptr(Q),
                                  _ptr(Z), _ptr(L), _ptr(dY), _ptr(dQs), _ptr(dKs), _ptr(dVs), _ptr(dQf),
                                  _ptr(dgate), _ptr(dQ_out), _ptr(dK), _ptr(dV), B, H, N, M, D, dt, float(scale),
                                  _ptr(ws), _ws_bytes(ws), _stream(dev))
    _check("flare_pp_backward", rc)
    return dQs, dKs, dVs, dQf, dgate, dK, dV, dQ_out


def flare_pp_backward_norm(Qs, Ks, Vs, Qf, gate, K, V, Q, Z, L, dY, norm_flags: int, alpha_qs=None, alpha_ks=None,
                           alpha_k=None, eps: float = 1e-6, scale: float = 0.0, dQ_out=None, ws=None):
    """Backward of flare_pp_forward_norm (flare_pp_backward_norm in include/flare.h):
    cotangents of the raw inputs and of the norms' channel scales.  Q, Z, L are
    that forward's routing queries, latents and log-normalisers.  Returns
    (dQs, dKs, dVs, dQf, dgate, dK, dV, dalpha_qs, dalpha_ks, dalpha_k, dQ_out);
    dVs is None when Vs is Ks, each dalpha None unless its scale is given and
    its flag set."""
    if K.dim() != 4:
        raise ValueError("K must be [B,H,N,D]")
    B, H, N, D = K.shape
    if Qs.dim() != 3 or Qs.shape[0] != H or Qs.shape[2] != D or Qf.shape != Qs.shape:
        raise ValueError("Qs and Qf must be [H,M,D]")
    M = Qs.shape[1]
    dt = _dtype_code(K)
    for t in (Qs, Ks, Vs, Qf, V, dY):
        if t.dtype != K.dtype:
            raise ValueError("Qs, Ks, Vs, Qf, K, V, dY must share one dtype")
    if Ks.shape != K.shape or Vs.shape != K.shape or V.shape != K.shape or dY.shape != K.shape:
        raise ValueError("Ks, Vs, K, V, dY must all be [B,H,N,D]")
    if gate.dtype != torch.float32 or gate.numel() != H:
        raise ValueError("gate must be float32 [H]")
    for t, shp in ((Q, (B, H, M, D)), (Z, (B, H, M, D)), (L, (B, H, M))):
        if t.dtype != torch.float32 or tuple(t.shape) != shp:
            raise ValueError("Q, Z must be float32 [B,H,M,D] and L float32 [B,H,M]")
    for a in (alpha_qs, alpha_ks, alpha_k):
        if a is not None and (a.dtype != torch.float32 or tuple(a.shape) != (H, D)):
            raise ValueError("alpha arrays must be float32 [H, D]")
    alias = Vs.data_ptr() == Ks.data_ptr()
    dev = K.device
    dQs = torch.empty((H, M, D), dtype=torch.float32, device=dev)
    dQf = torch.empty((H, M, D), dtype=torch.float32, device=dev)
    dgate = torch.empty((H,), dtype=torch.float32, device=dev)
    dKs, dK, dV = torch.empty_like(K), torch.empty_like(K), torch.empty_like(K)
    dVs = None if alias else torch.empty_like(K)

    def da(a, bit):
        return torch.empty((H, D), dtype=torch.float32, device=dev) if a is not None and norm_flags & bit else None
    da_qs, da_ks, da_k = da(alpha_qs, NORM_QS), da(alpha_ks, NORM_KS), da(alpha_k, NORM_K)
    _out("dQ_out", dQ_out, (B, H, M, D), torch.float32)
    _same(K, Qs, Ks, Vs, Qf, gate, V, Q, Z, L, dY, dQ_out, alpha_qs, alpha_ks, alpha_k, ws)
    ws = workspace(OP_PP_BACKWARD_NORM, B, H, N, M, D, dt, dev) if ws is None else ws
    rc = load().flare_pp_backward_norm(_ptr(Qs), _ptr(Ks), _ptr(Vs), _ptr(Qf), _ptr(gate), _ptr(K), _ptr(V), _ptr(Q),
                                       _ptr(Z), _ptr(L), _ptr(dY), _ptr(dQs), _ptr(dKs), _ptr(dVs), _ptr(dQf),
                                       _ptr(dgate), _ptr(dQ_out), _ptr(dK), _ptr(dV), _ptr(da_qs), _ptr(da_ks),
                                       _ptr(da_k), B, H, N, M, D, dt, float(scale), int(norm_flags), _ptr(alpha_qs),
                                       _ptr(alpha_ks), _ptr(alpha_k), float(eps), _ptr(ws),
                                       _ws_bytes(ws), _stream(dev))
    _check("flare_pp_backward_norm", rc)
    return dQs, dKs, dVs, dQf, dgate, dK, dV, da_qs, da_ks, da_k, dQ_out
