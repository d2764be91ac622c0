"""Seeded synthetic inputs for the FLARE / FLARE++ routing operator.

This module only *draws* inputs: token keys K, values V, latent queries Q and,
for FLARE++, the synthesis seeds, synthesis keys/values, fixed queries and
gates.  It contains none of the routing arithmetic (no attention, no softmax,
no merge); both the fp64 oracle and the GPU path consume exactly the arrays
returned here.

Recipes follow the workload descriptions of the five benchmark shapes, which
stand in for the datasets named by the FLARE++ paper ("FLARE++: Low-rank
attention with attention-synthesized routing", Table 6 in App. C.1: Pipe
129x129, Darcy 85x85, DrivAerML; the million-token runs of Sec. 5.2 / D.3).
Readings of under-specified steps:

* ``N(0, s2)`` reads its second argument as a variance.
* Per-head RMS normalisation N0 (paper Table 2, App. A.7) is applied here, in
  float64, to the tensors the FLARE++ block normalises (synthesis seeds and
  keys, fixed queries, routing keys).  It is upstream of the routing boundary,
  so both sides see the same normalised values; eps = 1e-6.
* Everything is generated in float64, rounded to float32 (round to nearest
  even) and, for bf16 workloads, rounded again to bf16 (RNE).  Arrays are
  returned as float32 arrays whose values are exactly representable in the
  workload dtype.
* One ``numpy.random.Generator`` (PCG64) per named tensor, seeded with
  ``SeedSequence([seed, tag])`` so each tensor's stream is independent of the
  order in which tensors are drawn.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

RMS_EPS = 1e-6
GATE_LOGIT = 0.25  # paper App. A.4 / Table 2: gate logits start at 0.25

_TAGS = {
    "q": 1, "k": 2, "v": 3, "x": 4, "wk": 5, "wv": 6, "noise": 7, "lift": 8,
    "pts": 9, "omega": 10, "ids": 11, "emb": 12, "qs": 13, "qf": 14, "wks": 15,
    "vs": 16, "wvs": 17, "ks": 18, "qs_mag": 19, "ks_mag": 20, "k_mag": 21, "qf_mag": 22,
    "alpha_qs": 23, "alpha_ks": 24, "alpha_k": 25, "dy": 26, "dz": 27, "dl": 28,
}


def _rng(seed: int, tag: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), _TAGS[tag]])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (round to nearest even) and return float32.

    The input is first rounded to float32 (numpy's astype is RNE), then the
    low 16 bits of the float32 pattern are rounded away (RNE on the 16th bit).
    Inputs must be finite.
    """
    f = np.array(x, dtype=np.float32, order="C", copy=True)
    u = f.view(np.uint32)
    lsb = (u >> 16) & 1
    # finite patterns are at most 0xFF7FFFFF: adding 0x8000 stays below 2^32
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return f


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def rms_norm(x: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Per-row RMS normalisation over the last axis, no learned scale (N0)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


@dataclasses.dataclass
class Workload:
    """One routing-forward problem.

    FLARE:   Q [H,M,D] (shared over the batch), K, V [B,H,N,D].
    FLARE++: additionally Qs (synthesis seeds) [H,M,D], Ks [B,H,N,D],
             Vs [B,H,N,D] (``Vs is Ks`` when the block shares them),
             Qf (fixed queries) [H,M,D] and gate [H] (= sigmoid(gamma)).
    Raw FLARE++ (norm_flags != 0): the inputs are not normalised; the
             forward applies the per-head RMS norms of the flags (values as
             the library's FLARE_NORM_* bits) with the learned channel
             scales alpha_qs, alpha_ks, alpha_k [H,D] (None = no scale).
    """

    name: str
    B: int
    H: int
    N: int
    M: int
    D: int
    dtype: str  # "f32" or "bf16"
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    pp: bool = False
    Qs: Optional[np.ndarray] = None
    Ks: Optional[np.ndarray] = None
    Vs: Optional[np.ndarray] = None
    Qf: Optional[np.ndarray] = None
    gate: Optional[np.ndarray] = None
    scale: float = 0.0  # <= 0 means 1/sqrt(D)
    recipe: str = ""
    norm_flags: int = 0
    alpha_qs: Optional[np.ndarray] = None
    alpha_ks: Optional[np.ndarray] = None
    alpha_k: Optional[np.ndarray] = None
    # block input and per-head projections (the fused-projection forwards):
    # X [B,N,C]; WK, WV, WKs [H,C,D]; K, V (and Ks) are then X @ W per head
    X: Optional[np.ndarray] = None
    WK: Optional[np.ndarray] = None
    WV: Optional[np.ndarray] = None
    WKs: Optional[np.ndarray] = None

    @property
    def shared_vs(self) -> bool:
        return self.pp and self.Vs is self.Ks

    def arrays(self) -> Dict[str, np.ndarray]:
        out = {"Q": self.Q, "K": self.K, "V": self.V}
        if self.pp:
            out.update(Qs=self.Qs, Ks=self.Ks, Vs=self.Vs, Qf=self.Qf, gate=self.gate)
        return out


def _gauss(seed, tag, shape, std=1.0):
    return _rng(seed, tag).standard_normal(size=shape) * std


def _heads(X: np.ndarray, W: np.ndarray, H: int, D: int) -> np.ndarray:
    """X [B,N,C] times per-head W [C, H*D] / sqrt(C) -> [B,H,N,D]."""
    B, N, C = X.shape
    Y = (X.reshape(B * N, C) @ W) / math.sqrt(C)
    return np.ascontiguousarray(Y.reshape(B, N, H, D).transpose(0, 2, 1, 3))


def _rff(points: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """Random Fourier features [cos(2 pi w.p), sin(2 pi w.p)] -> [..., 2F]."""
    ang = 2.0 * np.pi * (points @ omega.T)
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=-1)


def make_gaussian(B, H, N, M, D, dtype="f32", seed=0, q_std=None, kv_std=1.0, name="gaussian"):
    """K, V ~ N(0, kv_std^2) i.i.d., Q ~ N(0, 1/D) (or N(0, q_std^2))."""
    q_std = 1.0 / math.sqrt(D) if q_std is None else q_std
    Q = to_dtype(_gauss(seed, "q", (H, M, D), q_std), dtype)
    K = to_dtype(_gauss(seed, "k", (B, H, N, D), kv_std), dtype)
    V = to_dtype(_gauss(seed, "v", (B, H, N, D), kv_std), dtype)
    return Workload(name, B, H, N, M, D, dtype, Q, K, V,
                    recipe=f"K,V~N(0,{kv_std}^2); Q~N(0,{q_std:.4g}^2); seed {seed}")


def make_gaussian_pp(B, H, N, M, D, dtype="bf16", seed=0, share_vs=True, gate=None, name="gaussian_pp"):
    """FLARE++ inputs with Gaussian tokens; norms as in the FLARE++ block."""
    base = make_gaussian(B, H, N, M, D, dtype, seed, name=name)
    Ks = to_dtype(rms_norm(_gauss(seed, "wks", (B, H, N, D))), dtype)
    Vs = Ks if share_vs else to_dtype(_gauss(seed, "vs", (B, H, N, D)), dtype)
    Qs = to_dtype(rms_norm(_gauss(seed, "qs", (H, M, D), 1.0 / math.sqrt(D))), dtype)
    Qf = to_dtype(rms_norm(_gauss(seed, "qf", (H, M, D), 1.0 / math.sqrt(D))), dtype)
    K = to_dtype(rms_norm(base.K.astype(np.float64)), dtype)
    g = np.full((H,), 1.0 / (1.0 + math.exp(-GATE_LOGIT)), dtype=np.float32) if gate is None \
        else np.asarray(gate, dtype=np.float32).reshape(H)
    return dataclasses.replace(base, K=K, pp=True, Qs=Qs, Ks=Ks, Vs=Vs, Qf=Qf, gate=g,
                               recipe=base.recipe + "; FLARE++: Ks=N0(N(0,1)), Qs,Qf=N0(N(0,1/D)), K=N0(K)")


def channel_scales(seed, tag, H, D, std=0.1) -> np.ndarray:
    """Per-head learned channel scales of an RMS norm: 1 + N(0, std^2), float32 [H, D]."""
    return (1.0 + _gauss(seed, tag, (H, D), std)).astype(np.float32)


def make_gaussian_pp_raw(B, H, N, M, D, dtype="bf16", seed=0, variant="flarepp", name="gaussian_pp_raw"):
    """Un-normalised FLARE++ inputs for the fused-norm forward.

    variant "flarepp": Vs is Ks; norms on Qs (N_a), Ks (N_0), Qf (N_0) and
    K (N_a), flags 15.  variant "simplified": a separate Vs; norms on Qs and
    Ks (both N_a), flags 3; Qf = 0 and gate = 1 so the routing query is the
    synthesised one.  Row magnitudes are spread (log-normal, sigma 0.5, per
    row) so the norms change every row, while the raw scores stay moderate;
    the learned channel scales are 1 + N(0, 0.1^2).
    """
    def rows(tag, shape, std):  # Gaussian rows with a per-row log-normal magnitude
        x = _gauss(seed, tag, shape, std)
        return x * np.exp(_gauss(seed, tag + "_mag", shape[:-1] + (1,), 0.5))
    Qs = to_dtype(rows("qs", (H, M, D), 0.6), dtype)
    Ks = to_dtype(rows("ks", (B, H, N, D), 0.7), dtype)
    K = to_dtype(rows("k", (B, H, N, D), 0.7), dtype)
    V = to_dtype(_gauss(seed, "v", (B, H, N, D)), dtype)
    if variant == "flarepp":
        Vs = Ks
        Qf = to_dtype(rows("qf", (H, M, D), 0.5), dtype)
        g = np.full((H,), 1.0 / (1.0 + math.exp(-GATE_LOGIT)), dtype=np.float32)
        flags, aks, ak = 15, None, channel_scales(seed, "alpha_k", H, D)
    elif variant == "simplified":
        Vs = to_dtype(_gauss(seed, "vs", (B, H, N, D), 1.3), dtype)
        Qf = to_dtype(np.zeros((H, M, D)), dtype)
        g = np.ones((H,), dtype=np.float32)
        flags, aks, ak = 3, channel_scales(seed, "alpha_ks", H, D), None
    else:
        raise ValueError(f"unknown variant {variant!r}")
    return Workload(name, B, H, N, M, D, dtype, Q=Qf, K=K, V=V, pp=True, Qs=Qs, Ks=Ks, Vs=Vs, Qf=Qf, gate=g,
                    norm_flags=flags, alpha_qs=channel_scales(seed, "alpha_qs", H, D), alpha_ks=aks, alpha_k=ak,
                    recipe=f"raw FLARE++ ({variant}): rows N(0, s^2) x lognormal(0, 0.5) magnitude, "
                           f"alpha = 1 + N(0, 0.01); seed {seed}")


# ---------------------------------------------------------------------------
# The five benchmark workloads.
# ---------------------------------------------------------------------------

def config1(seed=1):
    """Single-head FLARE, fp32: B1 H1 N1024 M32 D16, K,V~N(0,1), Q~N(0,1)/sqrt(D)."""
    w = make_gaussian(1, 1, 1024, 32, 16, "f32", seed, name="c1_single_head_f32")
    return w


def config2(dtype="f32", seed=2, N_side=129):
    """PDE-mesh-shaped FLARE: B4 H8 D16 M128 on a 129x129 grid (N=16641).

    X = [x, y, f(x,y)] W_lift + N(0, 0.01) noise with C = 128 channels,
    f = sum_{k=1..8} sin(k pi x) sin(k pi y) / k^2; K_h, V_h = X W_{K/V,h} / sqrt(C);
    Q ~ N(0, 1/D).  Grid x_i = i/(side-1), flattened row-major (n = iy*side + ix).
    The grid is shared over the batch; the noise is drawn per batch item.
    """
    B, H, D, M, C = 4, 8, 16, 128, 128
    t = np.arange(N_side) / (N_side - 1)
    yy, xx = np.meshgrid(t, t, indexing="ij")
    x, y = xx.reshape(-1), yy.reshape(-1)
    N = x.size
    f = np.zeros_like(x)
    for k in range(1, 9):
        f += np.sin(k * np.pi * x) * np.sin(k * np.pi * y) / (k * k)
    feats = np.stack([x, y, f], axis=-1)                      # [N, 3]
    W_lift = _gauss(seed, "lift", (3, C))
    X = feats @ W_lift                                        # [N, C]
    X = X[None, :, :] + _gauss(seed, "noise", (B, N, C), 0.1)  # [B, N, C]
    K = _heads(X, _gauss(seed, "wk", (C, H * D)), H, D)
    V = _heads(X, _gauss(seed, "wv", (C, H * D)), H, D)
    Q = _gauss(seed, "q", (H, M, D), 1.0 / math.sqrt(D))
    return Workload(f"c2_pde_mesh_{dtype}", B, H, N, M, D, dtype,
                    to_dtype(Q, dtype), to_dtype(K, dtype), to_dtype(V, dtype),
                    recipe="129x129 grid, X=[x,y,f]W_lift+N(0,0.01), C=128, K,V=XW/sqrt(C), Q~N(0,1/D)")


def config3(M=64, seed=3, N=7225):
    """Irregular point cloud, bf16: B8 H8 D16 N7225, M in {64, 256}.

    Points ~ U[0,1]^2 (one cloud per batch item); 64 frequencies w ~ N(0, 4^2 I)
    give 128 random Fourier features; K, V = RFF W / sqrt(128); Q ~ N(0, 1/D).
    """
    B, H, D, C = 8, 8, 16, 128
    pts = _rng(seed, "pts").random((B, N, 2))
    omega = _gauss(seed, "omega", (C // 2, 2), 4.0)
    X = _rff(pts, omega)                                      # [B, N, 128]
    K = _heads(X, _gauss(seed, "wk", (C, H * D)), H, D)
    V = _heads(X, _gauss(seed, "wv", (C, H * D)), H, D)
    Q = _gauss(seed, "q", (H, M, D), 1.0 / math.sqrt(D))
    return Workload(f"c3_point_cloud_M{M}_bf16", B, H, N, M, D, "bf16",
                    to_dtype(Q, "bf16"), to_dtype(K, "bf16"), to_dtype(V, "bf16"),
                    recipe="U[0,1]^2 points, RFF(64 w~N(0,16I)), K,V=RFF W/sqrt(128), Q~N(0,1/D)")


def config4(seed=4, B=32, N=4096):
    """Long-sequence classification-shaped FLARE++, bf16: B32 H4 D32 N4096 M64.

    ids ~ U{0..255}; X = E[ids] with E ~ N(0,1) [256,128].
    Ks = N0(X Wks / sqrt(128)) and Vs = Ks (shared); K = N0(X Wk / sqrt(128));
    V = X Wv / sqrt(128); Qs, Qf = N0(N(0, 1/D)); gate = sigmoid(0.25).
    """
    H, D, M, C = 4, 32, 64, 128
    ids = _rng(seed, "ids").integers(0, 256, size=(B, N))
    E = _gauss(seed, "emb", (256, C))
    X = E[ids]                                                # [B, N, C]
    Ks = rms_norm(_heads(X, _gauss(seed, "wks", (C, H * D)), H, D))
    K = rms_norm(_heads(X, _gauss(seed, "wk", (C, H * D)), H, D))
    V = _heads(X, _gauss(seed, "wv", (C, H * D)), H, D)
    Qs = rms_norm(_gauss(seed, "qs", (H, M, D), 1.0 / math.sqrt(D)))
    Qf = rms_norm(_gauss(seed, "qf", (H, M, D), 1.0 / math.sqrt(D)))
    g = np.full((H,), 1.0 / (1.0 + math.exp(-GATE_LOGIT)), dtype=np.float32)
    Ks_b = to_dtype(Ks, "bf16")
    return Workload("c4_long_seq_pp_bf16", B, H, N, M, D, "bf16",
                    Q=to_dtype(Qf, "bf16"), K=to_dtype(K, "bf16"), V=to_dtype(V, "bf16"),
                    pp=True, Qs=to_dtype(Qs, "bf16"), Ks=Ks_b, Vs=Ks_b, Qf=to_dtype(Qf, "bf16"), gate=g,
                    recipe="ids~U{0..255}, X=E[ids], Ks=N0(XWks/sqrt C)=Vs, K=N0(XWk/sqrt C), V=XWv/sqrt C")


def cotangent(seed: int, tag: str, shape, dtype: str = "bf16", std: float = 1.0) -> np.ndarray:
    """Seeded output cotangent for the backward (tags "dy", "dz", "dl"):
    i.i.d. N(0, std^2), rounded to ``dtype`` ("bf16", or "f32")."""
    return to_dtype(_gauss(seed, tag, tuple(shape), std), dtype)


def sphere_points(seed: int, B: int, N: int) -> np.ndarray:
    g = _rng(seed, "pts").standard_normal(size=(B, N, 3))
    return g / np.linalg.norm(g, axis=-1, keepdims=True)


def config5_raw(seed=5, N=1 << 20, H=8):
    """The million-point FLARE++ workload before its per-head norms: Ks, K, Qs
    and Qf as in config5(pp=True) but not normalised, and the learned channel
    scales of Qs and K drawn as 1 + N(0, 0.01); the forward normalises them
    (flags 15, the FLARE++ column of Table 2)."""
    B, D, M, C = 1, 32, 256, 128
    pts = sphere_points(seed, B, N).astype(np.float32)
    omega = _gauss(seed, "omega", (C // 2, 3), 4.0).astype(np.float32)
    X = _rff(pts, omega).astype(np.float32)
    K = _heads(X, _gauss(seed, "wk", (C, H * D)).astype(np.float32), H, D)
    V = _heads(X, _gauss(seed, "wv", (C, H * D)).astype(np.float32), H, D)
    Ks = to_dtype(_heads(X, _gauss(seed, "wks", (C, H * D)).astype(np.float32), H, D), "bf16")
    Qs = _gauss(seed, "qs", (H, M, D), 1.0 / math.sqrt(D))
    Qf = _gauss(seed, "qf", (H, M, D), 1.0 / math.sqrt(D))
    g = np.full((H,), 1.0 / (1.0 + math.exp(-GATE_LOGIT)), dtype=np.float32)
    return Workload("c5_surface_mesh_pp_raw_bf16", B, H, N, M, D, "bf16", Q=to_dtype(Qf, "bf16"),
                    K=to_dtype(K, "bf16"), V=to_dtype(V, "bf16"), pp=True, Qs=to_dtype(Qs, "bf16"), Ks=Ks, Vs=Ks,
                    Qf=to_dtype(Qf, "bf16"), gate=g, norm_flags=15,
                    alpha_qs=channel_scales(seed, "alpha_qs", H, D), alpha_k=channel_scales(seed, "alpha_k", H, D),
                    recipe="as c5pp before the norms: Ks=RFF Wks/sqrt 128 (=Vs), K, Qs, Qf raw; alpha=1+N(0,0.01)")


def config5_simplified(seed=5, N=1 << 20, H=8):
    """The million-point workload for simplified FLARE++ (Table 2, simplified
    column): raw Qs and Ks as in config5_raw with N_a on both (flags 3), a
    separate synthesis value Vs = RFF Wvs / sqrt(128), no blend (Qf = 0,
    gate = 1), and the routing keys and values of config5 without norms."""
    B, D, M, C = 1, 32, 256, 128
    pts = sphere_points(seed, B, N).astype(np.float32)
    omega = _gauss(seed, "omega", (C // 2, 3), 4.0).astype(np.float32)
    X = _rff(pts, omega).astype(np.float32)
    K = _heads(X, _gauss(seed, "wk", (C, H * D)).astype(np.float32), H, D)
    V = _heads(X, _gauss(seed, "wv", (C, H * D)).astype(np.float32), H, D)
    Ks = to_dtype(_heads(X, _gauss(seed, "wks", (C, H * D)).astype(np.float32), H, D), "bf16")
    Vs = to_dtype(_heads(X, _gauss(seed, "wvs", (C, H * D)).astype(np.float32), H, D), "bf16")
    Qs = _gauss(seed, "qs", (H, M, D), 1.0 / math.sqrt(D))
    Qf = np.zeros((H, M, D), dtype=np.float32)
    g = np.ones((H,), dtype=np.float32)
    return Workload("c5_surface_mesh_pp_simplified_bf16", B, H, N, M, D, "bf16", Q=Qf, K=to_dtype(K, "bf16"),
                    V=to_dtype(V, "bf16"), pp=True, Qs=to_dtype(Qs, "bf16"), Ks=Ks, Vs=Vs, Qf=Qf, gate=g,
                    norm_flags=3, alpha_qs=channel_scales(seed, "alpha_qs", H, D),
                    alpha_ks=channel_scales(seed, "alpha_ks", H, D),
                    recipe="as c5pp before the norms, separate Vs=RFF Wvs/sqrt 128, N_a on Qs and Ks, Qf=0, g=1")


def config5(pp=False, seed=5, N=1 << 20, H=8):
    """Million-point surface mesh, bf16: B1 H8 D32 N=2^20 M256.

    Points uniform on the unit sphere (normalised 3-D Gaussians); 64
    frequencies w ~ N(0, 4^2 I) give 128 RFF channels of xyz; K, V per head =
    RFF W / sqrt(128); Q ~ N(0, 1/D).  FLARE++ adds Ks = N0(RFF Wks/sqrt(128))
    = Vs, K -> N0(K), Qs and Qf = N0(N(0, 1/D)) and gate = sigmoid(0.25).
    The feature matrix is formed in float32 to keep generation fast.
    """
    B, D, M, C = 1, 32, 256, 128
    pts = sphere_points(seed, B, N).astype(np.float32)
    omega = _gauss(seed, "omega", (C // 2, 3), 4.0).astype(np.float32)
    X = _rff(pts, omega).astype(np.float32)                   # [B, N, 128]
    K = _heads(X, _gauss(seed, "wk", (C, H * D)).astype(np.float32), H, D)
    V = _heads(X, _gauss(seed, "wv", (C, H * D)).astype(np.float32), H, D)
    Q = _gauss(seed, "q", (H, M, D), 1.0 / math.sqrt(D))
    name = "c5_surface_mesh_pp_bf16" if pp else "c5_surface_mesh_bf16"
    if not pp:
        return Workload(name, B, H, N, M, D, "bf16", to_dtype(Q, "bf16"), to_dtype(K, "bf16"),
                        to_dtype(V, "bf16"),
                        recipe="unit-sphere points, RFF(64 w~N(0,16I)) of xyz, K,V=RFF W/sqrt(128), Q~N(0,1/D)")
    Ks = to_dtype(_rms_norm_f32(_heads(X, _gauss(seed, "wks", (C, H * D)).astype(np.float32), H, D)), "bf16")
    K = to_dtype(_rms_norm_f32(K), "bf16")
    Qs = rms_norm(_gauss(seed, "qs", (H, M, D), 1.0 / math.sqrt(D)))
    Qf = rms_norm(_gauss(seed, "qf", (H, M, D), 1.0 / math.sqrt(D)))
    g = np.full((H,), 1.0 / (1.0 + math.exp(-GATE_LOGIT)), dtype=np.float32)
    return Workload(name, B, H, N, M, D, "bf16", Q=to_dtype(Qf, "bf16"), K=K, V=to_dtype(V, "bf16"),
                    pp=True, Qs=to_dtype(Qs, "bf16"), Ks=Ks, Vs=Ks, Qf=to_dtype(Qf, "bf16"), gate=g,
                    recipe="as c5 plus Ks=N0(RFF Wks/sqrt 128)=Vs, K=N0(K), Qs,Qf=N0(N(0,1/D)), g=sigmoid(0.25)")


def _per_head(W: np.ndarray, H: int, D: int) -> np.ndarray:
    """[C, H*D] / sqrt(C) -> [H, C, D]: the per-head projection matrices of _heads."""
    C = W.shape[0]
    return np.ascontiguousarray((W / math.sqrt(C)).reshape(C, H, D).transpose(1, 0, 2))


def make_gaussian_proj(B, H, N, M, D, C=128, seed=0, pp=False, name="gaussian_proj"):
    """Fused-projection inputs, bf16: X ~ N(0,1) [B,N,C], W_K, W_V (and for
    FLARE++ W~_K) ~ N(0, 1/C) [H,C,D], Q ~ N(0, 1/D); FLARE++ adds raw seeds
    Qs and fixed queries Qf, channel scales as make_gaussian_pp_raw, gate
    sigmoid(0.25) and the norms of Table 2 (flags 15)."""
    X = to_dtype(_gauss(seed, "x", (B, N, C)), "bf16")
    WK = to_dtype(_gauss(seed, "wk", (H, C, D), 1.0 / math.sqrt(C)), "bf16")
    WV = to_dtype(_gauss(seed, "wv", (H, C, D), 1.0 / math.sqrt(C)), "bf16")
    Q = to_dtype(_gauss(seed, "q", (H, M, D), 1.0 / math.sqrt(D)), "bf16")
    w = Workload(name, B, H, N, M, D, "bf16", Q=Q, K=None, V=None, X=X, WK=WK, WV=WV,
                 recipe=f"X~N(0,1) [B,N,{C}], W~N(0,1/{C}), Q~N(0,1/D); seed {seed}")
    if pp:
        w.pp = True
        w.WKs = to_dtype(_gauss(seed, "wks", (H, C, D), 1.0 / math.sqrt(C)), "bf16")
        w.Qs = to_dtype(_gauss(seed, "qs", (H, M, D), 0.6), "bf16")
        w.Qf = to_dtype(_gauss(seed, "qf", (H, M, D), 0.5), "bf16")
        w.Q = w.Qf
        w.gate = np.full((H,), 1.0 / (1.0 + math.exp(-GATE_LOGIT)), dtype=np.float32)
        w.norm_flags = 15
        w.alpha_qs = channel_scales(seed, "alpha_qs", H, D)
        w.alpha_k = channel_scales(seed, "alpha_k", H, D)
    return w


def config5_proj(pp=False, seed=5, N=1 << 20, H=8):
    """The million-point surface mesh from its block input: X = the 128 RFF
    channels of the points (bf16 [1, N, 128]) and the per-head projections
    W / sqrt(128) of config5 as [H, 128, 32] bf16 matrices, so that K = X W_K
    and V = X W_V are formed inside the forward.  FLARE++ adds the synthesis
    projection W~_K, raw Qs and Qf and the Table 2 norms (flags 15) with the
    channel scales of config5_raw."""
    B, D, M, C = 1, 32, 256, 128
    pts = sphere_points(seed, B, N).astype(np.float32)
    omega = _gauss(seed, "omega", (C // 2, 3), 4.0).astype(np.float32)
    X = to_dtype(_rff(pts, omega).astype(np.float32), "bf16")
    WK = to_dtype(_per_head(_gauss(seed, "wk", (C, H * D)), H, D), "bf16")
    WV = to_dtype(_per_head(_gauss(seed, "wv", (C, H * D)), H, D), "bf16")
    Q = to_dtype(_gauss(seed, "q", (H, M, D), 1.0 / math.sqrt(D)), "bf16")
    name = "c5_surface_mesh_proj_pp_bf16" if pp else "c5_surface_mesh_proj_bf16"
    w = Workload(name, B, H, N, M, D, "bf16", Q=Q, K=None, V=None, X=X, WK=WK, WV=WV,
                 recipe="unit-sphere points, X = RFF(64 w~N(0,16I)) of xyz [1,N,128], W_K, W_V = W/sqrt(128) "
                        "per head, Q~N(0,1/D)")
    if pp:
        w.pp = True
        w.WKs = to_dtype(_per_head(_gauss(seed, "wks", (C, H * D)), H, D), "bf16")
        w.Qs = to_dtype(_gauss(seed, "qs", (H, M, D), 1.0 / math.sqrt(D)), "bf16")
        w.Qf = to_dtype(_gauss(seed, "qf", (H, M, D), 1.0 / math.sqrt(D)), "bf16")
        w.Q = w.Qf
        w.gate = np.full((H,), 1.0 / (1.0 + math.exp(-GATE_LOGIT)), dtype=np.float32)
        w.norm_flags = 15
        w.alpha_qs = channel_scales(seed, "alpha_qs", H, D)
        w.alpha_k = channel_scales(seed, "alpha_k", H, D)
        w.recipe += "; FLARE++: W~_K = Wks/sqrt(128), raw Qs, Qf, Table 2 norms (flags 15)"
    return w


def _rms_norm_f32(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + np.float32(RMS_EPS))


CONFIGS = {
    "c1": lambda: config1(),
    "c2f": lambda: config2("f32"),
    "c2b": lambda: config2("bf16"),
    "c3a": lambda: config3(64),
    "c3b": lambda: config3(256),
    "c4": lambda: config4(),
    "c5": lambda: config5(False),
    "c5pp": lambda: config5(True),
}
