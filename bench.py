"""Benchmark of the FLARE routing forward on one MI355X.

One step = one flare_forward call (encode partials -> merge -> decode) over
the whole million-token surface-mesh workload: B=1, H=8, N=1,048,576, M=256,
D=32, bf16 inputs with float32 accumulation, inputs resident in HBM before
the timed region.  FLOPs are counted as 8*B*H*N*M*D per routing pass.

Prints one JSON line with the throughput, the roofline position of the
dominant kernel (timed with HIP events on the stream the library launches
on) and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FLARE routing fwd tokens/s at N=1M,M=256 (1 GPU); % of bf16 MFMA roofline"
METRIC_BWD = "FLARE routing bwd tokens/s at N=1M,M=256 (1 GPU); % of bf16 MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# v_exp_f32 peak on the same 2.4 GHz basis as the MFMA and HBM peaks: the
# transcendental unit retires 8 lanes per clock per SIMD (half the 16-lane
# VALU rate; a microbenchmark of back-to-back v_exp_f32 reaches 16 T/s at the
# ~1.95 GHz sustained clock, i.e. 8 lanes per clock), so
# 1024 SIMDs x 8 x 2.4 GHz = 19.66 T exponentials/s
PEAK_EXP_T = 1024 * 8 * 2.4e9 / 1e12


KERNEL_SRC_DIR = os.path.join(ROOT, "rank_latent_attention_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_info() -> dict:
    """Where the line was measured: device name, gfx architecture, HIP runtime."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "hip": torch.version.hip}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def kernel_source_sha256() -> str:
    """sha256 over the code of the kernel sources (csrc/*.hip and *.h, by name), with
    // comments, trailing blanks and empty lines left out: a comment edit does not
    invalidate counters taken on the same code."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(KERNEL_SRC_DIR)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            for line in open(os.path.join(KERNEL_SRC_DIR, f), encoding="utf-8"):
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (already scaled by the copy-kernel calibration), or None
    when they were taken on another version of the kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_sha256") != kernel_source_sha256():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, target_s: float = 15.0):
    """The fp64 oracle of the same routing forward (FLARE, or FLARE++ with its
    synthesis step) on a bounded sample: all N tokens of the first k heads,
    k chosen from a one-head timing so the sample takes about target_s."""
    import oracle
    oracle.build(force=False)
    cores = oracle.threads()

    def heads(x, k):
        return np.ascontiguousarray(x[:, :k])

    def run(k):
        t0 = time.perf_counter()
        if w.pp and w.norm_flags:
            f = w.norm_flags
            Ks = heads(w.Ks, k)
            oracle.flare_pp_forward_normed(
                w.Qs[:k], Ks, Ks if w.Vs is w.Ks else heads(w.Vs, k), w.Qf[:k], w.gate[:k], heads(w.K, k),
                heads(w.V, k), norm_qs=bool(f & 1), norm_ks=bool(f & 2), norm_qf=bool(f & 4), norm_k=bool(f & 8),
                alpha_qs=None if w.alpha_qs is None else w.alpha_qs[:k],
                alpha_ks=None if w.alpha_ks is None else w.alpha_ks[:k],
                alpha_k=None if w.alpha_k is None else w.alpha_k[:k])
        elif w.pp:
            oracle.flare_pp_forward(w.Qs[:k], heads(w.Ks, k), heads(w.Vs, k), w.Qf[:k], w.gate[:k],
                                    heads(w.K, k), heads(w.V, k))
        else:
            oracle.flare_forward(w.Q[:k], heads(w.K, k), heads(w.V, k))
        return time.perf_counter() - t0

    t1 = run(1)
    k = int(max(1, min(w.H, round(target_s / max(t1, 1e-3)))))
    t = run(k) if k > 1 else t1
    # a token of the whole routing pass needs all H heads
    value = w.B * w.N * k / (t * w.H)
    what = "FLARE++ forward (synthesis encode, blend, encode + decode)" if w.pp else "FLARE forward (encode + decode)"
    if w.norm_flags:
        what = "FLARE++ forward with its per-head RMS norms (norms, synthesis encode, blend, encode + decode)"
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "host_logical_cpus": os.cpu_count(),
            "sample": f"fp64 oracle {what} on heads 0..{k - 1} of {w.H}, all {w.N} tokens, "
                      f"M={w.M}, D={w.D}: {t:.1f} s on {cores} OpenMP threads; tokens/s scaled by {k}/{w.H} heads"}


def oracle_times(w) -> dict:
    """Wall time of the fp64 oracle of this workload's forward on the host,
    on one thread and on all the threads the oracle uses by default."""
    import oracle
    oracle.build(force=False)
    full = oracle.threads()

    def run():
        t0 = time.perf_counter()
        if w.pp:
            oracle.flare_pp_forward(w.Qs, w.Ks, w.Vs, w.Qf, w.gate, w.K, w.V)
        else:
            oracle.flare_forward(w.Q, w.K, w.V)
        return time.perf_counter() - t0

    oracle.threads(1)
    t1 = run()
    oracle.threads(full)
    tn = run()
    return {"oracle_s_1_thread": round(t1, 3), "oracle_s": round(tn, 3), "oracle_threads": full,
            "oracle_tokens_per_s": w.B * w.N / tn}


def time_configs(names: str, with_oracle: bool = False) -> None:
    """Per-workload forward timing (inputs resident, events on the library's
    stream): one JSON line per workload, not the bench line."""
    import torch
    import rank_latent_attention_amd as flare
    from rank_latent_attention_amd.inputs import CONFIGS
    F = flare.flare
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    todo = list(CONFIGS) if names == "all" else names.split(",")
    for name in todo:
        w = CONFIGS[name]()
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        code = F.BF16 if w.dtype == "bf16" else F.F32

        def up(x):
            return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)

        B, H, N, M, D = w.B, w.H, w.N, w.M, w.D
        K, V = up(w.K), up(w.V)
        Y = torch.empty_like(K)
        Z = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
        L = torch.empty((B, H, M), dtype=torch.float32, device=dev)
        if w.pp:
            Qs, Ks, Qf = up(w.Qs), up(w.Ks), up(w.Qf)
            Vs = Ks if w.shared_vs else up(w.Vs)
            gate = torch.from_numpy(w.gate).to(dev)
            Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
            ws = flare.workspace(F.OP_PP_FORWARD, B, H, N, M, D, code, dev)

            def step():
                F.flare_pp_forward(Qs, Ks, Vs, Qf, gate, K, V, Y=Y, Q_out=Qo, Z=Z, L=L, ws=ws)
            flops = 12.0 * B * H * N * M * D
        else:
            Q = up(w.Q)
            ws = flare.workspace(F.OP_FORWARD, B, H, N, M, D, code, dev)

            def step():
                F.flare_forward(Q, K, V, Y=Y, Z=Z, L=L, ws=ws)
            flops = 8.0 * B * H * N * M * D
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        n = 50
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for i in range(n):
            ev[2 * i].record(stream)
            step()
            ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        t = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(n))
        med = t[n // 2]
        # algorithmic HBM bytes of the forward: the encode reads K and V, the
        # decode reads K and writes Y (FLARE++ also reads the synthesis keys,
        # and their values when separate); queries and latents are negligible
        tok = B * H * N * D * K.element_size()
        hbm = 4 * tok + ((1 if w.shared_vs else 2) * tok if w.pp else 0)
        rec = {"workload": w.name, "B": B, "H": H, "N": N, "M": M, "D": D, "dtype": w.dtype,
               "flare_pp": bool(w.pp), "us_median": round(med, 1), "us_min": round(t[0], 1),
               "us_max": round(t[-1], 1), "tokens_per_s": B * N / (med * 1e-6),
               "tflops": round(flops / (med * 1e-6) / 1e12, 1),
               "mfma_frac": round(flops / (med * 1e-6) / 1e12 / (PEAK_BF16_TFLOPS if w.dtype == "bf16" else 157.3), 4),
               "algorithmic_bytes": hbm, "hbm_frac": round(hbm / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        # Working sets under the 256 MB last-level cache stay resident between
        # back-to-back calls; the cold variant writes a 512 MB buffer before
        # every timed call so the inputs come from HBM.
        resident = sum(x.numel() * x.element_size() for x in (K, V, Y))
        if resident < (256 << 20):
            flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
            for i in range(n):
                flush.fill_(float(i))
                ev[2 * i].record(stream)
                step()
                ev[2 * i + 1].record(stream)
            torch.cuda.synchronize()
            tc = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(n))
            rec["us_median_cold"] = round(tc[n // 2], 1)
            rec["hbm_frac_cold"] = round(hbm / (tc[n // 2] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
            del flush
        if with_oracle and w.N * w.B * w.H * w.M <= (1 << 30):  # the million-token runs stay with the bench line
            rec.update(oracle_times(w))
        print(json.dumps(rec), flush=True)
        del K, V, Y, Z, L, ws
        torch.cuda.empty_cache()


def cpu_baseline_backward(w, dY, target_s: float = 15.0):
    """The fp64 oracle of the FLARE (or FLARE++) backward (forward recompute,
    decoder and encoder backward, and for FLARE++ the blend and synthesis
    backward) on a bounded sample: the first n tokens of head 0, n chosen
    from a 2^16-token timing so the sample takes about target_s."""
    import oracle
    oracle.build(force=False)
    cores = oracle.threads()

    def tok(x, n):
        return np.ascontiguousarray(x[:, :1, :n])

    def run(n):
        t0 = time.perf_counter()
        if w.pp and w.norm_flags:
            f = w.norm_flags
            Ks = tok(w.Ks, n)

            def a(x):
                return None if x is None else x[:1]
            oracle.flare_pp_backward_normed(
                w.Qs[:1], Ks, Ks, w.Qf[:1], w.gate[:1], tok(w.K, n), tok(w.V, n), tok(dY, n),
                norm_qs=bool(f & 1), norm_ks=bool(f & 2), norm_qf=bool(f & 4), norm_k=bool(f & 8),
                alpha_qs=a(w.alpha_qs), alpha_ks=a(w.alpha_ks), alpha_k=a(w.alpha_k))
        elif w.pp:
            Ks = tok(w.Ks, n)
            oracle.flare_pp_backward(w.Qs[:1], Ks, Ks, w.Qf[:1], w.gate[:1], tok(w.K, n), tok(w.V, n), tok(dY, n))
        else:
            oracle.flare_backward(w.Q[:1], tok(w.K, n), tok(w.V, n), tok(dY, n))
        return time.perf_counter() - t0

    n1 = min(w.N, 1 << 16)
    t1 = run(n1)
    n = int(min(w.N, max(n1, n1 * target_s / max(t1, 1e-3))))
    t = run(n) if n > n1 else t1
    value = w.B * n / (t * w.H)   # a token of the whole pass needs all H heads
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "host_logical_cpus": os.cpu_count(),
            "sample": f"fp64 oracle {'FLARE++' if w.pp else 'FLARE'} backward (forward recompute, decoder and "
                      f"encoder backward{', blend and synthesis backward' if w.pp else ''}"
                      f"{', through the per-head RMS norms' if w.norm_flags else ''}) on head 0 of "
                      f"{w.H}, first {n} of {w.N} tokens, M={w.M}, D={w.D}: {t:.1f} s on {cores} OpenMP threads; "
                      f"tokens/s scaled by 1/{w.H} heads (the work is linear in the token count)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=["flare", "flare_pp", "flare_pp_norm", "flare_pp_simplified", "flare_backward",
                                           "flare_pp_backward", "flare_pp_norm_backward", "flare_proj",
                                           "flare_proj_unfused"],
                    default="flare",
                    help="FLARE or FLARE++ routing forward on the million-point surface mesh; flare_pp_norm feeds "
                         "the FLARE++ inputs before their per-head RMS norms and normalises inside the kernels; "
                         "flare_pp_simplified is simplified FLARE++ (N_a on the seeds and synthesis keys, separate "
                         "synthesis values, no blend) through the same fused-norm entry point; "
                         "flare_backward times the FLARE backward (dQ, dK, dV from dY) after one untimed forward; "
                         "flare_pp_backward the FLARE++ backward likewise, flare_pp_norm_backward the backward of flare_pp_norm "
                         "(through the fused norms); flare_proj starts from the block input X [B,N,128] with the "
                         "per-head projections K = X W_K, V = X W_V fused into the encode (flare_forward_proj), "
                         "flare_proj_unfused runs the same from X with the projections as torch.mm calls writing K "
                         "and V, then flare_forward")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps, so the GPU clock has ramped up "
                         "(0 to skip)")
    ap.add_argument("--configs", default="",
                    help="instead of the bench line, time the forward of these workloads (comma-separated names "
                         "from rank_latent_attention_amd.inputs.CONFIGS, or 'all'): 10 warmup and 50 timed calls "
                         "each, one JSON line per workload with the median, min and max, plus a cold-cache "
                         "median (512 MB written before each call) where the working set is under 256 MB")
    ap.add_argument("--oracle-times", action="store_true",
                    help="with --configs: also time the fp64 oracle of each workload's forward on the host, on one "
                         "thread and on all of them (skipped for the million-token workloads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB float32 scale kernel (read 256 MiB, write 256 MiB) before the steps, as a "
                         "known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the library runs on one GPU and its sharding "
              "over several is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_latent_attention_amd as flare
    from rank_latent_attention_amd.inputs import config5, config5_raw, config5_simplified

    if args.configs:
        time_configs(args.configs, args.oracle_times)
        return
    if args.workload in ("flare_backward", "flare_pp_backward", "flare_pp_norm_backward"):
        bench_backward(args, pp=args.workload != "flare_backward", norm=args.workload == "flare_pp_norm_backward")
        return
    if args.workload in ("flare_proj", "flare_proj_unfused"):
        bench_proj(args, fused=args.workload == "flare_proj")
        return

    pp = args.workload in ("flare_pp", "flare_pp_norm", "flare_pp_simplified")
    norm = args.workload in ("flare_pp_norm", "flare_pp_simplified")
    t0 = time.perf_counter()
    if args.workload == "flare_pp_simplified":
        w = config5_simplified()
    else:
        w = config5_raw() if norm else config5(pp=pp)
    log(f"generated {w.name} in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)

    B, H, N, M, D = w.B, w.H, w.N, w.M, w.D
    K, V = up(w.K), up(w.V)
    Y = torch.empty_like(K)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
    L = torch.empty((B, H, M), dtype=torch.float32, device=dev)
    if pp:
        Qs, Ks, Qf = up(w.Qs), up(w.Ks), up(w.Qf)
        Vs = Ks if w.shared_vs else up(w.Vs)
        gate = torch.from_numpy(w.gate).to(dev)
        Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
        ws = flare.workspace(flare.flare.OP_PP_FORWARD, B, H, N, M, D, flare.flare.BF16, dev)

        if norm:
            def opt(a):
                return None if a is None else torch.from_numpy(a).to(dev)
            aqs, aks, ak = opt(w.alpha_qs), opt(w.alpha_ks), opt(w.alpha_k)

            def step():
                flare.flare_pp_forward_norm(Qs, Ks, Vs, Qf, gate, K, V, w.norm_flags, aqs, aks, ak, Y=Y, Q_out=Qo,
                                            Z=Z, L=L, ws=ws)
        else:
            def step():
                flare.flare_pp_forward(Qs, Ks, Ks, Qf, gate, K, V, Y=Y, Q_out=Qo, Z=Z, L=L, ws=ws)
    else:
        Q = up(w.Q)
        ws = flare.workspace(flare.flare.OP_FORWARD, B, H, N, M, D, flare.flare.BF16, dev)

        def step():
            flare.flare_forward(Q, K, V, Y=Y, Z=Z, L=L, ws=ws)

    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = src * 1.0
        torch.cuda.synchronize()
        del src, dst
    settle(step, args.settle)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"{args.steps} steps: {ms:.3f} ms/step")

    if not norm:
        # Per-phase times with events between the launches: the encode entry
        # point (encode partials + merge) and the decode entry point (decode
        # kernel alone), run back to back exactly as one flare_forward step runs them.
        Qr = Qo if pp else Q
        qb = Qr.to(torch.bfloat16).contiguous() if pp else Qr
        nrep = max(args.steps, 5)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * nrep)]
        wse = flare.workspace(flare.flare.OP_ENCODE, B, H, N, M, D, flare.flare.BF16, dev)
        for i in range(nrep):
            ev[3 * i].record(stream)
            flare.flare_encode(qb, K, V, Z=Z, L=L, ws=wse)
            ev[3 * i + 1].record(stream)
            flare.flare_decode(qb, K, Z, Y=Y)
            ev[3 * i + 2].record(stream)
        torch.cuda.synchronize()
        t_enc = sorted(ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(nrep))[nrep // 2]
        t_dec = sorted(ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(nrep))[nrep // 2]
        log(f"phases (median of {nrep}): encode+merge {t_enc * 1e3:.1f} us, decode {t_dec * 1e3:.1f} us")

        # Roofline of the dominant kernel, measured here: the decode entry point
        # launches the decode kernel alone, so events around that call time
        # exactly it; the encode entry point launches the encode kernel and
        # the split merge (about 2% of it), so its phase time counts the merge
        # against the encode.  Whichever phase is longer is reported, the
        # other beside it.  Each pass has 4 BHNMD FLOPs and one exponential
        # per score.
        half_flops = 4.0 * B * H * N * M * D
        exps = B * H * N * M
        if t_enc > t_dec:
            kname, kt = "encode_dma_kernel+merge_kernel", t_enc
            kb = B * H * N * D * 2 * 2                 # algorithmic: read K and V (bf16)
        else:
            kname, kt = "decode_kernel", t_dec
            kb = B * H * N * D * 2 * 2                 # algorithmic: read K, write Y (bf16)
        achieved = half_flops / (kt * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic(kname, args.workload),
                    "kernel": kname, "kernel_us": round(kt * 1e3, 2), "algorithmic_bytes": kb,
                    "hbm_frac": round(kb / (kt * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "exp_rate_T_per_s": round(exps / (kt * 1e-3) / 1e12, 2),
                    "exp_frac": round(exps / (kt * 1e-3) / 1e12 / PEAK_EXP_T, 4),
                    "encode_and_merge_us": round(t_enc * 1e3, 2), "decode_us": round(t_dec * 1e3, 2),
                    "encode_phase_frac": round(half_flops / (t_enc * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "decode_frac": round(half_flops / (t_dec * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}

    flops = (12.0 if pp else 8.0) * B * H * N * M * D
    if norm:
        # The normalising kernels are reached only through the whole forward
        # (the encode and decode entry points take no norms), so this
        # workload's roofline is the step's: its 12 BHNMD FLOPs over the step
        # time.  Per-kernel times are in the kernel trace.
        achieved = flops / (ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic("whole_step", args.workload),
                    "kernel": "whole step (5 launches)", "kernel_us": round(ms * 1e3, 2),
                    # read Ks (and Vs when separate), K, V; write Y
                    "algorithmic_bytes": (4 if w.shared_vs else 5) * B * H * N * D * 2}
    tok_s = B * N / (ms * 1e-3)
    out = {"metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "settle_s": args.settle, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": ("FLARE++" if pp else "FLARE") + " routing forward, million-point surface mesh"
                      + (", simplified (no blend, separate synthesis values)"
                         if args.workload == "flare_pp_simplified" else "")
                      + (", per-head RMS norms fused" if norm else ""),
                      "B": B, "H": H, "N": N, "M": M, "D": D, "inputs": "bf16", "accumulate": "f32"},
           "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "step_frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "roofline": roofline, "device": device_info()}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


def bench_proj(args, fused: bool):
    """One step = the FLARE routing forward from the block input X of the
    million-point workload (config5_proj): fused, one flare_forward_proj call
    (the encode forms K and V per tile from X, writes K for the decode);
    unfused, one torch.mm per batch element for all heads' K and V (hipBLASLt),
    a copy into the [B,H,N,D] layout and then flare_forward.  FLOPs: 8 BHNMD for the routing plus 4 BNCHD for the two
    projections."""
    import torch
    import rank_latent_attention_amd as flare
    from rank_latent_attention_amd.inputs import config5_proj
    t0 = time.perf_counter()
    w = config5_proj()
    log(f"generated {w.name} in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)

    B, H, N, M, D = w.B, w.H, w.N, w.M, w.D
    C = w.X.shape[-1]
    X, WK, WV, Q = up(w.X), up(w.WK), up(w.WV), up(w.Q)
    Y = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
    L = torch.empty((B, H, M), dtype=torch.float32, device=dev)
    if fused:
        ws = flare.workspace(flare.flare.OP_FORWARD_PROJ, B, H, N, M, D, flare.flare.BF16, dev)

        def step():
            flare.flare_forward_proj(X, WK, WV, Q, Y=Y, Z=Z, L=L, ws=ws)
    else:
        K = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
        V = torch.empty_like(K)
        ws = flare.workspace(flare.flare.OP_FORWARD, B, H, N, M, D, flare.flare.BF16, dev)
        # one GEMM per batch element for every head's K and V ([C, 2 H D]
        # weights: X is read once), then a copy into the [H, N, D] layout
        Wcat = torch.cat([WK.permute(1, 0, 2).reshape(C, H * D), WV.permute(1, 0, 2).reshape(C, H * D)],
                         dim=1).contiguous()
        KV = torch.empty((N, 2 * H * D), dtype=torch.bfloat16, device=dev)

        def step():
            for b in range(B):
                torch.mm(X[b], Wcat, out=KV)
                K[b].copy_(KV[:, :H * D].view(N, H, D).permute(1, 0, 2))
                V[b].copy_(KV[:, H * D:].view(N, H, D).permute(1, 0, 2))
            flare.flare_forward(Q, K, V, Y=Y, Z=Z, L=L, ws=ws)
    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration:  # a 256 MiB read and write that scales the byte counters
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = src * 1.0
        torch.cuda.synchronize()
        del src, dst
    settle(step, args.settle)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"{args.steps} steps: {ms:.3f} ms/step ({'fused' if fused else 'unfused'} projections)")
    flops = 8.0 * B * H * N * M * D + 4.0 * B * N * C * H * D
    achieved = flops / (ms * 1e-3) / 1e12
    # algorithmic bytes: read X once and write Y
    kb = B * N * C * 2 + B * H * N * D * 2
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "kernel": "whole step (%s)" % ("3 launches" if fused else f"{B} GEMMs, {2 * B} copies + 3 launches"),
                "kernel_us": round(ms * 1e3, 2), "algorithmic_bytes": kb,
                "hbm_frac": round(kb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    out = {"metric": METRIC + " (from the block input X)", "value": B * N / (ms * 1e-3), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_s": args.settle, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "FLARE routing forward from the block input, million-point surface mesh, "
                                  + ("projections fused into the encode" if fused
                                     else "projections as one torch.mm, copied to [B,H,N,D], then flare_forward"),
                      "B": B, "H": H, "N": N, "M": M, "D": D, "C": C, "inputs": "bf16", "accumulate": "f32"},
           "tflops": round(achieved, 2), "routing_tflops": round(8.0 * B * H * N * M * D / (ms * 1e-3) / 1e12, 2),
           "roofline": roofline, "device": device_info()}
    print(json.dumps(out), flush=True)


def settle(step, seconds: float) -> None:
    """Run the step untimed for at least `seconds` of wall time (then sync):
    the GPU's clock ramps up over the first tens of milliseconds of this
    sustained load, and the first launches after idle run up to 1.5 times
    slower.  Nothing of it is timed."""
    import torch
    if seconds <= 0:
        return
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        step()
        torch.cuda.synchronize()


def bench_backward(args, pp=False, norm=False):
    """One step = one flare_backward call (center, statistics, decode-side
    col pass, dZ sum, encoder-side col pass, dQ sum, row pass) over the
    million-point workload, given Z and L of one untimed forward; with pp,
    one flare_pp_backward call (synthesis recomputation, that routing
    backward with float32 queries, blend backward, synthesis encoder
    backward) given the routing queries, Z and L of one untimed FLARE++
    forward; with norm, one flare_pp_backward_norm call (the inputs normalised
    again, that FLARE++ backward, the norms' backward) after one untimed
    flare_pp_forward_norm."""
    import torch
    import rank_latent_attention_amd as flare
    from rank_latent_attention_amd.inputs import config5, config5_raw, cotangent
    t0 = time.perf_counter()
    w = config5_raw() if norm else config5(pp=pp)
    dYh = cotangent(114 if pp else 101, "dy", w.K.shape)
    log(f"generated {w.name} in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)

    B, H, N, M, D = w.B, w.H, w.N, w.M, w.D
    K, V, dY = up(w.K), up(w.V), up(dYh)
    Z = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
    L = torch.empty((B, H, M), dtype=torch.float32, device=dev)
    if pp:
        Qs, Ks, Qf = up(w.Qs), up(w.Ks), up(w.Qf)
        Vs = Ks if w.shared_vs else up(w.Vs)
        gate = torch.from_numpy(w.gate).to(dev)
        Qo = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
        if norm:
            aqs, ak = torch.from_numpy(w.alpha_qs).to(dev), torch.from_numpy(w.alpha_k).to(dev)
            flare.flare_pp_forward_norm(Qs, Ks, Ks, Qf, gate, K, V, w.norm_flags, aqs, None, ak, Q_out=Qo, Z=Z, L=L)
            ws = flare.workspace(flare.flare.OP_PP_BACKWARD_NORM, B, H, N, M, D, flare.flare.BF16, dev)

            def step():
                flare.flare_pp_backward_norm(Qs, Ks, Ks, Qf, gate, K, V, Qo, Z, L, dY, w.norm_flags, aqs, None, ak,
                                             ws=ws)
        else:
            flare.flare_pp_forward(Qs, Ks, Ks, Qf, gate, K, V, Q_out=Qo, Z=Z, L=L)
            ws = flare.workspace(flare.flare.OP_PP_BACKWARD, B, H, N, M, D, flare.flare.BF16, dev)

            def step():
                flare.flare_pp_backward(Qs, Ks, Ks, Qf, gate, K, V, Qo, Z, L, dY, ws=ws)
    else:
        Q = up(w.Q)
        flare.flare_forward(Q, K, V, Z=Z, L=L)
        dQ = torch.empty((H, M, D), dtype=torch.float32, device=dev)
        dK, dV = torch.empty_like(K), torch.empty_like(K)
        ws = flare.workspace(flare.flare.OP_BACKWARD, B, H, N, M, D, flare.flare.BF16, dev)

        def step():
            flare.flare_backward(Q, K, V, Z, L, dY, dQ=dQ, dK=dK, dV=dV, ws=ws)

    stream = torch.cuda.current_stream(dev)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = src * 1.0
        torch.cuda.synchronize()
        del src, dst
    settle(step, args.settle)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"{args.steps} steps: {ms:.3f} ms/step")
    # Algorithmic FLOPs: the backward of each attention pass is five
    # products of 2 BHNMD each (scores recomputed, the output-cotangent
    # product, and the three gradients): 20 BHNMD for the FLARE pair, 30 with
    # the FLARE++ synthesis pass.  The kernels of one call are reached only
    # through the whole entry point, so the roofline is the step's; per-kernel
    # times are in the kernel trace.
    flops = (30.0 if pp else 20.0) * B * H * N * M * D
    achieved = flops / (ms * 1e-3) / 1e12
    # read K, V, dY (and the synthesis keys = values) and write dK, dV (and dKs) once each, bf16
    kb = (7 if pp else 5) * B * H * N * D * 2
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("whole_step", args.workload),
                # launches per call, as in the committed kernel traces
                "kernel": "whole step (%d launches)" % ((25 if norm else 16) if pp else 8),
                "kernel_us": round(ms * 1e3, 2),
                "algorithmic_bytes": kb, "hbm_frac": round(kb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    what = "FLARE++" if pp else "FLARE"
    out = {"metric": METRIC_BWD, "value": B * N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_s": args.settle, "ms_per_step": ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"{what} routing backward, million-point surface mesh"
                                  + (", through the per-head RMS norms" if norm else ""), "B": B, "H": H, "N": N,
                      "M": M, "D": D, "inputs": "bf16", "accumulate": "f32"},
           "tflops": round(achieved, 2), "roofline": roofline, "device": device_info()}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_backward(w, dYh)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
