"""Benchmark: sparse MoE layer forward on one MI355X.

A step is one full layer forward (router, dispatch scan with f/p/loss, permute, grouped
SwiGLU gate/up GEMM, grouped down GEMM, combine) over one batch of synthetic
tokens already resident in HBM. Default workload: the Mixtral 8x7B layer shape
(T=16384 tokens, d_model=4096, d_ff=14336, E=8, top-2, bf16, router bias
N(0,1) per expert giving a skewed load).

Prints one JSON line (rank 0). The timed steps run with no per-stage events; the
per-kernel durations come from a second pass of the same steps in which the library
records HIP events around each launch on the stream it launches on.

Options select the other workloads (--workload NAME) and the token-choice variants at a
workload's shape (--variant capacity | noisy | zloss).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402  (seeded input generators only)

METRIC = "MoE-layer tokens/sec + expert GEMM TFLOP/s (% bf16 MFMA peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (vector and matrix)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def stage_work(w, R=None, noisy=False):
    """Algorithmic work per stage for one layer call: FLOP for the GEMMs, bytes for the
    streaming stages (minimum each stage must move). R: rows the GEMMs run (the kept
    rows under an expert capacity); noisy: the router also reads W_noise and the draw."""
    s = 2 if w.dtype == "bf16" else 4
    T, d, f, E = w.T, w.d, w.f, w.E
    R = w.rows if R is None else R
    work = {
        "gemm_gate_up": ("flop", 4.0 * d * f * R),
        "gemm_down": ("flop", 2.0 * f * d * R),
    }
    if w.mode == "ec":
        # logits written once [E, T]; each chosen row gathered (copied in fp32); o, the
        # choice lists and y for the combine
        work["router"] = ("bytes", T * d * s + d * E * s + T * E * 4)
        if w.dtype != "bf16" or T * d >= 2 ** 31:
            work["permute"] = ("bytes", 2 * R * d * s + R * 4)
        work["combine"] = ("bytes", R * d * 4 + R * 8 + T * d * 4)
        return work
    k = w.k
    router = T * d * s + d * E * s + T * k * 8 + T * E * 4
    if noisy:
        router += d * E * s + T * E * 4
    work["router"] = ("bytes", router)
    if w.dtype != "bf16" or T * d >= 2 ** 31:
        # rows copied into expert order (bf16 layers otherwise gather them inside the
        # gate/up GEMM, and the permute only writes row indices: a latency-bound stage)
        work["permute"] = ("bytes", T * d * s + R * d * s + R * 4 + T * k * 4)
    work["combine"] = ("bytes", R * d * 4 + T * k * 8 + T * d * 4)
    return work


def gemm_traffic_from_profile():
    """HBM bytes per gate/up GEMM launch from the committed FETCH_SIZE/WRITE_SIZE summary,
    scaled by the copy-kernel calibration; None when the GEMM source changed since."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "mixtral_layer_hbm_traffic.md")
    src = os.path.join(ROOT, "sparse_mixture_experts_sum_amd", "csrc", "gemm.hip")
    try:
        rec = {}
        for line in open(prof):
            if ":" in line and line.startswith("    "):
                k, v = line.strip().split(":", 1)
                rec[k.strip()] = v.strip()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if rec.get("gemm_source_sha256") != sha:
            return None
        return int(1024 * (float(rec["gemm_gate_up_fetch_kib"]) * float(rec["fetch_scale"])
                           + float(rec["gemm_gate_up_write_kib"]) * float(rec["write_scale"])))
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w, inp, sample_tokens):
    """The fp64 oracle as it stands, on the first `sample_tokens` tokens."""
    from oracle import moe_oracle as O
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"),
                      default=1)
    except Exception:
        threads = 1
    n = min(sample_tokens, w.T)
    xs = inp["x"][:n]
    t0 = time.perf_counter()
    if w.mode == "tc":
        O.forward_tc(xs, inp["Wg"], inp["b"], inp["Wgate"], inp["Wup"], inp["Wdown"], w.k,
                     w.renormalize)
    else:
        O.forward_ec(xs, inp["Wg"], inp["b"], inp["Wgate"], inp["Wup"], inp["Wdown"], w.cf)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {w.T} tokens of the same workload through the fp64 NumPy "
                      f"oracle (router, top-k, per-expert fp64 GEMMs, combine); {dt:.1f} s",
            "seconds": dt, "host_cpus": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_layer_skewed_top2_bf16",
                    choices=sorted(W.WORKLOADS), help="workload (default: the Mixtral-size layer)")
    ap.add_argument("--cpu-sample", type=int, default=16384,
                    help="tokens the CPU oracle baseline runs (0 = skip)")
    ap.add_argument("--variant", default="plain", choices=("plain", "capacity", "noisy", "zloss"),
                    help="token-choice variant: an expert capacity (--cf), training noise "
                         "softplus(x W_noise) * eps, or the router z-loss as an extra output")
    ap.add_argument("--cf", type=float, default=1.0, help="capacity factor of --variant capacity")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB read + 256 MiB write kernel (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              f"(the layer is benchmarked on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_mixture_experts_sum_amd as M

    M.load_library()
    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = W.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to_dev(a, t=dt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(t)

    x, Wg = to_dev(inp["x"]), to_dev(inp["Wg"])
    b = to_dev(inp["b"], torch.float32)
    Wgate, Wup, Wdown = to_dev(inp["Wgate"]), to_dev(inp["Wup"]), to_dev(inp["Wdown"])
    y = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)
    kw = dict(k=w.k, mode=w.mode, capacity_factor=w.cf, renormalize=w.renormalize,
              want_stats=(w.mode == "tc"))
    if args.variant != "plain" and w.mode != "tc":
        print("bench.py: --variant applies to token-choice workloads", file=sys.stderr)
        sys.exit(2)
    if args.variant == "capacity":
        kw.update(mode="tc_capacity", capacity_factor=args.cf)
    elif args.variant == "noisy":
        nz = W.make_noise(w, wn_std=0.02)
        kw.update(W_noise=to_dev(nz["Wn"]), eps=to_dev(nz["eps"], torch.float32))
    elif args.variant == "zloss":
        kw.update(want_z_loss=True)
    out = M.moe_forward(x, Wg, b, Wgate, Wup, Wdown, y=y, **kw)
    ws = out["workspace"]
    torch.cuda.synchronize()
    counts = out["counts"].cpu().numpy()
    R_run = None
    if args.variant == "capacity":
        C = M.capacity(out["shape"])
        R_run = int(np.minimum(counts, C).sum())

    if args.copy_calibration:
        # a plain streaming kernel of known traffic (reads and writes 256 MiB each) so that
        # HBM counters can be scaled: torch.neg on fp32
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        M.moe_forward(x, Wg, b, Wgate, Wup, Wdown, y=y, workspace=ws, **kw)
    torch.cuda.synchronize()
    # the timed steps run without per-stage events; a second pass of the same steps
    # records HIP events around every kernel launch for the per-stage figures
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        M.moe_forward(x, Wg, b, Wgate, Wup, Wdown, y=y, workspace=ws, **kw)
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    M.profile_enable(True)
    M.profile_read()  # clear
    for _ in range(args.steps):
        M.moe_forward(x, Wg, b, Wgate, Wup, Wdown, y=y, workspace=ws, **kw)
    torch.cuda.synchronize()
    M.profile_enable(False)
    stages = M.profile_read()
    ms_step = ms_total / args.steps
    tokens_s = w.T / (ms_step * 1e-3)

    work = stage_work(w, R_run, noisy=args.variant == "noisy")
    peak_tf = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    st_out = {}
    for name, (tot, n) in stages.items():
        if n == 0:
            continue
        avg_ms = tot / n
        rec = {"avg_us": round(avg_ms * 1e3, 2), "launches": n}
        if name in work:
            kind, amount = work[name]
            if kind == "flop":
                a = amount / (avg_ms * 1e-3) / 1e12
                rec.update(achieved=round(a, 1), unit="TFLOP/s", frac=round(a / peak_tf, 4))
            else:
                a = amount / (avg_ms * 1e-3) / 1e9
                rec.update(achieved=round(a, 1), unit="GB/s", frac=round(a / PEAK_HBM_GBS, 4))
        st_out[name] = rec
    gu = stages["gemm_gate_up"]
    dn = stages["gemm_down"]
    gu_ms = gu[0] / max(gu[1], 1)
    dn_ms = dn[0] / max(dn[1], 1)
    gemm_flop = work["gemm_gate_up"][1] + work["gemm_down"][1]
    gemm_tf = gemm_flop / ((gu_ms + dn_ms) * 1e-3) / 1e12
    gu_tf = work["gemm_gate_up"][1] / (gu_ms * 1e-3) / 1e12

    cpu = None
    if args.cpu_sample > 0 and args.variant == "plain":
        cpu = cpu_baseline(w, inp, args.cpu_sample)

    line = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d_model": w.d, "d_ff": w.f, "E": w.E,
                   "k": w.k if w.mode == "tc" else None, "mode": w.mode,
                   "capacity_factor": w.cf if w.mode == "ec" else None,
                   "router_bias": w.bias_std is not None, "rows": w.rows,
                   "expert_rows_min_max": [int(counts.min()), int(counts.max())]},
        "expert_gemm_tflops": round(gemm_tf, 1),
        "expert_gemm_frac_of_peak": round(gemm_tf / peak_tf, 4),
        "roofline": {"bound": "mfma", "kernel": "gemm_gate_up", "achieved": round(gu_tf, 1),
                     "peak": peak_tf, "unit": "TFLOP/s", "frac": round(gu_tf / peak_tf, 4),
                     "traffic": (gemm_traffic_from_profile()
                                 if w is W.MIXTRAL_LAYER and args.variant == "plain" else None)},
        "stages": st_out,
        "cpu_baseline": cpu,
    }
    if args.variant != "plain":
        line["config"]["variant"] = args.variant
        if args.variant == "capacity":
            line["config"].update(capacity_factor=args.cf, capacity=C, rows_kept=R_run)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
