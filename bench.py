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
workload's shape (--variant capacity | noisy | noisy_eps | zloss).
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


def stage_work(w, R=None, noisy=None):
    """Algorithmic work per stage for one layer call: FLOP for the GEMMs, bytes for the
    streaming stages (minimum each stage must move). R: rows the GEMMs run (the kept
    rows under an expert capacity); noisy: "eps", the router also reads W_noise and the
    draw; "drawn", it reads W_noise and draws in the kernel."""
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
        router += d * E * s + (T * E * 4 if noisy == "eps" else 0)
    work["router"] = ("bytes", router)
    if w.dtype != "bf16" or T * d >= 2 ** 31:
        # rows copied into expert order (bf16 layers otherwise gather them inside the
        # gate/up GEMM, and the permute only writes row indices: a latency-bound stage)
        work["permute"] = ("bytes", T * d * s + R * d * s + R * 4 + T * k * 4)
    work["combine"] = ("bytes", R * d * 4 + T * k * 8 + T * d * 4)
    return work


TRAFFIC_SOURCE = ("HBM bytes per gate/up launch from profiles/mixtral_layer_hbm_traffic.md "
                  "(rocprofv3 FETCH_SIZE and WRITE_SIZE runs scaled by a copy kernel), valid for "
                  "the gemm.hip source whose SHA-256 it records; not measured in this run")


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
    """The fp64 oracle as it stands, on the first `sample_tokens` tokens. Returns the
    baseline record and the oracle's outputs (for the parity check after the timing)."""
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
        ref = O.forward_tc(xs, inp["Wg"], inp["b"], inp["Wgate"], inp["Wup"], inp["Wdown"], w.k,
                           w.renormalize)
    else:
        ref = O.forward_ec(xs, inp["Wg"], inp["b"], inp["Wgate"], inp["Wup"], inp["Wdown"], w.cf)
    dt = time.perf_counter() - t0
    rec = {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"first {n} of {w.T} tokens of the same workload through the fp64 NumPy "
                     f"oracle (router, top-k, per-expert fp64 GEMMs, combine); {dt:.1f} s",
           "seconds": dt, "host_cpus": os.cpu_count()}
    return rec, ref, n


def parity_vs_oracle(w, inp, ref, n, y_dev, idx_dev):
    """The timed run's output against the oracle's on the tokens the CPU leg ran: routing
    (tokens whose top-k margin exceeds 1e-5 must pick the oracle's experts) and y, by the
    bf16 rule max|dy| / rms(y) <= 2e-2 (fp32: max|dy| / max|y| <= 1e-4). Near-tie tokens
    are compared with the oracle evaluated on the device's experts."""
    from oracle import moe_oracle as O
    bf = w.dtype == "bf16"
    y_ref = ref["y"]
    out = {"tokens": int(n), "tol": 2e-2 if bf else 1e-4,
           "norm": "max|dy| / rms(y_ref)" if bf else "max|dy| / max|y_ref|"}
    if w.mode == "tc":
        idx_ref = ref["idx"]
        exempt = O.topk_margin(ref["probs"], w.k) <= 1e-5
        idx_d = idx_dev[:n].astype(np.int64)
        diff = np.any(np.sort(idx_d, 1) != np.sort(idx_ref, 1), axis=1)
        out["idx_mismatch_tokens"] = int(np.sum(diff & ~exempt))
        out["exempt_tokens"] = int(exempt.sum())
        redo = np.nonzero(diff & exempt)[0]
        if redo.size:
            y_ref = y_ref.copy()
            w_use = O.gate_weights(ref["probs"][redo], idx_d[redo], w.renormalize)
            y_ref[redo] = O.mix(inp["x"][redo], idx_d[redo], w_use, inp["Wgate"], inp["Wup"],
                                inp["Wdown"])
    else:
        if n != w.T:  # expert choice ranks every token: only the full batch is comparable
            return None
        out["idx_mismatch_experts"] = int(np.sum(np.any(idx_dev.astype(np.int64) != ref["idx"],
                                                        axis=1)))
    dy = np.max(np.abs(y_dev[:n].astype(np.float64) - y_ref))
    scale = np.sqrt(np.mean(y_ref ** 2)) if bf else np.max(np.abs(y_ref))
    out["y_err"] = float(dy / scale)
    out["ok"] = bool(out["y_err"] <= out["tol"] and out.get("idx_mismatch_tokens", 0) == 0
                     and out.get("idx_mismatch_experts", 0) == 0)
    return out


def router_bound(torch, M, x, weights, y, ws, kw, steps, w, router_bytes):
    """A plain streaming read of x in the router's place: each step runs one layer call, then
    torch.sum(x) (every element read once, an fp32 result: the bytes of x and a few partials),
    timed alone with HIP events; and the same read with x warm (right after another read).
    Returns the median read rates against the router's own (its event pass in this run)."""
    Wg, b, Wgate, Wup, Wdown = weights
    xb = x.numel() * x.element_size()
    ev = []
    for _ in range(steps):
        M.moe_forward(x, Wg, b, Wgate, Wup, Wdown, y=y, workspace=ws, **kw)
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r = torch.sum(x, dtype=torch.float32)
        z.record()
        ev.append((a, z))
    torch.cuda.synchronize()
    after_layer = float(np.median([a.elapsed_time(z) for a, z in ev]))
    ev = []
    for _ in range(steps):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r = torch.sum(x, dtype=torch.float32)
        z.record()
        ev.append((a, z))
    torch.cuda.synchronize()
    warm = float(np.median([a.elapsed_time(z) for a, z in ev]))
    del r
    return {"what": "torch.sum(x, dtype=float32) timed alone: after a layer call (the router's "
                    "place) and back to back (x warm)",
            "x_bytes": xb, "after_layer_us": round(after_layer * 1e3, 2),
            "after_layer_gbs": round(xb / (after_layer * 1e-3) / 1e9, 1),
            "warm_us": round(warm * 1e3, 2), "warm_gbs": round(xb / (warm * 1e-3) / 1e9, 1),
            "router_bytes": router_bytes}


def reference_gemm(torch, w, group_rows, steps, warmup, gu_ms, dn_ms):
    """torch's bf16 matmul (hipBLASLt) on the grouped GEMMs' problems, one matmul per expert:
    gate and up as one [d, 2 d_ff] weight (the same FLOP as the fused gate/up GEMM, without its
    SwiGLU epilogue) and the down projection; random bf16 operands of the same sizes. Timed
    with one event pair around all experts' matmuls per step; median over the steps."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    rows = [int(n) for n in group_rows]
    nmax = max(rows)
    xa = torch.randn(nmax, w.d, device=dev, generator=g).to(torch.bfloat16)
    ha = torch.randn(nmax, w.f, device=dev, generator=g).to(torch.bfloat16)
    Wgu = torch.randn(w.E, w.d, 2 * w.f, device=dev, generator=g).to(torch.bfloat16)
    Wd = torch.randn(w.E, w.f, w.d, device=dev, generator=g).to(torch.bfloat16)
    out_gu = torch.empty(nmax, 2 * w.f, device=dev, dtype=torch.bfloat16)
    out_d = torch.empty(nmax, w.d, device=dev, dtype=torch.bfloat16)

    def run(which):
        for e, n in enumerate(rows):
            if n == 0:
                continue
            if which == "gu":
                torch.matmul(xa[:n], Wgu[e], out=out_gu[:n])
            else:
                torch.matmul(ha[:n], Wd[e], out=out_d[:n])

    res = {}
    R = sum(rows)
    for which, flop, ours in (("gate_up", 4.0 * w.d * w.f * R, gu_ms),
                              ("down", 2.0 * w.f * w.d * R, dn_ms)):
        key = "gu" if which == "gate_up" else "down"
        for _ in range(warmup):
            run(key)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for a, z in ev:
            a.record()
            run(key)
            z.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(z) for a, z in ev]))
        res[which] = {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                      "frac_of_peak": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "ours_ms": round(ours, 4), "ours_over_reference": round(ms / ours, 4)}
    res["what"] = ("torch.matmul bf16 per expert (hipBLASLt), bf16 output, same group sizes; "
                   "gate/up as one [d, 2 d_ff] weight without the SwiGLU epilogue")
    return res


def one_expert_gemm(torch, M, w, steps, warmup, rows=4096):
    """The grouped GEMMs on a regular problem, against torch's bf16 matmul (hipBLASLt) on
    operands of the same sizes: a layer with one expert and `rows` tokens at the workload's
    d_model and d_ff (every token routed to it), its gate/up and down stages timed with the
    library's per-stage events; torch: x [rows, d] times [W_gate | W_up] [d, 2 d_ff] (no SwiGLU
    epilogue) and h [rows, d_ff] times W_down [d_ff, d]. Medians over the steps."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    T, d, f = rows, w.d, w.f
    x = torch.randn(T, d, device=dev, generator=g).to(torch.bfloat16)
    Wg = torch.zeros(d, 1, device=dev, dtype=torch.bfloat16)
    Wgate = (torch.randn(1, d, f, device=dev, generator=g) * 0.01).to(torch.bfloat16)
    Wup = (torch.randn(1, d, f, device=dev, generator=g) * 0.01).to(torch.bfloat16)
    Wdown = (torch.randn(1, f, d, device=dev, generator=g) * 0.01).to(torch.bfloat16)
    out = M.moe_forward(x, Wg, None, Wgate, Wup, Wdown, k=1, want_stats=False)
    ws, y = out["workspace"], out["y"]
    for _ in range(warmup):
        M.moe_forward(x, Wg, None, Wgate, Wup, Wdown, k=1, y=y, workspace=ws, want_stats=False)
    torch.cuda.synchronize()
    M.profile_enable(True)
    M.profile_read()
    for _ in range(steps):
        M.moe_forward(x, Wg, None, Wgate, Wup, Wdown, k=1, y=y, workspace=ws, want_stats=False)
    torch.cuda.synchronize()
    st = M.profile_read()
    M.profile_enable(False)
    res = {"rows": T, "d_model": d, "d_ff": f}
    h = torch.randn(T, f, device=dev, generator=g).to(torch.bfloat16)
    Wgu = torch.cat([Wgate[0], Wup[0]], 1).contiguous()
    o1 = torch.empty(T, 2 * f, device=dev, dtype=torch.bfloat16)
    o2 = torch.empty(T, d, device=dev, dtype=torch.bfloat16)
    for name, stage, fn, flop in (
            ("gate_up", "gemm_gate_up", lambda: torch.matmul(x, Wgu, out=o1), 4.0 * d * f * T),
            ("down", "gemm_down", lambda: torch.matmul(h, Wdown[0], out=o2), 2.0 * f * d * T)):
        ours = st[stage][0] / max(st[stage][1], 1)
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for a, z in ev:
            a.record()
            fn()
            z.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(z) for a, z in ev]))
        res[name] = {"ours_us": round(ours * 1e3, 1),
                     "ours_tflops": round(flop / (ours * 1e-3) / 1e12, 1),
                     "torch_us": round(ms * 1e3, 1),
                     "torch_tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    res["what"] = ("one expert, every token routed to it; ours: per-stage events (mean over the "
                   "steps), torch.matmul bf16: median; gate/up without the SwiGLU epilogue in torch")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_layer_skewed_top2_bf16",
                    choices=sorted(W.WORKLOADS), help="workload (default: the Mixtral-size layer)")
    ap.add_argument("--cpu-sample", type=int, default=16384,
                    help="tokens the CPU oracle baseline runs (0 = skip)")
    ap.add_argument("--variant", default="plain",
                    choices=("plain", "capacity", "noisy", "noisy_eps", "zloss"),
                    help="token-choice variant: an expert capacity (--cf), training noise "
                         "softplus(x W_noise) * eps with eps drawn in the router kernel (noisy) "
                         "or passed as a [T, E] input (noisy_eps), or the router z-loss as an "
                         "extra output")
    ap.add_argument("--cf", type=float, default=1.0, help="capacity factor of --variant capacity")
    ap.add_argument("--reference-gemm", action="store_true",
                    help="after the layer, also time torch's bf16 matmul (hipBLASLt) on the same "
                         "per-expert problems as the grouped GEMMs: x_e [n_e, d] @ [d, 2 d_ff] "
                         "and h_e [n_e, d_ff] @ [d_ff, d], n_e the layer's group sizes")
    ap.add_argument("--router-bound", action="store_true",
                    help="after the layer, time a plain streaming read of x (torch.sum over its "
                         "bf16 values, fp32 result) placed where the router runs: right after a "
                         "layer call, repeated; the read rate x allows in that cache state")
    ap.add_argument("--one-expert-gemm", action="store_true",
                    help="also time the GEMMs on a one-expert layer of 4096 tokens against "
                         "torch's bf16 matmul on operands of the same sizes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB read + 256 MiB write kernel (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
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
        kw.update(W_noise=to_dev(nz["Wn"]), eps=M.NoiseDraw(seed=2024, offset=0))
    elif args.variant == "noisy_eps":
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
    # the timed steps: one event pair per step on the stream the library launches on
    # (torch's current stream), no per-stage events; a second pass of the same steps
    # records HIP events around every kernel launch for the per-stage figures
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for a, z in ev:
        a.record()
        last = M.moe_forward(x, Wg, b, Wgate, Wup, Wdown, y=y, workspace=ws, **kw)
        z.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_ms = np.array([a.elapsed_time(z) for a, z in ev])
    M.profile_enable(True)
    M.profile_read()  # clear
    for _ in range(args.steps):
        M.moe_forward(x, Wg, b, Wgate, Wup, Wdown, y=y, workspace=ws, **kw)
    torch.cuda.synchronize()
    M.profile_enable(False)
    stages = M.profile_read()
    ms_step = float(np.median(step_ms))
    tokens_s = w.T / (ms_step * 1e-3)

    work = stage_work(w, R_run, noisy={"noisy": "drawn", "noisy_eps": "eps"}.get(args.variant))
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

    traffic = (gemm_traffic_from_profile()
               if w is W.MIXTRAL_LAYER and args.variant == "plain" else None)
    cpu = parity = None
    if args.cpu_sample > 0 and args.variant == "plain":
        y_dev = y.cpu().numpy()
        idx_dev = last["idx"].cpu().numpy()
        cpu, ref, n_ref = cpu_baseline(w, inp, args.cpu_sample)
        parity = parity_vs_oracle(w, inp, ref, n_ref, y_dev, idx_dev)
        del ref

    line = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_stats": {"median": round(ms_step, 4), "mean": round(float(step_ms.mean()), 4),
                              "min": round(float(step_ms.min()), 4),
                              "max": round(float(step_ms.max()), 4),
                              "timing": "hipEvent pair per step on the launch stream; median"},
        "timed_wall_s": round(t_wall, 4),
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
                     "traffic": traffic,
                     "traffic_source": (TRAFFIC_SOURCE if traffic is not None else None)},
        "stages": st_out,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    if args.router_bound:
        line["router_bound"] = router_bound(torch, M, x, (Wg, b, Wgate, Wup, Wdown), y, ws, kw,
                                            args.steps, w, work["router"][1])
    if args.reference_gemm and w.dtype == "bf16":
        line["reference_gemm"] = reference_gemm(torch, w, counts if w.mode != "ec" else
                                                np.full(w.E, w.capacity), args.steps, args.warmup,
                                                gu_ms, dn_ms)
    if args.one_expert_gemm and w.dtype == "bf16":
        line["one_expert_gemm"] = one_expert_gemm(torch, M, w, args.steps, args.warmup)
    if args.variant != "plain":
        line["config"]["variant"] = args.variant
        if args.variant == "capacity":
            line["config"].update(capacity_factor=args.cf, capacity=C, rows_kept=R_run)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
