"""Benchmark of the MoE SwiGLU feed-forward forward pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one moe_forward over one batch of synthetic tokens (router,
dispatch, grouped expert SwiGLU, shared experts, combine), inputs resident
in HBM. Prints ONE JSON line on stdout; details go to stderr.

The timed steps are plain forwards. After them, the dominant kernel (the
grouped gate/up GEMM) is timed with HIP events recorded by the library on the
launch stream: around that launch in single forwards, and around 20
back-to-back passes of it (which removes the events' own overhead from short
launches); its algorithmic flops (or bytes, for weight-streaming batches) per
launch divided by the mean duration of one pass gives roofline.achieved.

cpu_baseline: the CPU oracle timed on a bounded sample of the same tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec and achieved fraction of MFMA/HBM roofline, 1 GPU"
PEAK = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA TFLOP/s (MI355X)
HBM_GBS = 8000.0                        # HBM3E GB/s (MI355X)
DEFAULT_WORKLOAD = "small"              # the second configuration of the layer


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, counts, merged=False):
    """Per-step algorithmic work of the layer and of the gate/up launch
    (merged: the shared experts' gate/up GEMM runs in the same launch)."""
    es = 2 if w.act == "bf16" else 4
    de, f, rows = w.d_e, w.d_ff, w.T * w.K
    touched = int((counts > 0).sum())
    fl_router = 2.0 * w.T * w.d * w.E
    fl_routed = 6.0 * rows * de * f
    fl_shared = 6.0 * w.T * w.d * w.d_shared
    fl_latent = 4.0 * w.T * w.d * w.latent
    bytes_w = (w.E * w.d * 4 + touched * 3 * de * f * es + 3 * w.d * w.d_shared * es
               + 2 * w.d * w.latent * es)
    bytes_act = 2 * w.T * w.d * es
    gu_flops = 4.0 * rows * de * f
    # gate/up launch: touched experts' gate+up weights, gathered rows in, h out
    gu_bytes = touched * 2 * f * de * es + rows * de * es + rows * f * es
    if merged:  # + shared gate/up: its weights, x in, its h out
        gu_flops += 4.0 * w.T * w.d * w.d_shared
        gu_bytes += 2 * w.d_shared * w.d * es + w.T * w.d * es + w.T * w.d_shared * es
    return dict(flops=fl_router + fl_routed + fl_shared + fl_latent, bytes=bytes_w + bytes_act,
                gu_flops=gu_flops, gu_bytes=gu_bytes, touched=touched)


def kernel_source_hash() -> str:
    """Hash of the HIP sources: traffic figures are only valid for the kernels they came from."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_ffn_fp32_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (copy-calibrated), or None when absent or
    taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def calibrate_copy(mib: int, reps: int = 5):
    """Plain device-to-device copy of a known size, for counter calibration."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps}), flush=True)


def cpu_baseline(w, a, budget_s=15.0):
    """Time the CPU oracle (as it stands) on a seeded token sample."""
    import oracle
    orc = oracle.Oracle(w, a)
    rng = np.random.default_rng(7)
    probe = rng.choice(w.T, size=min(w.T, 8), replace=False)
    t0 = time.perf_counter()
    orc.forward(tokens=probe)
    per_tok = (time.perf_counter() - t0) / len(probe)
    n = int(max(8, min(w.T, budget_s / max(per_tok, 1e-9))))
    toks = np.sort(rng.choice(w.T, size=n, replace=False))
    t0 = time.perf_counter()
    orc.forward(tokens=toks)
    dt = time.perf_counter() - t0
    # a whole batch shorter than the budget: repeat it (up to 10 passes)
    passes = 1
    while n == w.T and dt < 0.8 * budget_s and passes < 10:
        orc.forward(tokens=toks)
        passes += 1
        dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    rep = f" x {passes} passes" if passes > 1 else ""
    return {"value": n * passes / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {w.T} tokens (seeded){rep}, full layer per token in fp64, "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass timing")
    ap.add_argument("--calibrate-copy", type=int, metavar="MiB", default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer's "
              "multi-GPU sharding is not part of this build", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_ffn_fp32_amd as moe
    import moe_synth

    w = moe_synth.get(args.workload)
    log(f"workload {w.name}: T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} K={w.K} "
        f"shared={w.d_shared} latent={w.latent} act={w.act}")
    t0 = time.perf_counter()
    a = moe_synth.generate(w)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layer = moe.Layer(w, moe.to_device(a, dev), device=dev)
    x = layer.dev["x"]
    out = torch.empty((w.T, w.d), dtype=layer.act, device=dev)
    counts = torch.zeros(w.E, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        layer.forward(x, out, counts=counts)
    torch.cuda.synchronize()

    # the timed steps: plain forwards (no timing events inside the layer)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        layer.forward(x, out, counts=counts)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt / args.steps * 1e3

    # after them: the gate/up launch bracketed by HIP events that the library
    # records on the launch stream, once per forward (the events' own cost
    # included) ...
    stage = moe.STAGES["expert_gate_up"]
    n_ev = min(args.steps, 20)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_ev)]
    for b, e in evs:  # materialise the events on the launch stream
        b.record(stream)
        e.record(stream)
    torch.cuda.synchronize()
    for b, e in evs:
        layer.forward(x, out, counts=counts,
                      probe=moe.MoeProbe(stage=stage, repeat=1, ev_begin=b.cuda_event,
                                         ev_end=e.cuda_event))
    torch.cuda.synchronize()
    gu_ms_event = float(np.mean([b.elapsed_time(e) for b, e in evs]))

    # ... and without the events' own overhead (a few us, which matters for
    # short launches): forwards whose gate/up stage enqueues the launch REPS
    # times back to back between the two events (each pass recomputes the
    # same rows); one launch = elapsed / REPS.
    REPS, PASSES = 20, 5
    rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(PASSES)]
    for b, e in rev:
        b.record(stream)
        e.record(stream)
    torch.cuda.synchronize()
    for b, e in rev:
        layer.forward(x, out, counts=counts,
                      probe=moe.MoeProbe(stage=stage, repeat=REPS, ev_begin=b.cuda_event,
                                         ev_end=e.cuda_event))
    torch.cuda.synchronize()
    gu_ms = float(np.mean([b.elapsed_time(e) for b, e in rev])) / REPS

    cnt = counts.cpu().numpy()
    plan = moe.moe_plan(layer.desc)
    alg = algorithmic(w, cnt, merged=bool(plan["merged_shared"]))

    # bias-based balancer step on this step's loads (a scratch bias, so the
    # layer's routing is untouched)
    bias_scratch = torch.zeros(w.E, dtype=torch.float32, device=dev)
    b_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 200
    moe.moe_balance_bias(w.E, w.K, w.T, counts, 1e-3, bias_scratch, stream)
    b_ev.record(stream)
    for _ in range(reps):
        moe.moe_balance_bias(w.E, w.K, w.T, counts, 1e-3, bias_scratch, stream)
    e_ev.record(stream)
    torch.cuda.synchronize()
    balance_us = b_ev.elapsed_time(e_ev) / reps * 1e3

    # QuantileBalancer update (sigmoid-routed layers): router + per-expert
    # quantile of thresh - s over all tokens, into a scratch bias
    qb = None
    if w.route == "sigmoid_bias" and w.K < w.E:
        nb = torch.empty(w.E, dtype=torch.float32, device=dev)
        moe.moe_quantile_balance(layer.desc, layer.weights, x, nb, layer.ws, stream)
        b_ev.record(stream)
        for _ in range(10):
            moe.moe_quantile_balance(layer.desc, layer.weights, x, nb, layer.ws, stream)
        e_ev.record(stream)
        torch.cuda.synchronize()
        qb = {"ms_per_call": round(b_ev.elapsed_time(e_ev) / 10, 4), "tokens": w.T, "experts": w.E}
    # router auxiliary losses (load-balancing + z-loss) on this step's loads
    losses = torch.empty(2, dtype=torch.float32, device=dev)
    moe.moe_router_losses(layer.desc, layer.weights, x, counts, 0.01, 0.001, losses, layer.ws,
                          stream)
    b_ev.record(stream)
    for _ in range(10):
        moe.moe_router_losses(layer.desc, layer.weights, x, counts, 0.01, 0.001, losses, layer.ws,
                              stream)
    e_ev.record(stream)
    torch.cuda.synchronize()
    rl = {"ms_per_call": round(b_ev.elapsed_time(e_ev) / 10, 4), "tokens": w.T, "experts": w.E,
          "load_balancing_loss": round(float(losses[0]), 7),
          "z_loss": round(float(losses[1]), 7)}
    # backward pass: input and all weight gradients for an output gradient of ones
    bwd = None
    if not args.no_backward:
        dy = torch.ones((w.T, w.d), dtype=layer.act, device=dev)
        de = w.d_e
        shapes = {"w_router": (w.E, w.d), "w_gate": (w.E, w.d_ff, de),
                  "w_up": (w.E, w.d_ff, de), "w_down": (w.E, de, w.d_ff)}
        if w.d_shared:
            shapes.update(ws_gate=(w.d_shared, w.d), ws_up=(w.d_shared, w.d),
                          ws_down=(w.d, w.d_shared))
        if w.latent:
            shapes.update(w_lat_down=(w.latent, w.d), w_lat_up=(w.d, w.latent))
            if w.has_rmsnorm:
                shapes["rms_gamma"] = (w.latent,)
        grads = {k: torch.empty(v, dtype=torch.float32, device=dev) for k, v in shapes.items()}
        d_x = torch.empty_like(x)
        layer.backward(x, dy, d_x=d_x, grads=grads, stream=stream)
        b_ev.record(stream)
        for _ in range(3):
            layer.backward(x, dy, d_x=d_x, grads=grads, stream=stream)
        e_ev.record(stream)
        torch.cuda.synchronize()
        bms = b_ev.elapsed_time(e_ev) / 3
        # routed + shared: forward gate/up recomputed, d(h), d(x), 3 weight gradients;
        # latent: + the routed down GEMM recomputed, the two projections' three
        fl = 2.0 * (w.T * w.K * de * w.d_ff + w.T * w.d * w.d_shared) * (2 + 1 + 2 + 3)
        if w.latent:
            fl += 2.0 * w.T * w.K * de * w.d_ff + 2.0 * w.T * w.d * w.latent * 5
        bwd = {"ms_per_call": round(bms, 4), "tokens_per_s": round(w.T / (bms / 1e3), 1),
               "tflops": round(fl / (bms / 1e3) / 1e12, 2),
               "note": "moe_backward: input, router, expert and shared weight gradients "
                       "(routing recomputed), output gradient of ones; tflops counts the "
                       "recomputed gate/up GEMM"}
        del grads, d_x, dy
        layer.ws_bwd = None
        torch.cuda.empty_cache()
    tok_s = w.T / (ms / 1e3)
    peak_tf = PEAK[w.act]
    intensity = alg["gu_flops"] / alg["gu_bytes"]
    ridge = peak_tf * 1e12 / (HBM_GBS * 1e9)
    if intensity >= ridge:
        ach = alg["gu_flops"] / (gu_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(ach / peak_tf, 4), "traffic": None}
    else:
        ach = alg["gu_bytes"] / (gu_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_GBS, 4), "traffic": None}
    roof["traffic"] = measured_traffic(w.name)
    roof["kernel"] = "grouped gate/up GEMM + SiLU*up" + (
        " (+ the shared experts' gate/up GEMM in the same launch)" if plan["merged_shared"] else "")
    roof["tile"] = f"{plan['gate_up_tile_m']}x{plan['gate_up_tile_n']}"
    roof["kernel_ms"] = round(gu_ms, 4)
    roof["timing"] = (f"mean of {PASSES} x {REPS} back-to-back launches between HIP events on "
                      f"the launch stream; a single launch bracketed by events, after the timed steps: "
                      f"{gu_ms_event:.4f} ms (includes the events' own overhead)")
    log(f"step {ms:.4f} ms, {tok_s:.4g} tokens/s; gate/up kernel {gu_ms:.4f} ms; "
        f"experts touched {alg['touched']}/{w.E}; loads max {cnt.max()} min {cnt.min()}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, a)
        log(f"cpu baseline: {cpu}")

    line = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "d_model": w.d, "d_ff": w.d_ff,
                   "experts": w.E, "top_k": w.K, "shared_width": w.d_shared,
                   "latent": w.latent, "route": w.route, "parallelism": "single-gpu"},
        "layer": {"algorithmic_tflop": round(alg["flops"] / 1e12, 5),
                  "tflops": round(alg["flops"] / (ms / 1e3) / 1e12, 2),
                  "frac_of_mfma_peak": round(alg["flops"] / (ms / 1e3) / 1e12 / peak_tf, 4),
                  "algorithmic_gb": round(alg["bytes"] / 1e9, 4),
                  "gbs": round(alg["bytes"] / (ms / 1e3) / 1e9, 1),
                  "experts_touched": alg["touched"]},
        "roofline": roof,
        "balance_bias": {"us_per_call": round(balance_us, 2), "experts": w.E,
                         "note": "one bias-based balancer step, back-to-back launches"},
        "quantile_balance": qb,
        "router_losses": rl,
        "backward": bwd,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
