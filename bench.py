"""Benchmark of the MoE SwiGLU feed-forward forward pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
python bench.py --peak            (peak-rate microbenchmarks only)
python bench.py --calibrate-copy MiB   (plain device copy, counter calibration)

One step = one moe_forward over one batch of synthetic tokens (router,
dispatch, grouped expert SwiGLU, shared experts, combine), inputs resident
in HBM. Prints ONE JSON line on stdout; details go to stderr.

The default workload is the largest single-GPU configuration, the large
layer (E=256, K=8, d=7168, d_ff=2048, 2 shared) at T=16384 tokens; the same
resident weights are then also timed at the decode batch of T=64 tokens
(the `decode` object of the line).

The timed steps are plain forwards (each also bracketed by HIP events on the
launch stream for the median / min figures). After them, each GEMM stage of
the layer is timed with HIP events the library records on its launch stream,
around 20 back-to-back passes of the stage (removing the events' own
overhead); the dominant kernel (the grouped gate/up GEMM) gives
roofline.achieved = its algorithmic flops (or bytes, for weight-streaming
batches) per launch / the mean duration of one pass.

cpu_baseline: the CPU oracle timed on a bounded sample of the same tokens
(all host cores, then one core), plus its routing and dispatch over all T.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec and achieved fraction of MFMA/HBM roofline, 1 GPU"
PEAK = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA TFLOP/s (MI355X datasheet, 2.4 GHz)
HBM_GBS = 8000.0                        # HBM3E GB/s (MI355X datasheet)
DEFAULT_WORKLOAD = "large_prefill"      # the largest configuration that fits one GPU
DECODE_OF = {"large_prefill": "large_decode"}  # same layer at the decode batch
CU_COUNT = 256
MFMA_FLOP_PER_CLK_CU = 4096             # dense bf16: 2.5 PFLOP/s / (256 CUs x 2.4 GHz)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, counts, merged=False):
    """Per-step algorithmic work of the layer and of each GEMM launch
    (merged: the shared experts' GEMMs run in the grouped launches)."""
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
    # down launch: touched experts' down weights, h in, y out
    dn_flops = 2.0 * rows * de * f
    dn_bytes = touched * f * de * es + rows * f * es + rows * de * es
    sh_gu_flops = 4.0 * w.T * w.d * w.d_shared
    sh_gu_bytes = 2 * w.d_shared * w.d * es + w.T * w.d * es + w.T * w.d_shared * es
    if merged:
        gu_flops += sh_gu_flops
        gu_bytes += sh_gu_bytes
        dn_flops += 2.0 * w.T * w.d * w.d_shared
        dn_bytes += w.d_shared * w.d * es + w.T * w.d_shared * es + w.T * w.d * 4
    return dict(flops=fl_router + fl_routed + fl_shared + fl_latent, bytes=bytes_w + bytes_act,
                gu_flops=gu_flops, gu_bytes=gu_bytes, dn_flops=dn_flops, dn_bytes=dn_bytes,
                sh_gu_flops=sh_gu_flops, sh_gu_bytes=sh_gu_bytes, touched=touched)


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


# ------------------------------------------------------------ peak rates

PEAK_MODES = {0: "mfma_16x16x32_bf16", 1: "mfma_32x32x16_bf16", 2: "lds_read_16B",
              3: "mfma_16x16x32_bf16+lds(3 reads/8 mfma)", 4: "mfma_32x32x16_bf16+lds(3 reads/4 mfma)",
              5: "mfma_16x16x32_bf16+lds(2 reads/8 mfma)", 6: "mfma_32x32x16_bf16+lds(2 reads/4 mfma)",
              7: "lds_frag16_swz_row", 8: "lds_frag16_swz_row_half", 9: "lds_frag32_swz_row",
              10: "lds_frag32_swz_row_half"}
LDS_MODES = (2, 7, 8, 9, 10)


def peak_rates(modes=tuple(PEAK_MODES), threads=(256, 512), iters=4000, rounds=4):
    """Peak-rate microbenchmarks (moe_peak): per mode and wavefronts per SIMD,
    the rate over the whole launch (HIP events) and per CU at the running
    shader clock (from each workgroup's s_memtime / s_memrealtime)."""
    import torch
    import mixture_experts_ffn_fp32_amd as moe
    groups = CU_COUNT * rounds
    out = []
    for mode in modes:
        for th in threads:
            clk = torch.zeros(2 * groups, dtype=torch.int64, device="cuda")
            sink = torch.zeros(groups * th, dtype=torch.int32, device="cuda")
            moe.moe_peak(mode, th, groups, 200, clk, sink)  # warm-up
            b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b.record()
            moe.moe_peak(mode, th, groups, iters, clk, sink)
            e.record()
            torch.cuda.synchronize()
            ms = b.elapsed_time(e)
            c = clk.cpu().numpy().reshape(groups, 2).astype(np.float64)
            cycles, ticks = np.median(c[:, 0]), np.median(c[:, 1])
            ghz = cycles / (ticks / 100e6) / 1e9
            waves = th // 64
            rec = {"mode": PEAK_MODES[mode], "waves_per_simd": waves // 4,
                   "clock_ghz": round(ghz, 3), "launch_ms": round(ms, 4)}
            if mode in LDS_MODES:
                by = 8 * 1024 * 2 * iters * waves  # bytes per workgroup (= per CU)
                rec["lds_bytes_per_clk_cu"] = round(by / cycles, 1)
                rec["lds_tbs"] = round(by * groups / (ms / 1e3) / 1e12, 2)
            else:
                fl = 131072.0 * 2 * iters * waves
                rec["tflops"] = round(fl * groups / (ms / 1e3) / 1e12, 1)
                rec["frac_of_clock_peak"] = round(fl / cycles / MFMA_FLOP_PER_CLK_CU, 4)
                rec["frac_of_datasheet"] = round(rec["tflops"] / PEAK["bf16"], 4)
            out.append(rec)
            log(f"peak {rec}")
    return out


# ------------------------------------------------------------ timing

def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def timed_steps(layer, x, out, counts, steps, warmup):
    """Wall time of `steps` plain forwards (synchronised on both sides), and
    each step's duration between HIP events on the launch stream."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        layer.forward(x, out, counts=counts)
    evs = _events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for b, e in evs:
        b.record(stream)
        layer.forward(x, out, counts=counts)
        e.record(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    per = np.array([b.elapsed_time(e) for b, e in evs])
    return dt / steps * 1e3, {"mean": round(float(per.mean()), 5),
                              "median": round(float(np.median(per)), 5),
                              "min": round(float(per.min()), 5),
                              "max": round(float(per.max()), 5)}


def stage_ms(layer, x, out, counts, stage, reps, passes=5):
    """Mean duration of one pass of a stage: `passes` forwards whose stage is
    bracketed by HIP events the library records on its launch stream, the
    GEMM stages enqueued `reps` times back to back between them."""
    import torch
    import mixture_experts_ffn_fp32_amd as moe
    stream = torch.cuda.current_stream()
    evs = _events(passes)
    for b, e in evs:  # materialise the events on the launch stream
        b.record(stream)
        e.record(stream)
    torch.cuda.synchronize()
    for b, e in evs:
        layer.forward(x, out, counts=counts,
                      probe=moe.MoeProbe(stage=moe.STAGES[stage], repeat=reps,
                                         ev_begin=b.cuda_event, ev_end=e.cuda_event))
    torch.cuda.synchronize()
    return float(np.mean([b.elapsed_time(e) for b, e in evs])) / reps


REPEATABLE = ("latent_down", "expert_gate_up", "expert_down", "shared_gate_up")


def stages_of(layer, x, out, counts, w, alg, plan, peak_tf):
    """Per-stage times; the GEMM stages with their algorithmic rate."""
    st = {}
    for name in ("route", "dispatch", "latent_down", "expert_gate_up", "expert_down",
                 "shared_gate_up", "combine"):
        if name == "latent_down" and not w.latent:
            continue
        if name == "shared_gate_up" and (not w.d_shared or plan["merged_shared"]):
            continue
        reps = 20 if name in REPEATABLE else 1
        ms = stage_ms(layer, x, out, counts, name, reps)
        rec = {"ms": round(ms, 4)}
        fl = {"expert_gate_up": alg["gu_flops"], "expert_down": alg["dn_flops"],
              "shared_gate_up": alg["sh_gu_flops"],
              "latent_down": 2.0 * w.T * w.d * w.latent}.get(name)
        by = {"expert_gate_up": alg["gu_bytes"], "expert_down": alg["dn_bytes"],
              "shared_gate_up": alg["sh_gu_bytes"]}.get(name)
        if fl:
            rec["tflops"] = round(fl / (ms / 1e3) / 1e12, 1)
            rec["frac_of_mfma_peak"] = round(fl / (ms / 1e3) / 1e12 / peak_tf, 4)
        if by:
            rec["gbs"] = round(by / (ms / 1e3) / 1e9, 1)
        st[name] = rec
    return st


def roofline_of(alg, gu_ms, peak_tf, name, plan):
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
    roof["traffic"] = measured_traffic(name)
    roof["kernel"] = "grouped gate/up GEMM + SiLU*up" + (
        " (+ the shared experts' gate/up GEMM in the same launch)" if plan["merged_shared"] else "")
    roof["tile"] = f"{plan['gate_up_tile_m']}x{plan['gate_up_tile_n']}"
    roof["kernel_ms"] = round(gu_ms, 4)
    roof["algorithmic"] = (f"{alg['gu_flops'] / 1e12:.4f} TFLOP, {alg['gu_bytes'] / 1e9:.4f} GB "
                           "per launch")
    roof["timing"] = ("mean of 5 x 20 back-to-back launches between HIP events on the launch "
                      "stream, after the timed steps")
    return roof


def layer_rates(alg, ms, peak_tf):
    return {"algorithmic_tflop": round(alg["flops"] / 1e12, 5),
            "tflops": round(alg["flops"] / (ms / 1e3) / 1e12, 2),
            "frac_of_mfma_peak": round(alg["flops"] / (ms / 1e3) / 1e12 / peak_tf, 4),
            "algorithmic_gb": round(alg["bytes"] / 1e9, 4),
            "gbs": round(alg["bytes"] / (ms / 1e3) / 1e9, 1),
            "frac_of_hbm_peak": round(alg["bytes"] / (ms / 1e3) / 1e9 / HBM_GBS, 4),
            "experts_touched": alg["touched"]}


# ------------------------------------------------------------ CPU oracle

def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _omp_threads(n):
    """Thread count of the oracle's OpenMP loops (its runtime is libgomp)."""
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
        return True
    except OSError:
        return False


def _time_sample(orc, w, rng, budget_s):
    probe = rng.choice(w.T, size=min(w.T, 8), replace=False)
    t0 = time.perf_counter()
    orc.forward(tokens=probe)
    per_tok = (time.perf_counter() - t0) / len(probe)
    n = int(max(8, min(w.T, budget_s / max(per_tok, 1e-9))))
    toks = np.sort(rng.choice(w.T, size=n, replace=False))
    t0 = time.perf_counter()
    orc.forward(tokens=toks)
    dt = time.perf_counter() - t0
    passes = 1  # a whole batch shorter than the budget: repeat it (up to 10 passes)
    while n == w.T and dt < 0.8 * budget_s and passes < 10:
        orc.forward(tokens=toks)
        passes += 1
        dt = time.perf_counter() - t0
    return n, passes, dt


def cpu_baseline(w, a, budget_s=12.0, budget_1_s=6.0):
    """Time the CPU oracle (as it stands) on seeded token samples: all host
    cores, then one core; and its routing + dispatch over all T tokens."""
    import oracle
    orc = oracle.Oracle(w, a)
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    _omp_threads(cores)
    n, passes, dt = _time_sample(orc, w, np.random.default_rng(7), budget_s)
    rep = f" x {passes} passes" if passes > 1 else ""
    res = {"value": n * passes / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"{n} of {w.T} tokens (seeded){rep}, full layer per token in fp64 "
                     f"(per-token cost is independent of the other tokens), {dt:.1f} s",
           "cpu_model": _cpu_model()}
    if _omp_threads(1):
        n1, p1, dt1 = _time_sample(orc, w, np.random.default_rng(8), budget_1_s)
        res["one_core"] = {"value": n1 * p1 / dt1, "unit": "tokens/s", "cores": 1,
                           "sample": f"{n1} tokens x {p1} passes, {dt1:.1f} s"}
        _omp_threads(cores)
    t0 = time.perf_counter()
    idx, g, _, _ = orc.route()
    t1 = time.perf_counter()
    oracle.dispatch(idx, g.astype(np.float32), w.E)
    t2 = time.perf_counter()
    res["route_dispatch_all_tokens"] = {"tokens": w.T, "route_s": round(t1 - t0, 3),
                                        "dispatch_s": round(t2 - t1, 3), "cores": cores,
                                        "tokens_per_s": round(w.T / (t2 - t0), 1)}
    return res


# ------------------------------------------------------------ main

def run_workload(w, a_dev, steps, warmup, probe_stages=True):
    """Time one workload on resident device tensors; returns the pieces of
    its bench record."""
    import torch
    import mixture_experts_ffn_fp32_amd as moe
    dev = torch.device("cuda:0")
    layer = moe.Layer(w, a_dev, device=dev)
    x = layer.dev["x"]
    out = torch.empty((w.T, w.d), dtype=layer.act, device=dev)
    counts = torch.zeros(w.E, dtype=torch.int32, device=dev)
    ms, step_ms = timed_steps(layer, x, out, counts, steps, warmup)
    gu_ms = stage_ms(layer, x, out, counts, "expert_gate_up", 20)
    cnt = counts.cpu().numpy()
    plan = moe.moe_plan(layer.desc)
    alg = algorithmic(w, cnt, merged=bool(plan["merged_shared"]))
    peak_tf = PEAK[w.act]
    rec = {"ms": ms, "step_ms": step_ms, "alg": alg, "plan": plan, "counts": cnt,
           "roofline": roofline_of(alg, gu_ms, peak_tf, w.name, plan),
           "layer": layer_rates(alg, ms, peak_tf),
           "layer_obj": layer, "x": x, "out": out, "counts_t": counts}
    if probe_stages:
        rec["stages"] = stages_of(layer, x, out, counts, w, alg, plan, peak_tf)
    return rec


def expert_shard(spec: str, workload: str, reps: int = 10):
    """One GPU's share of an expert-parallel layer of G GPUs (experts
    [g E/G, (g+1) E/G) on this GPU): the grouped expert SwiGLU on the rows
    routed to those experts (their true count, from the whole batch's routing
    and dispatch), plus routing, dispatch, shared experts and combine for this
    GPU's T/G tokens. The all-to-all exchanges between them are not part of a
    one-GPU run; they are left out of the sum, which says so."""
    import torch

    import mixture_experts_ffn_fp32_amd as moe
    import moe_synth
    g, G = (int(v) for v in spec.split("/"))
    w = moe_synth.get(workload)
    if not (0 <= g < G and w.E % G == 0 and w.T % G == 0) or w.latent:
        raise SystemExit(f"--expert-shard {spec}: need 0 <= g < G, G dividing E={w.E} and T={w.T}, "
                         "and a layer without latent projections")
    a = moe_synth.generate(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d_all = moe.to_device(a, dev)
    layer = moe.Layer(w, d_all, device=dev)
    i32 = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    T, K, E = w.T, w.K, w.E
    idx, gw = i32((T, K)), torch.empty((T, K), dtype=torch.float32, device=dev)
    moe.moe_route(layer.desc, layer.weights, d_all["x"], idx, gw, ws=layer.ws)
    counts, offsets, perm, st, inv = i32(E), i32(E + 1), i32(T * K), i32(T * K), i32(T * K)
    sw = torch.empty(T * K, dtype=torch.float32, device=dev)
    moe.moe_dispatch(layer.desc, idx, gw, None, counts, offsets, perm, st, inv, sw, None, layer.ws)
    torch.cuda.synchronize()
    e0, e1 = g * E // G, (g + 1) * E // G
    off = offsets.cpu().numpy()
    lo, hi = int(off[e0]), int(off[e1])
    # the shard: E/G experts, their rows [lo, hi) of the sorted order
    ws_ = dataclasses.replace(w, E=E // G)
    desc_s = moe.make_desc(ws_)
    shard_w = {k: d_all[k][e0:e1] for k in ("w_gate", "w_up", "w_down")}
    shard_w["w_router"] = d_all["w_router"][e0:e1]
    weights_s = moe.make_weights(shard_w)
    offs_s = (offsets[e0:e1 + 1] - lo).contiguous()
    y = torch.empty((T * K, w.d_e), dtype=layer.act, device=dev)
    ws_s = torch.empty(moe.moe_workspace_size(desc_s), dtype=torch.uint8, device=dev)
    row_idx, row_w = st[lo:hi], sw[lo:hi]

    def ffn():
        moe.moe_expert_ffn(desc_s, weights_s, d_all["x"], row_idx, offs_s, row_w, y, ws_s)

    def timed(fn):
        fn()
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return b.elapsed_time(e) / reps

    ffn_ms = timed(ffn)
    rows = hi - lo
    fl = 6.0 * rows * w.d_e * w.d_ff
    # this GPU's T/G tokens: routing + dispatch, shared experts + combine
    wt = w.with_T(T // G)
    lt = moe.Layer(wt, {**d_all, "x": d_all["x"][: T // G]}, device=dev)
    idx_t, g_t = i32((wt.T, K)), torch.empty((wt.T, K), dtype=torch.float32, device=dev)
    c_t, o_t, p_t, s_t, v_t = i32(E), i32(E + 1), i32(wt.T * K), i32(wt.T * K), i32(wt.T * K)
    w_t = torch.empty(wt.T * K, dtype=torch.float32, device=dev)
    y_t = torch.zeros((wt.T * K, w.d_e), dtype=layer.act, device=dev)
    out_t = torch.empty((wt.T, w.d), dtype=layer.act, device=dev)

    def route_dispatch():
        moe.moe_route(lt.desc, lt.weights, lt.dev["x"], idx_t, g_t, ws=lt.ws)
        moe.moe_dispatch(lt.desc, idx_t, g_t, None, c_t, o_t, p_t, s_t, v_t, w_t, None, lt.ws)

    def combine():
        moe.moe_combine(lt.desc, lt.weights, lt.dev["x"], y_t, v_t, out_t, lt.ws)

    rd_ms = timed(route_dispatch)
    cb_ms = timed(combine)
    loads = counts.cpu().numpy()
    per_gpu = [int(loads[k * E // G:(k + 1) * E // G].sum()) for k in range(G)]
    rec = {"expert_shard": spec, "workload": workload, "experts": [e0, e1], "rows": rows,
           "rows_per_gpu_min_max": [min(per_gpu), max(per_gpu)],
           "expert_ffn_ms": round(ffn_ms, 4), "expert_ffn_tflops": round(fl / ffn_ms / 1e9, 1),
           "route_dispatch_ms_tokens_of_this_gpu": round(rd_ms, 4),
           "shared_and_combine_ms_tokens_of_this_gpu": round(cb_ms, 4),
           "sum_ms_without_all_to_all": round(ffn_ms + rd_ms + cb_ms, 4),
           "note": "one GPU's share of an expert-parallel layer; the two all-to-all exchanges "
                   "(rows to the expert owners and back) are not measured"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass timing")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-batch timing of the same layer")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage timings")
    ap.add_argument("--peak", action="store_true",
                    help="only run the peak-rate microbenchmarks (MFMA issue, LDS reads)")
    ap.add_argument("--calibrate-copy", type=int, metavar="MiB", default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    ap.add_argument("--expert-shard", metavar="g/G", default=None,
                    help="only time one GPU's share (experts g E/G .. (g+1) E/G) of an "
                         "expert-parallel layer over G GPUs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); sharding the "
              "layer over several GPUs is not implemented (--expert-shard g/G times one "
              "GPU's share of an expert-parallel layer)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.peak:
        print(json.dumps({"peak_rates": peak_rates()}), flush=True)
        return
    if args.expert_shard:
        expert_shard(args.expert_shard, args.workload)
        return

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
    a_dev = moe.to_device(a, dev)
    stream = torch.cuda.current_stream()
    r = run_workload(w, a_dev, args.steps, args.warmup, probe_stages=not args.no_stages)
    layer, x, out, counts = r["layer_obj"], r["x"], r["out"], r["counts_t"]
    ms, alg, cnt = r["ms"], r["alg"], r["counts"]
    peak_tf = PEAK[w.act]
    log(f"step {ms:.4f} ms (events: {r['step_ms']}), {w.T / (ms / 1e3):.4g} tokens/s; "
        f"gate/up kernel {r['roofline']['kernel_ms']:.4f} ms; experts touched "
        f"{alg['touched']}/{w.E}; loads max {cnt.max()} min {cnt.min()}")
    if "stages" in r:
        log(f"stages: {r['stages']}")

    # measured MFMA peak of this part (two wavefronts per SIMD), for the
    # fraction against the running clock beside the datasheet's
    meas = peak_rates(modes=(0,), threads=(512,), iters=2000)[0]

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

    # the same resident weights at the decode batch
    decode = None
    if w.name in DECODE_OF and not args.no_decode:
        wd = moe_synth.get(DECODE_OF[w.name])
        ad = moe_synth.generate(wd, experts=False)
        assert np.array_equal(ad["w_router"], a["w_router"]), "decode layer differs"
        dd = dict(a_dev)
        dd["x"] = moe.to_device({"x": ad["x"]}, dev)["x"]
        rd = run_workload(wd, dd, max(args.steps, 100), max(args.warmup, 20), probe_stages=False)
        decode = {"workload": wd.name, "tokens": wd.T,
                  "value": round(wd.T / (rd["ms"] / 1e3), 1),
                  "unit": "tokens/s", "ms_per_step": round(rd["ms"], 5),
                  "step_ms": rd["step_ms"], "layer": rd["layer"], "roofline": rd["roofline"],
                  "note": "same weights as the prefill layer, own tokens; the layer's bound is "
                          "HBM: layer.frac_of_hbm_peak = touched expert + shared + router "
                          "weight bytes / mean step"}
        log(f"decode: {decode}")
        del rd
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, a)
        log(f"cpu baseline: {cpu}")

    roof = r["roofline"]
    if roof["bound"] == "mfma":
        roof["frac_of_measured_peak"] = round(roof["achieved"] / meas["tflops"], 4)
    line = {
        "metric": METRIC,
        "value": round(w.T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "step_ms": r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "d_model": w.d, "d_ff": w.d_ff,
                   "experts": w.E, "top_k": w.K, "shared_width": w.d_shared,
                   "latent": w.latent, "route": w.route, "parallelism": "single-gpu"},
        "layer": r["layer"],
        "roofline": roof,
        "stages": r.get("stages"),
        "decode": decode,
        "measured_mfma_peak": meas,
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
