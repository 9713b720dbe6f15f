"""Benchmark of the MoE FFN layer forward pass on one MI355X.

One step = one moe_forward call (route, group, expert GEMMs, combine, aux) over
one batch of seeded synthetic input already resident in HBM.

Headline (`value`): tokens/s on the Mixtral-shaped prefill layer (T=4096,
d=4096, E=8, top-2, SwiGLU width 14336, bf16). The decode-shaped layer (T=16),
the Switch-style top-1 layer (T=8192, E=64, width 1376), the two small layers
(micro fp32, skewed small experts) and the backward pass of the prefill layer
are reported in extra objects of the same JSON line. The large layers carry a
roofline for their dominant kernel: algorithmic flops or bytes per launch
divided by that kernel's mean duration, measured with HIP events that the
library records on the launch stream during the timed region. Every layer
also reports per-step event times (median, minimum), launches per step and
the layer's roofline fraction max(F / F_peak, B / B_peak) / t; decode and
Switch also cold-cache times (two copies of the weights, alternated), and
`context` the box's plain-copy rate and the vendor GEMM on one expert's shape.

cpu_baseline: the CPU oracle (never tuned) on a bounded sample of the
prefill workload: the same layer restricted to its first tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_mixture_experts_48_amd as moe  # noqa: E402
from sparse_mixture_experts_48_amd import workloads as W  # noqa: E402

METRIC = "MoE-layer tokens/s + TFLOP/s (% MFMA peak) prefill; HBM GB/s (% peak) decode"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def bpe(cfg):
    return 2 if cfg.dtype == W.DT_BF16 else 4


def algorithmic(cfg, counts):
    """Flops and bytes the method itself needs (only experts that are hit are read)."""
    n_mat = 3 if cfg.act == W.ACT_SWIGLU else 2
    hit = int((counts > 0).sum())
    flops_router = 2.0 * cfg.T * cfg.d * cfg.E
    flops_g1 = 2.0 * cfg.S * cfg.d * cfg.width * (n_mat - 1)
    flops_g2 = 2.0 * cfg.S * cfg.width * cfg.d
    b = bpe(cfg)
    w_g1 = hit * (n_mat - 1) * cfg.width * cfg.d * b + (hit * cfg.width * b if cfg.act == W.ACT_GELU else 0)
    w_g2 = hit * cfg.d * cfg.width * b + (hit * cfg.d * b if cfg.act == W.ACT_GELU else 0)
    bytes_total = cfg.T * cfg.d * b * 2 + cfg.d * cfg.E * 4 + w_g1 + w_g2
    return {"flops": flops_router + flops_g1 + flops_g2, "flops_gemm1": flops_g1, "flops_gemm2": flops_g2,
            "bytes": bytes_total, "weight_bytes_gemm1": w_g1, "weight_bytes_gemm2": w_g2, "experts_hit": hit}


def layer_roofline_frac(cfg, alg, ms):
    """max(F / F_peak, B / B_peak) / t: the ideal time at the binding peak over the measured time."""
    peak = PEAK_BF16_TFLOPS if cfg.dtype == W.DT_BF16 else PEAK_F32_TFLOPS
    return round(max(alg["flops"] / (peak * 1e12), alg["bytes"] / (PEAK_HBM_GBPS * 1e9)) / (ms * 1e-3), 4)


def step_times(run, steps):
    """Per-step durations (ms) of `run` from HIP events on the current stream
    (the stream the library launches on)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def time_workload(cfg, steps, warmup, label, cold=False):
    """Eager and graph-replayed steps of moe_forward, the library's per-launch
    events, and per-step event times. cold: alternate between two copies of the
    weights, so that no weight byte can still be in the 256 MB Infinity Cache
    from the previous step (the step times are then the cold ones)."""
    sys.stderr.write("[bench] %s: generating inputs %s\n" % (label, cfg))
    sys.stderr.flush()
    inp = W.make_inputs(cfg)
    layer = moe.MoELayer(cfg, inp)
    twin = moe.MoELayer(cfg, inp) if cold else None
    del inp
    for _ in range(warmup):
        layer.forward()
    torch.cuda.synchronize()
    counts = layer.counts.cpu().numpy()
    sys.stderr.write("[bench] %s: timing %d steps\n" % (label, steps))
    sys.stderr.flush()
    # wall-clock steps with the library's tracing off (the headline figure) ...
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    # ... then the same steps again with HIP events around every launch (per-kernel times)
    with moe.Trace(capacity=16 * steps + 16) as tr:
        for _ in range(steps):
            layer.forward()
        torch.cuda.synchronize()
        events = tr.read()
    # the same step replayed from a captured HIP graph (no per-kernel launch gaps)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        layer.forward()
    g.replay()
    torch.cuda.synchronize()
    tg0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms_graph = (time.perf_counter() - tg0) * 1e3 / steps
    del g
    per_step = step_times(layer.forward, steps)
    cold_steps = None
    if twin is not None:
        flip = [0]

        def alternate():
            (layer if flip[0] % 2 == 0 else twin).forward()
            flip[0] += 1
        cold_steps = step_times(alternate, 2 * steps)
        del twin
    per_kernel = {}
    for name, dur in events:
        per_kernel.setdefault(name, []).append(dur)
    kernels = {k: {"mean_ms": float(np.mean(v)), "launches_per_step": len(v) / steps}
               for k, v in per_kernel.items()}
    alg = algorithmic(cfg, counts)
    aux = float(layer.aux.cpu()[0])
    del layer
    torch.cuda.empty_cache()
    stats = {"ms_median": round(float(np.median(per_step)), 4), "ms_min": round(float(np.min(per_step)), 4),
             "launches_per_step": round(len(events) / steps, 2),
             "layer_roofline_frac": layer_roofline_frac(cfg, alg, float(np.median(per_step)))}
    if cold_steps is not None:
        stats["cold_ms_median"] = round(float(np.median(cold_steps)), 4)
        stats["cold_ms_min"] = round(float(np.min(cold_steps)), 4)
        stats["cold_layer_roofline_frac"] = layer_roofline_frac(cfg, alg, float(np.median(cold_steps)))
    return ms, kernels, alg, counts, aux, ms_graph, stats


def time_backward(cfg, steps, warmup):
    """moe_backward on one layer (first-GEMM recompute + gradients of every input)."""
    sys.stderr.write("[bench] backward %s: generating inputs\n" % cfg.name)
    sys.stderr.flush()
    inp = W.make_inputs(cfg)
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    del inp
    g = torch.Generator().manual_seed(cfg.seed + 1000)
    dy = torch.randn((cfg.T, cfg.d), generator=g).to(torch.bfloat16).cuda()
    desc = moe.desc_of(cfg)
    ws = moe.backward_workspace(desc)

    def step():
        return moe.backward(desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"], dev["W3"], dev["W2"],
                            dev["b2"], dy, 0.01, ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    sys.stderr.write("[bench] backward: timing %d steps\n" % steps)
    sys.stderr.flush()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps  # tracing off
    with moe.Trace(capacity=64 * steps + 64) as tr:
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        events = tr.read()
    per_call = len(events) // steps
    calls = [events[i * per_call:(i + 1) * per_call] for i in range(steps)]

    def launches(name):  # durations of the launches of `name`, in call order
        return [[ms_ for n, ms_ in c if n == name] for c in calls]

    wg = launches("wgrad")
    g1 = launches("gemm1")
    per_kernel = {}
    for name, dur in events:
        per_kernel.setdefault(name, []).append(dur)
    del ws, dev
    torch.cuda.empty_cache()
    return ms, {"dW13_ms": float(np.mean([c[-1] for c in wg])), "dW2_ms": float(np.mean([c[0] for c in wg])),
                "dX_ms": float(np.mean([c[-1] for c in g1])),
                "kernels_ms": {k: round(float(np.sum(v)) / steps, 4) for k, v in per_kernel.items()},
                "launches_ms": [[calls[0][i][0], round(float(np.mean([c[i][1] for c in calls])), 4)]
                                for i in range(per_call)]}


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary of `workload` (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy);
    None if there is none or the kernel source changed since it was taken."""
    from sparse_mixture_experts_48_amd import profiling
    return profiling.traffic_bytes(os.path.join(ROOT, "profiles", "hbm_traffic_%s.md" % workload), kernel, ROOT)


def roofline_mfma(flops, mean_ms, peak, traffic=None):
    achieved = flops / (mean_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic}


def roofline_hbm(nbytes, mean_ms, traffic=None):
    achieved = nbytes / (mean_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic}


def small_workload(name, steps, warmup):
    """The latency-bound layers (micro fp32, skewed small experts): step times,
    launches and the roofline fraction, which is small by nature at these sizes."""
    c = W.WORKLOADS[name]
    ms, k, alg, counts, aux, ms_g, st = time_workload(c, steps, warmup, name)
    return {"workload": name, "ms_per_step": round(ms, 4), "ms_per_step_graph": round(ms_g, 4),
            "tokens_per_s": round(c.T / (st["ms_median"] * 1e-3), 1),
            "tokens_per_s_graph": round(c.T / (ms_g * 1e-3), 1), **st,
            "layer_tflops": round(alg["flops"] / (st["ms_median"] * 1e-3) / 1e12, 3),
            "layer_hbm_GBps": round(alg["bytes"] / (st["ms_median"] * 1e-3) / 1e9, 1),
            "aux_loss": round(aux, 6), "experts_hit": alg["experts_hit"], "idle_experts": int((counts == 0).sum()),
            "max_expert_share": round(float(counts.max()) / max(c.S, 1), 4),
            "kernels_ms": {kk: round(v["mean_ms"], 4) for kk, v in k.items()}}


def context_ceilings():
    """Practical ceilings on this machine, as context (not dependencies of the
    path): a plain 1 GiB device copy, and torch.matmul (the vendor GEMM) on one
    expert's first-GEMM shape, 1024 x 4096 x 28672 in bf16."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    t = float(np.median(step_times(lambda: dst.copy_(src), 10)))
    copy_gbps = 2 * (1 << 30) / (t * 1e-3) / 1e9
    del src, dst
    a = torch.randn(1024, 4096, device="cuda").to(torch.bfloat16)
    b = torch.randn(4096, 28672, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    t = float(np.median(step_times(lambda: torch.matmul(a, b), 10)))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_1GiB_GBps_read_plus_write": round(copy_gbps, 1),
            "vendor_gemm_1024x4096x28672_bf16_tflops": round(2.0 * 1024 * 4096 * 28672 / (t * 1e-3) / 1e12, 1)}


def cpu_baseline(cfg, n_tokens):
    """The CPU oracle on the first n_tokens tokens of the workload (same weights)."""
    from oracle import moe_oracle as O
    sub = cfg.with_(T=n_tokens)
    inp = W.make_inputs(cfg)
    p = {"h": W.as_float32(inp["h"][:n_tokens]), "W_r": W.as_float32(inp["W_r"]),
         "b_r": W.as_float32(inp["b_r"])}

    class PerExpert:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return W.as_float32(self.t[e])

    for k in ("W1", "W3", "W2", "b1", "b2"):
        p[k] = None if inp[k] is None else PerExpert(inp[k])
    O.build()
    t0 = time.perf_counter()
    O.moe_forward(p, sub.T, sub.d, sub.E, sub.K, sub.act, sub.gate)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "first %d of %d tokens of %s (full layer: routing, %d experts' float64 FFNs, combine, "
                      "aux); %.1f s wall" % (n_tokens, cfg.T, cfg.name, cfg.E, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="time only the prefill workload")
    ap.add_argument("--only", choices=["prefill", "decode", "switch", "backward"], default=None,
                    help="time one workload only (for per-workload profiles); prints its own JSON object")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="also run a plain device-to-device copy of this many MiB (a reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X only: this layer's path is built and measured on a single GPU "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    moe.lib()  # fail loudly if the HIP library is missing
    if args.calibrate_copy > 0:
        src = torch.empty(args.calibrate_copy << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only == "backward":
        c = W.WORKLOADS["mixtral_prefill"]
        bms, bk = time_backward(c, args.steps, args.warmup)
        print(json.dumps({"workload": c.name, "backward_ms_per_step": round(bms, 4), **bk}))
        return
    if args.only is not None:
        name = {"prefill": "mixtral_prefill", "decode": "mixtral_decode", "switch": "switch_top1"}[args.only]
        c = W.WORKLOADS[name]
        ms, kernels, alg, counts, aux, msg, _ = time_workload(c, args.steps, args.warmup, args.only)
        print(json.dumps({"workload": name, "ms_per_step": round(ms, 4), "ms_per_step_graph": round(msg, 4),
                          "tokens_per_s": round(c.T / (ms * 1e-3), 1),
                          "kernels_ms": {k: round(v["mean_ms"], 4) for k, v in kernels.items()}}))
        return

    cfg = W.WORKLOADS["mixtral_prefill"]
    ms, kernels, alg, counts, aux, ms_g, pstats = time_workload(cfg, args.steps, args.warmup, "prefill")
    g1 = kernels["gemm1"]["mean_ms"]
    out = {
        "metric": METRIC,
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_graph": round(ms_g, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal inputs, random-init weights; no dataset)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "K": cfg.K, "width": cfg.width,
                   "act": "swiglu", "gate": "renorm", "router": "float32", "parallelism": "single GPU"},
        "roofline": dict(roofline_mfma(alg["flops_gemm1"], g1, PEAK_BF16_TFLOPS,
                                       measured_traffic(cfg.name, "gemm1")), kernel="gemm1",
                         algorithmic_bytes=int(alg["weight_bytes_gemm1"] + cfg.T * cfg.d * bpe(cfg)
                                               + cfg.S * cfg.width * bpe(cfg))),
        "layer_tflops": round(alg["flops"] / (ms * 1e-3) / 1e12, 2),
        "layer_mfma_frac": round(alg["flops"] / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        **pstats,
        "aux_loss": round(aux, 6),
        "kernels_ms": {k: round(v["mean_ms"], 4) for k, v in kernels.items()},
    }
    if not args.no_extra:
        dcfg = W.WORKLOADS["mixtral_decode"]
        dsteps = max(args.steps, 50)
        dms, dk, dalg, dcounts, _, dms_g, dstats = time_workload(dcfg, dsteps, args.warmup, "decode", cold=True)
        out["decode"] = {**dstats,
            "workload": dcfg.name, "steps": dsteps, "ms_per_step": round(dms, 4),
            "ms_per_step_graph": round(dms_g, 4), "tokens_per_s_graph": round(dcfg.T / (dms_g * 1e-3), 1),
            "layer_hbm_frac_graph": round(dalg["bytes"] / (dms_g * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "tokens_per_s": round(dcfg.T / (dms * 1e-3), 1),
            "layer_hbm_GBps": round(dalg["bytes"] / (dms * 1e-3) / 1e9, 1),
            "layer_hbm_frac": round(dalg["bytes"] / (dms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "experts_hit": dalg["experts_hit"],
            "roofline": dict(roofline_hbm(dalg["weight_bytes_gemm1"], dk["gemm1"]["mean_ms"],
                                          measured_traffic(dcfg.name, "gemm1")), kernel="gemm1"),
            "roofline_gemm2": dict(roofline_hbm(dalg["weight_bytes_gemm2"], dk["gemm2"]["mean_ms"],
                                                measured_traffic(dcfg.name, "gemm2")), kernel="gemm2"),
            "kernels_ms": {k: round(v["mean_ms"], 4) for k, v in dk.items()},
        }
        scfg = W.WORKLOADS["switch_top1"]
        sms, sk, salg, scounts, saux, sms_g, sstats = time_workload(scfg, args.steps, args.warmup, "switch",
                                                                    cold=True)
        out["switch_top1"] = {**sstats,
            "workload": scfg.name, "ms_per_step": round(sms, 4), "ms_per_step_graph": round(sms_g, 4),
            "tokens_per_s": round(scfg.T / (sms * 1e-3), 1),
            "layer_tflops": round(salg["flops"] / (sms * 1e-3) / 1e12, 2),
            "layer_hbm_GBps": round(salg["bytes"] / (sms * 1e-3) / 1e9, 1),
            "layer_hbm_frac": round(salg["bytes"] / (sms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "roofline": dict(roofline_hbm(salg["weight_bytes_gemm1"], sk["gemm1"]["mean_ms"],
                                          measured_traffic(scfg.name, "gemm1")), kernel="gemm1"),
            "aux_loss": round(saux, 6), "experts_hit": salg["experts_hit"],
            "max_expert_rows": int(scounts.max()),
            "kernels_ms": {k: round(v["mean_ms"], 4) for k, v in sk.items()},
        }
    if not args.no_extra:
        out["micro"] = small_workload("micro", max(args.steps, 200), args.warmup)
        out["skewed"] = small_workload("skewed", max(args.steps, 200), args.warmup)
        out["context"] = context_ceilings()
        bcfg = W.WORKLOADS["mixtral_prefill"]
        bms, bk = time_backward(bcfg, max(args.steps // 4, 3), 2)
        F = 2.0 * bcfg.S * bcfg.d * bcfg.width * 3  # forward expert flops (SwiGLU: 3 matrices)
        f13 = 2.0 * bcfg.S * (2 * bcfg.width) * bcfg.d  # dW1 and dW3 together
        out["backward"] = {
            "workload": bcfg.name, "ms_per_step": round(bms, 4),
            "tokens_per_s": round(bcfg.T / (bms * 1e-3), 1),
            "gradient_tflops": round(2 * F / (bms * 1e-3) / 1e12, 2),
            "note": "moe_backward: input and weight gradients of the expert FFNs (2F, the flops counted) plus a "
                    "recompute of the first expert GEMM (2F/3), router gradient, dh",
            "roofline": dict(roofline_mfma(f13, bk["dW13_ms"], PEAK_BF16_TFLOPS), kernel="wgrad dW1+dW3"),
            "dX_tflops": round(f13 / (bk["dX_ms"] * 1e-3) / 1e12, 2),
            "dW2_tflops": round(F / 3 / (bk["dW2_ms"] * 1e-3) / 1e12, 2),
            "kernels_ms": bk["kernels_ms"], "launches_ms": bk["launches_ms"],
        }
    if not args.no_cpu:
        sys.stderr.write("[bench] cpu baseline: oracle on %d tokens\n" % args.cpu_tokens)
        sys.stderr.flush()
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_tokens)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
