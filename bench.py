"""Benchmark: one GPU's share of a sparse MoE layer on MI355X through libmoe.

A step is one pass of the whole hot path over one batch of synthetic input:
router logits -> route -> dispatch layout -> permute -> grouped gate/up GEMM +
SwiGLU -> grouped down GEMM -> shared expert (when the workload has one) -> combine.  Inputs and
weights are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config dsv3_bf16]

Prints one JSON line.  Kernel durations come from HIP events recorded on the
stream the kernels run on, around every call of every timed step.  `kernels` holds
the warm figures of the back-to-back steps that `value` is taken from;
`kernels_cold` the same stages timed again with L2 and the MALL flushed before
each one (their GB/s then count HBM reads, not cache hits).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_MFMA = {"bf16": 2.5e15, "fp8": 5.0e15, "f32": 157.3e12}
METRIC = "MoE-layer tokens/s; grouped-GEMM MFMA util; permute/combine HBM GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_traffic_{}.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="dsv3_bf16")
    p.add_argument("--cpu-tokens", type=int, default=-1,
                   help="tokens of the batch the CPU oracle runs for the baseline (-1 = the whole batch, "
                        "0 = skip)")
    p.add_argument("--other-configs", default="all",
                   help="comma-separated workloads also timed (compactly) into other_configs, 'all' (every "
                        "workload but --config) or 'none'")
    p.add_argument("--other-steps", type=int, default=10, help="timed steps per other workload")
    p.add_argument("--chunks", type=int, default=2,
                   help="also time the layer cut into this many chunks of tokens, each chunk's combine on a "
                        "second stream beside the next chunk's GEMMs (A/B against the unchunked layer; 1 = skip)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (calibrates HBM byte counters)")
    p.add_argument("--gate-in-down", action="store_true",
                   help="multiply the routed rows by their gates in the down GEMM's epilogue; combine sums")
    p.add_argument("--no-fuse-shared", action="store_true",
                   help="run the shared expert as launches of its own instead of inside the routed GEMMs")
    p.add_argument("--no-gather", action="store_true",
                   help="bf16: run the permute and read the gate/up rows from its copy")
    p.add_argument("--overlap", action="store_true",
                   help="run the shared expert on a second stream beside the routed path (it then "
                        "holds the CUs while route/layout wait, so per-stage times mix)")
    p.add_argument("--train", action="store_true",
                   help="time a training step instead: the forward, then the backward pass for a fixed "
                        "upstream gradient (bf16 layers; weight gradients in bf16)")
    p.add_argument("--overlap-backward", action="store_true",
                   help="--train: run the shared expert's backward on a second stream beside the routed "
                        "backward (the backward is then one timed stage)")
    p.add_argument("--graph", action="store_true",
                   help="also capture one step in a HIP graph and time its replays; value is then the "
                        "replayed throughput (the per-kernel figures stay those of the eager steps)")
    p.add_argument("--cold-steps", type=int, default=5,
                   help="extra steps timed with L2 and the 256 MB MALL flushed (1 GiB written) before "
                        "every stage, so each stage reads its inputs from HBM (0 = skip)")
    p.add_argument("--rows-per-expert", type=int, default=0,
                   help="diagnostic: replace the router's routes by fixed ones giving exactly this many rows to "
                        "each of as many experts as the batch fills (the batch shrinks to a multiple that fits); "
                        "the step is then layout, GEMMs and combine")
    p.add_argument("--quiet", action="store_true")
    return p.parse_args()


def log(args, msg):
    if not args.quiet:
        print(msg, file=sys.stderr, flush=True)


def source_sha(*paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# sources of the dominant kernel (the routed gate/up GEMM): a stored traffic figure is used
# only while they are unchanged since its counters were taken
GEMM_SOURCES = [os.path.join(ROOT, "combine_grouped_gemm_amd", "csrc", n)
                for n in ("grouped_gemm_wide.hip", "gemm_device.h", "moe_common.h")]


def algorithmic(cfg, n_e, gather=False, fused=False):
    """Algorithmic bytes and flops of each step (what the method must move or compute).

    gather: the gate/up GEMM reads its rows straight from x (each token row at least once)
    instead of from a permuted copy.  fused: the shared expert runs inside the routed
    gate/up and down launches (its work is counted there)."""
    import numpy as np
    N, H, E, k, I = cfg.N, cfg.H, cfg.E, cfg.k, cfg.I
    rows = N * k
    act = 4 if cfg.dtype == "f32" else 2          # x, h, expert outputs, y
    pay = 1 if cfg.dtype == "fp8" else act        # permuted payload
    wb = 1 if cfg.dtype == "fp8" else act         # weights
    touched = int((np.asarray(n_e) > 0).sum())
    fp8_scale = 4.0 / 128 if cfg.dtype == "fp8" else 0.0
    d = {}
    d["router"] = {"bytes": N * H * act + E * H * act + N * E * 4, "flops": 2.0 * N * H * E}
    d["route"] = {"bytes": N * E * 4 + (E * 4 if cfg.zipf_s else 0) + rows * 8}
    d["layout"] = {"bytes": rows * 4 + (2 * E + 1) * 4 + 2 * rows * 4}
    d["permute"] = {"bytes": N * H * act + rows * H * (pay + fp8_scale)}
    if gather and cfg.dtype == "fp8":   # each token quantized once (codes, scales), then its bf16 values
        d["permute"] = {"bytes": N * H * act + 2 * N * H * (1 + fp8_scale) + N * H * act}
    a_bytes = N * H * act if gather else rows * H * (pay + fp8_scale)
    d["gate_up"] = {"bytes": touched * 2 * I * H * (wb + fp8_scale) + a_bytes + rows * I * 2,
                    "flops": 4.0 * rows * H * I}
    d["down"] = {"bytes": touched * H * I * (wb + fp8_scale) + rows * I * 2 + rows * H * act,
                 "flops": 2.0 * rows * H * I}
    if cfg.shared and fused:
        d["gate_up"]["bytes"] += 2 * I * H * (wb + fp8_scale) + N * I * 2     # x is read once for both
        d["gate_up"]["flops"] += 4.0 * N * H * I
        d["down"]["bytes"] += H * I * (wb + fp8_scale) + N * I * 2 + N * H * act
        d["down"]["flops"] += 2.0 * N * H * I
    elif cfg.shared:
        d["shared"] = {"bytes": 3 * I * H * wb + N * H * act + N * I * 2 + N * H * act,
                       "flops": 6.0 * N * H * I}
    d["combine"] = {"bytes": (rows + (N if cfg.shared else 0)) * H * act + N * H * act + rows * 8}
    return d


def algorithmic_backward(cfg, n_e):
    """Algorithmic bytes and flops of each backward step (bf16 operands and gradients)."""
    import numpy as np
    N, H, E, k, I = cfg.N, cfg.H, cfg.E, cfg.k, cfg.I
    rows = N * k
    touched = int((np.asarray(n_e) > 0).sum())

    def ffn(rows, touched, E, d_out_rows):
        return {
            "gate_up_preact": {"bytes": touched * 2 * I * H * 2 + N * H * 2 + rows * 2 * I * 2,
                               "flops": 4.0 * rows * H * I},
            "down_dgrad": {"bytes": touched * H * I * 2 + d_out_rows * H * 2 + rows * I * 2,
                           "flops": 2.0 * rows * H * I},
            "swiglu_bwd": {"bytes": 2 * (rows * 2 * I * 2 + rows * I * 2)},
            "down_wgrad": {"bytes": d_out_rows * H * 2 + rows * I * 2 + E * H * I * 2, "flops": 2.0 * rows * H * I},
            "gate_up_wgrad": {"bytes": rows * 2 * I * 2 + d_out_rows * H * 2 + E * 2 * I * H * 2,
                              "flops": 4.0 * rows * H * I},
            "gate_up_dgrad": {"bytes": touched * 2 * I * H * 2 + rows * 2 * I * 2 + rows * H * 2,
                              "flops": 4.0 * rows * H * I},
        }
    d = {"combine_bwd": {"bytes": N * H * 2 + 2 * rows * H * 2 + rows * 8},
         "x_permute": {"bytes": N * H * 2 + rows * H * 2}}
    d.update(ffn(rows, touched, E, rows))
    if cfg.shared:
        d.update({"shared_" + n: v for n, v in ffn(N, 1, 1, N).items()})
    d["router_bwd"] = {"bytes": rows * H * 2 + E * H * 2 + rows * 12}
    d["router_dx"] = {"bytes": E * H * 2 + N * H * 2 * (2 if cfg.shared else 1) + rows * 8}
    d["dx"] = {"bytes": rows * H * 2 + N * H * 2 * 2 + rows * 4}
    return d


class _StagedWeights:
    """Weight source of the oracle: expert e's weights, held on the host in their storage
    dtype, converted to float64 when the oracle asks for them.  The conversion is input
    staging, not the oracle's arithmetic: its time is recorded and left out of the timing."""

    def __init__(self, host):
        self.host = host
        self.spent = 0.0

    def __call__(self, e):
        import torch
        t0 = time.perf_counter()
        a = self.host[e].to(torch.float64).numpy()
        self.spent += time.perf_counter() - t0
        return a


def cpu_baseline(cfg, inp, T):
    """The oracle, as it stands, on the first T tokens of the batch (T < 0: all of it): router
    logits, route, layout, permute, every expert's SwiGLU FFN on its rows (float64), the
    shared expert and combine.  Weights are copied to the host before timing and converted
    expert by expert as the oracle asks for them; that conversion is excluded."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle

    T = cfg.N if T < 0 else min(T, cfg.N)
    if cfg.dtype == "fp8":
        return None   # (its weights would first be quantized by the oracle's codec, minutes of staging)
    x = inp["x"][:T].detach().cpu().double().numpy()
    w_r = inp["w_r"].detach().cpu().double().numpy()
    b = inp["bias_cpu"]
    w13 = _StagedWeights(inp["w13"].detach().cpu())
    w2 = _StagedWeights(inp["w2"].detach().cpu())
    kw = {}
    if cfg.shared:
        kw = dict(shared_w13=inp["sw13"][0].cpu().double().numpy(), shared_w2=inp["sw2"][0].cpu().double().numpy())
    t0 = time.perf_counter()
    z = moe_oracle.router_logits(x, w_r)
    res = moe_oracle.moe_layer(x, z, cfg.k, w13, w2, bias=None if b is None else b.numpy(),
                               n_group=cfg.n_group, topk_group=cfg.topk_group, **kw)
    wall = time.perf_counter() - t0
    dt = wall - w13.spent - w2.spent
    touched = int((res["n_e"] > 0).sum())
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{'the whole batch' if T == cfg.N else f'the first {T} tokens'} of {cfg.name} "
                      f"({T} tokens, {touched} experts touched, max n_e {int(res['n_e'].max())}) through the "
                      f"whole oracle layer in float64, router logits included; {dt:.1f} s timed "
                      f"({w13.spent + w2.spent:.1f} s of bf16 -> float64 weight conversion left out)"}


def summarize(per, alg, dtype):
    kernels = {}
    for name, times in per.items():
        t = sorted(times)
        avg = sum(t) / len(t)
        k = {"avg_ms": round(avg, 4), "median_ms": round(t[len(t) // 2], 4),
             "p99_ms": round(t[min(len(t) - 1, int(math.ceil(0.99 * len(t))) - 1)], 4)}
        a = alg.get(name, {})
        if "bytes" in a:
            k["GB_per_s"] = round(a["bytes"] / (avg * 1e-3) / 1e9, 1)
            k["hbm_frac"] = round(a["bytes"] / (avg * 1e-3) / PEAK_HBM, 4)
        if "flops" in a:
            k["TFLOP_per_s"] = round(a["flops"] / (avg * 1e-3) / 1e12, 1)
            k["mfma_frac"] = round(a["flops"] / (avg * 1e-3) / PEAK_MFMA[dtype], 4)
        kernels[name] = k
    return kernels


def roofline(cfg, alg, per, fused, gather, with_traffic=True):
    """Roofline of the dominant kernel (the gate/up GEMM) from its average event time."""
    g = alg["gate_up"]
    g_avg = sum(per["gate_up"]) / len(per["gate_up"]) * 1e-3
    t_mfma = g["flops"] / PEAK_MFMA[cfg.dtype]
    t_hbm = g["bytes"] / PEAK_HBM
    traffic = None
    tf = TRAFFIC_FILE.format(cfg.name)
    if with_traffic and os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("source_sha") == source_sha(*GEMM_SOURCES):
            traffic = rec.get("bytes_per_launch")
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(g["bytes"] / g_avg / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(g["flops"] / g_avg / 1e12, 1),
                "peak": PEAK_MFMA[cfg.dtype] / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic
    roof["kernel"] = ("grouped gate/up GEMM + SwiGLU on e4m3 weights, routed rows gathered from the tokens' fp8 "
                      "values and the shared expert in the same launch (moe_expert_gate_up_gathered_shared_e4m3)"
                      if fused and cfg.dtype == "fp8" else
                      "grouped gate/up GEMM + SwiGLU, routed rows gathered from x and the shared expert in the "
                      "same launch (moe_expert_gate_up_gathered_shared)" if fused else
                      "grouped gate/up GEMM + SwiGLU, rows gathered from x (moe_expert_gate_up_gathered)"
                      if gather else "grouped gate/up GEMM + SwiGLU (moe_expert_gate_up)")
    roof["algorithmic_bytes"] = int(g["bytes"])
    roof["algorithmic_flops"] = g["flops"]
    return roof


def workload_name(cfg):
    return (f"{cfg.name}: N={cfg.N} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I}"
            + (f" groups {cfg.topk_group}/{cfg.n_group}" if cfg.n_group else "")
            + (" +shared expert" if cfg.shared else "")
            + (f" zipf bias s={cfg.zipf_s}" if cfg.zipf_s else ""))


def build_layer(cfg, args, dev):
    import workload
    from combine_grouped_gemm_amd.layer import MoELayer
    inp = workload.make_layer_inputs(cfg, dev)
    layer = MoELayer(cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, cfg.dtype, inp["w13"], inp["w2"],
                     inp.get("sw13"), inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"],
                     gather=not args.no_gather, overlap_shared=args.overlap,
                     fuse_shared=not args.no_fuse_shared, gate_in_down=args.gate_in_down, w_r=inp["w_r"])
    return inp, layer


def layer_stages(cfg, layer, x):
    """The layer's own calls, one stage each, as MoELayer.forward issues them (bf16 layers fold
    the permute into gate/up; the shared expert runs on the layer's side stream)."""
    stages = [("router", lambda: layer.router(x)),
              ("route", lambda: layer.route(layer.z)),
              ("layout", layer.dispatch)]
    if not layer.gather or layer.fp8:   # (gathered fp8: each token's quantize and dequantize)
        stages.append(("permute", lambda: layer.permute(x)))
    stages += [("gate_up", lambda: layer.gate_up(x)),
               ("down", layer.down)]
    if cfg.shared and layer.side is None and not layer.fuse:
        stages.append(("shared", lambda: layer.shared_expert(x)))
    stages.append(("combine", layer.combine))
    return stages


def time_steps(stages, layer, x, steps, warmup, stream):
    """Warm-up steps, then `steps` timed ones: (wall ms per step, per-stage event times,
    per-step event times)."""
    import torch
    side = layer.side

    def step(ev=None):
        if side is not None:
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                if ev is not None:
                    ev["shared"][0].record(side)
                layer.shared_expert(x)
                if ev is not None:
                    ev["shared"][1].record(side)
                layer.shared_done.record(side)
        for name, f in stages:
            if name == "combine" and side is not None:
                stream.wait_event(layer.shared_done)
            if ev is not None:
                ev[name][0].record(stream)
            f()
            if ev is not None:
                ev[name][1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    names = [n for n, _ in stages] + (["shared"] if side is not None else [])
    ev = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(steps):
        step(ev[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: [ev[s_][n][0].elapsed_time(ev[s_][n][1]) for s_ in range(steps)] for n in names}
    first = "shared" if side is not None else stages[0][0]
    step_ms = [ev[s_][first][0].elapsed_time(ev[s_][stages[-1][0]][1]) for s_ in range(steps)]
    return wall * 1e3 / steps, per, step_ms, step


def other_config(name, args, dev):
    """A compact measurement of another workload: ms per step, tokens/s, the dominant kernel's
    roofline fraction, per-stage times and the routing imbalance."""
    import torch
    import workload
    cfg = workload.CONFIGS[name]
    log(args, f"other workload {name}")
    inp, layer = build_layer(cfg, args, dev)
    x = inp["x"]
    stages = layer_stages(cfg, layer, x)
    steps = args.other_steps * (10 if cfg.name == "tiny_f32" else 1)
    ms, per, _, _ = time_steps(stages, layer, x, steps, 3, torch.cuda.current_stream())
    n_e = layer.layout[0].cpu().numpy()
    alg = algorithmic(cfg, n_e, layer.gather, layer.fuse)
    kernels = summarize(per, alg, cfg.dtype)
    roof = roofline(cfg, alg, per, layer.fuse, layer.gather)
    mem = {**layer.device_bytes(), "input_x": x.nbytes}
    del layer, inp, x, stages
    torch.cuda.empty_cache()
    return {"workload": workload_name(cfg), "dtype": cfg.dtype, "steps": steps, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(cfg.N / (ms / 1e3), 1), "imbalance": round(float(n_e.max() / n_e.mean()), 4),
            "max_n_e": int(n_e.max()), "empty_experts": int((n_e == 0).sum()), "device_bytes": mem,
            "roofline": {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "kernel")},
            "grouped_gemm_mfma_util": {"gate_up": kernels["gate_up"].get("mfma_frac"),
                                       "down": kernels["down"].get("mfma_frac")},
            "kernels": {n: {k: v for k, v in d.items() if k in ("avg_ms", "GB_per_s", "hbm_frac", "TFLOP_per_s",
                                                                  "mfma_frac")} for n, d in kernels.items()}}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import workload
    import combine_grouped_gemm_amd as moe

    cfg = workload.CONFIGS[args.config]
    fixed = None
    if args.rows_per_expert > 0:
        # E' experts of R rows each, with E' R a multiple of k and at most the batch's N k rows
        R = args.rows_per_expert
        e_used = min(cfg.E, cfg.N * cfg.k // R)
        while e_used > 0 and (e_used * R) % cfg.k:
            e_used -= 1
        if e_used == 0 or R > e_used * R // cfg.k:
            raise SystemExit("--rows-per-expert does not fit this workload")
        fixed = workload.counted_route([R] * e_used + [0] * (cfg.E - e_used), cfg.k, seed=1)
        cfg = cfg.scaled(name=f"{cfg.name}_fixed{R}", N=e_used * R // cfg.k, n_group=0, topk_group=0, zipf_s=0.0)
        args.cpu_tokens, args.chunks = 0, 1   # (the oracle and the chunked layer route by themselves)
    dev = torch.device("cuda:0")
    moe.lib()
    log(args, f"generating {cfg.name} inputs on the GPU")
    inp, layer = build_layer(cfg, args, dev)
    x = inp["x"]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    stages = layer_stages(cfg, layer, x)
    if fixed is not None:
        layer.topk_idx.copy_(fixed.to(dev))
        stages = [st for st in stages if st[0] not in ("router", "route")]
    side = layer.side
    if args.train:
        if side is not None:
            raise SystemExit("--train runs the layer on one stream (no --overlap)")
        dy = workload.normal((cfg.N, cfg.H), workload.stream_key(cfg.seed, workload.T_EO, 5), dev, torch.bfloat16,
                             std=1.0)
        # the training forward keeps the gate/up pre-activations for the backward
        layer.forward(x, save_for_backward=True)
        if args.overlap_backward:
            layer.backward_steps(x, dy)   # (allocates the gradients)
            stages.append(("backward", lambda: layer.backward(x, dy, overlap_shared=True)))
        else:
            stages += layer.backward_steps(x, dy)

    if args.copy_probe_mib > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch scale the
        # byte counters read for the MoE kernels
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log(args, f"warmup {args.warmup}, timing {args.steps} steps")
    ms_per_step, per, step_ms, step = time_steps(stages, layer, x, args.steps, args.warmup, stream)
    value = cfg.N / (ms_per_step / 1e3)

    graph = None
    if args.graph:
        # one step captured in a HIP graph (the library allocates, clears and synchronises
        # nothing inside a call), replayed `steps` times between synchronisations
        if side is not None:
            raise SystemExit("--graph runs the layer on one stream (no --overlap)")
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            step()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        graph = {"ms_per_step": round(graph_ms, 4), "eager_ms_per_step": round(ms_per_step, 4)}
        ms_per_step = graph_ms
        value = cfg.N / (ms_per_step / 1e3)

    cold = {}
    fill_GBps = None
    if args.cold_steps > 0:
        # cold-cache figures: before each stage a 1 GiB write evicts L2 (4 MB per XCD) and the
        # 256 MB MALL, so the stage reads its inputs (weights, activations) from HBM; the
        # stages stay in order on one stream, so every stage still sees its true inputs
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        flush.fill_(0)
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_steps)]
        cev_ = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for n, _ in stages} for _ in range(args.cold_steps)]
        torch.cuda.synchronize()
        for s_ in range(args.cold_steps):
            for i, (name, f) in enumerate(stages):
                if i == 0:
                    fev[s_][0].record(stream)
                flush.fill_(s_ + i + 1)
                if i == 0:
                    fev[s_][1].record(stream)
                cev_[s_][name][0].record(stream)
                f()
                cev_[s_][name][1].record(stream)
        torch.cuda.synchronize()
        cold = {n: [cev_[s_][n][0].elapsed_time(cev_[s_][n][1]) for s_ in range(args.cold_steps)]
                for n, _ in stages}
        fill_GBps = round((1 << 30) / (sum(a.elapsed_time(b) for a, b in fev) / len(fev) * 1e-3) / 1e9, 1)
        del flush

    if layer.gather:
        # the layer folds the permute into gate/up; the permute kernel (the standalone
        # moe_permute, same rows) is timed on its own after the layer, outside `value`
        xp = torch.empty((cfg.N * cfg.k, cfg.H), dtype=x.dtype, device=dev)
        pev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        moe.moe_permute(x, layer.layout[2], cfg.k, None, xp)
        torch.cuda.synchronize()
        pev[0].record(stream)
        for s_ in range(args.steps):
            moe.moe_permute(x, layer.layout[2], cfg.k, None, xp)
            pev[s_ + 1].record(stream)
        torch.cuda.synchronize()
        per["permute (standalone)"] = [pev[s_].elapsed_time(pev[s_ + 1]) for s_ in range(args.steps)]
        del xp

    # the machine's practical copy rate (context for the HBM fractions): torch's device copy
    # of 1 GiB, read + write bytes over its event time
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cev[0].record(stream)
    for _ in range(5):
        cdst.copy_(csrc)
    cev[1].record(stream)
    torch.cuda.synchronize()
    copy_GBps = round(2 * 5 * (1 << 30) / (cev[0].elapsed_time(cev[1]) * 1e-3) / 1e9, 1)
    del csrc, cdst

    # the ceiling of combine's access mix (about 9 rows read per row written, every access
    # sequential): the library's read-mostly streaming probe over 1 GiB read
    n16 = (1 << 30) // (9 * 16)
    psrc = torch.zeros(9 * n16 * 16, dtype=torch.uint8, device=dev)
    pdst = torch.empty(n16 * 16, dtype=torch.uint8, device=dev)
    moe.moe_stream_probe(psrc, 9, pdst)
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    pev[0].record(stream)
    for _ in range(5):
        moe.moe_stream_probe(psrc, 9, pdst)
    pev[1].record(stream)
    torch.cuda.synchronize()
    probe_GBps = round(10 * n16 * 16 * 5 / (pev[0].elapsed_time(pev[1]) * 1e-3) / 1e9, 1)
    del psrc, pdst

    # the machine's achievable dense bf16 matrix rate on this machine (context for the MFMA
    # fractions): torch's library GEMM on 8192^3, flops over its event time
    ga = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    gb = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    for _ in range(2):
        gc = ga @ gb
    gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    gev[0].record(stream)
    for _ in range(5):
        gc = ga @ gb
    gev[1].record(stream)
    torch.cuda.synchronize()
    gemm_TFLOPs = round(2.0 * 8192 ** 3 * 5 / (gev[0].elapsed_time(gev[1]) * 1e-3) / 1e12, 1)
    del ga, gb, gc

    n_e = layer.layout[0].cpu().numpy()
    alg = algorithmic(cfg, n_e, layer.gather, layer.fuse)
    # (the standalone permute copies x's rows: bf16 for the gathered fp8 layer as well)
    alg["permute (standalone)"] = {"bytes": (cfg.N + cfg.N * cfg.k) * cfg.H * x.element_size()}
    if args.train:
        alg.update(algorithmic_backward(cfg, n_e))
    kernels = summarize(per, alg, cfg.dtype)
    kernels_cold = summarize(cold, alg, cfg.dtype) if cold else None
    roof = roofline(cfg, alg, per, layer.fuse, layer.gather)

    cpu = None
    if args.cpu_tokens != 0 and not args.train:
        log(args, f"CPU oracle baseline ({'whole batch' if args.cpu_tokens < 0 else args.cpu_tokens} tokens)")
        cpu = cpu_baseline(cfg, inp, args.cpu_tokens)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8" if cfg.dtype == "fp8" else cfg.dtype, "data": "synthetic",
        "config": {"workload": workload_name(cfg), "global_batch": cfg.N, "parallelism": "single GPU"},
        "roofline": roof,
        "router_logits_in_step": fixed is None,
        "ms_per_step_without_router": round(ms_per_step - kernels.get("router", {}).get("avg_ms", 0.0), 4),
        "tokens_per_s_without_router": round(cfg.N / ((ms_per_step - kernels.get("router", {}).get("avg_ms", 0.0))
                                                      / 1e3), 1),
        "fixed_rows_per_expert": args.rows_per_expert or None,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "grouped_gemm_mfma_util": {"gate_up": kernels["gate_up"].get("mfma_frac"),
                                   "down": kernels["down"].get("mfma_frac")},
        "permute_hbm_GBps": (kernels["permute"] if "permute" in kernels
                             else kernels["permute (standalone)"])["GB_per_s"],
        "permute_folded_into_gate_up": layer.gather,
        "shared_expert_on_side_stream": side is not None,
        "shared_expert_in_routed_launches": layer.fuse,
        "gates_in_down_epilogue": layer.gate_in_down,
        "combine_hbm_GBps": kernels["combine"]["GB_per_s"],
        "imbalance": round(float(n_e.max() / n_e.mean()), 4),
        "device_bytes": {**layer.device_bytes(), "input_x": inp["x"].nbytes},
        "device_copy_GBps": copy_GBps,
        "read_mostly_probe_GBps": probe_GBps,
        "combine_vs_read_mostly_probe": round(kernels["combine"]["GB_per_s"] / probe_GBps, 4),
        "device_fill_GBps": fill_GBps,
        "library_bf16_gemm_TFLOPs": gemm_TFLOPs,
        "kernels_cold": kernels_cold,
        "cold_steps": args.cold_steps,
        "event_ms_per_step_median": round(sorted(step_ms)[len(step_ms) // 2], 4),
        "hip_graph": graph,
    }
    if args.train:
        nb = 1 if args.overlap_backward else len(layer.backward_steps(x, dy))
        fwd_names = [n for n, _ in stages[:len(stages) - nb]]
        bwd_names = [n for n, _ in stages if n not in fwd_names]
        cands = [n for n in bwd_names if n in alg]
        broof = None
        if cands:   # (per-step figures exist when the backward's steps are timed one by one)
            slow = max(cands, key=lambda n: kernels[n]["avg_ms"])
            a = alg[slow]
            t = kernels[slow]["avg_ms"] * 1e-3
            if "flops" in a and a["flops"] / PEAK_MFMA[cfg.dtype] > a["bytes"] / PEAK_HBM:
                broof = {"bound": "mfma", "achieved": round(a["flops"] / t / 1e12, 1),
                         "peak": PEAK_MFMA[cfg.dtype] / 1e12, "unit": "TFLOP/s"}
            else:
                broof = {"bound": "hbm", "achieved": round(a["bytes"] / t / 1e9, 1), "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s"}
            broof["frac"] = round(broof["achieved"] / broof["peak"], 4)
            broof["traffic"] = None
            broof["kernel"] = f"backward step '{slow}' (the slowest of the backward pass)"
        out.update({
            "metric": "MoE-layer training step tokens/s (router logits, forward and backward; bf16 weight "
                      "gradients)",
            "forward_ms": round(sum(kernels[n]["avg_ms"] for n in fwd_names), 4),
            "backward_ms": round(sum(kernels[n]["avg_ms"] for n in bwd_names), 4),
            "backward_roofline": broof,
            "cpu_baseline": None,
        })

    # A/B: the same batch cut into chunks, one chunk's combine beside the next chunk's GEMMs
    # (bf16 layers; the batch must split into equal chunks)
    if args.chunks > 1 and not args.train and cfg.dtype == "bf16" and cfg.N % args.chunks == 0:
        from combine_grouped_gemm_amd.layer import PipelinedMoE
        log(args, f"chunked pipeline, {args.chunks} chunks")
        pipe = PipelinedMoE(args.chunks, cfg.N, cfg.H, cfg.E, cfg.k, cfg.I, inp["w13"], inp["w2"], inp.get("sw13"),
                            inp.get("sw2"), cfg.n_group, cfg.topk_group, inp["bias"], w_r=inp["w_r"])
        for _ in range(args.warmup):
            pipe.forward(x)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            pipe.forward(x)
        torch.cuda.synchronize()
        chunk_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        out["chunked_pipeline"] = {"chunks": args.chunks, "ms_per_step": round(chunk_ms, 4),
                                   "tokens_per_s": round(cfg.N / (chunk_ms / 1e3), 1),
                                   "vs_unchunked": round(ms_per_step / chunk_ms, 4)}
        del pipe
        torch.cuda.empty_cache()

    # the other workloads, each on its own after this one's buffers are released
    others = None
    if args.other_configs != "none" and not args.train:
        # (the five workloads, then the DeepSeek-V3-shaped layer in fp8 at the prefill batch)
        names = ([n for n in workload.CONFIG_ORDER + ["dsv3_fp8"] if n != cfg.name] if args.other_configs == "all"
                 else [n for n in args.other_configs.split(",") if n])
        del layer, inp, x, stages, step
        torch.cuda.empty_cache()
        others = {n: other_config(n, args, dev) for n in names}
    out["other_configs"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
