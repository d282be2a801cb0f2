#!/usr/bin/env python3
"""Benchmark of the dropless MoE expert-FFN layer (forward + backward) on one MI355X.

One step = one whole pass of the layer over one batch of synthetic inputs:
route top-k, permute, FC1 + GLU epilogue, FC2, combine, and the backward
(combine bwd, route bwd, FC2 dgrad + dGLU, FC2 wgrad, FC1 dgrad, FC1 wgrad,
unpermute-sum).  Inputs are resident in HBM before the timed region.

Default workload: the DeepSeek-V3-like one-GPU expert shard (T=16384 tokens,
d=7168, f=2048, 32 local experts, top-8 sigmoid gates, SwiGLU, Zipf(1.5)
routing skew with two empty experts), bf16 storage, fp32 accumulation.

Prints ONE JSON line: value = algorithmic GEMM TFLOP/s of the whole layer
(18 R d f FLOP per step / step time), plus the roofline of the dominant
kernel (HIP events on the launch stream) and the CPU oracle's rate on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2516.6       # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2        # MI355X dense fp8 MFMA (MXFP8 operands)
PEAK_FP4_TFLOPS = 10066.4       # MI355X dense fp4 MFMA (MXFP4 operands)
PEAK_F32_TFLOPS = 157.3         # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0
METRIC = "MoE FFN fwd+bwd TFLOPS and % of MFMA peak, 1×MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv3_fwdbwd")
    ap.add_argument("--cpu-tokens", type=int, default=1024,
                    help="tokens of the workload the CPU oracle runs (bounded sample)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--permute", choices=["fused", "copy"], default="fused",
                    help="bf16 / fp32 workloads: FC1 and FC1 wgrad read x through src_row "
                         "(fused) or a materialized permuted copy (copy)")
    ap.add_argument("--mx-dxp", action="store_true",
                    help="MX workloads: FC1's dgrad writes dXp as an MX row copy and dX is "
                         "summed from it (quantized plain-GEMM output)")
    ap.add_argument("--recompute", action="store_true",
                    help="bf16 / fp32 training workloads: H is not kept from the forward, the "
                         "backward runs FC1 + GLU again (its FLOP are not counted in the metric)")
    ap.add_argument("--no-transpose-w2", action="store_true",
                    help="bf16 / fp32 training workloads: FC2's dgrad reads W2 as stored "
                         "(MN-contiguous) instead of a transposed copy made in each backward "
                         "(default: the layer's choice by routed rows per expert)")
    ap.add_argument("--no-transpose-w1", action="store_true",
                    help="bf16 / fp32 training workloads: FC1's dgrad reads W1p as stored "
                         "(MN-contiguous) instead of a transposed copy made in each backward "
                         "(default: the layer's choice by routed rows per expert)")
    ap.add_argument("--router", action="store_true",
                    help="the layer computes its own logits: the router's map x w_router^T fused "
                         "with the top-k routing (w_router synthetic N(0, 1/d), so the routing is "
                         "not Zipf-skewed), and the router's backward (dWr, its share of dX)")
    ap.add_argument("--gate-in-act", action="store_true",
                    help="the routing gates scale FC1's activation output (feature scaling) "
                         "and the combine sums with unit weights; the gate gradient comes "
                         "from the dGLU epilogue, and the combine's backward does not read Y")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters of a profiler run) and exit")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_flops(cfg):
    R, d, f, n1 = cfg.R, cfg.d, cfg.f, cfg.n1
    fl = {"fc1_glu_fwd": 2 * R * d * n1, "fc2_fwd": 2 * R * d * f}
    if cfg.backward:
        fl.update({"fc2_dgrad_dglu": 2 * R * d * f, "fc2_wgrad": 2 * R * d * f,
                   "fc1_dgrad": 2 * R * d * n1, "fc1_wgrad": 2 * R * d * n1})
    return fl


def hbm_bytes(cfg, fused_permute=False, gate_in_act=False):
    """Algorithmic bytes of the memory-bound kernels (each tensor read or written once)."""
    b = 4 if cfg.dtype == "f32" else 2
    T, R, d, k, E = cfg.T, cfg.R, cfg.d, cfg.k, cfg.E
    out = {"route_topk": T * E * 4 + T * k * 8,
           "router_topk": T * cfg.d * (4 if cfg.dtype == "f32" else 2) + T * E * 4 + T * k * 8,
           "permute": T * d * b + R * d * b + T * k * 4 + 8 * R,
           "combine": R * d * b + T * d * b + 8 * R}
    if fused_permute:
        out["permute"] = T * k * 4 + 12 * R     # routing indices only: no row is copied
    if cfg.gemm in ("mxfp8", "mxfp4"):
        # MX copies of Xp and dY, written straight from x / d_out: each routed
        # row is gathered once, both copies (codes + scales) written
        cb = 1.0 if cfg.gemm == "mxfp8" else 0.5           # code bytes per element
        mxb = lambda n: int(R * n * cb) + R * n // 32
        out["permute"] = T * k * 4 + 12 * R
        out["quantize_x"] = R * d * b + 2 * mxb(d)
    if cfg.backward:
        if cfg.gemm in ("mxfp8", "mxfp4"):
            out["quantize_dy"] = R * d * b + 2 * mxb(d) + 8 * R
        f, n1 = cfg.f, cfg.n1
        out.update({"transpose_w2": 2 * E * d * f * b, "transpose_w1p": 2 * E * d * n1 * b})
        out["router_bwd"] = 3 * T * d * b + T * E * 4 + E * d * 4
        out.update({"combine_bwd": T * d * b + 2 * R * d * b + 12 * R,
                    "route_topk_bwd": T * E * 8 + T * k * 8,
                    "unpermute_dx": R * d * b + T * d * b + 4 * R})
        if gate_in_act:
            out["combine_bwd"] = T * d * b + R * d * b + 4 * R      # no Y, no gate gradient
            out["gate_grad"] = 12 * R
    if gate_in_act:
        out["gates_to_rows"] = 12 * R
    return out


def recorded_traffic(cfg, kernel, permute):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, scaled by the copy calibration; None when there is no
    record for this workload and permute mode or the kernel source changed
    since it was taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"traffic_grouped_gemm_{cfg.name}.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
        with open(os.path.join(here, rec["kernel_source"]), "rb") as fh:
            sha = hashlib.sha256(fh.read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    if sha != rec.get("kernel_source_sha256") or kernel not in rec.get("kernels", {}):
        return None
    if rec.get("permute", "copy") != permute:
        return None
    return rec["kernels"][kernel]["traffic_bytes"]


def cpu_baseline(cfg, inp, tokens):
    """The oracle, as it stands, on the first `tokens` tokens of the workload."""
    import numpy as np
    import synth
    from oracle import moe as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    Tc = min(tokens, cfg.T)
    sub = cfg.replace(T=Tc)
    f32 = lambda a: synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a
    x = f32(inp["x"][:Tc])
    lg = inp["logits"][:Tc]
    W1, W2 = f32(inp["W1"]), f32(inp["W2"])
    b1 = inp.get("b1") if cfg.bias else None
    b2 = inp.get("b2") if cfg.bias else None
    spec = om.LayerSpec(cfg.k, cfg.score, cfg.normalize, cfg.act, cfg.clamp, cfg.alpha,
                        store=cfg.dtype, gemm=cfg.gemm)
    t0 = time.perf_counter()
    fwd = om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)
    if cfg.backward:
        om.layer_backward(fwd, f32(inp["dOut"][:Tc]), lg, W1, W2, spec=spec, has_bias=cfg.bias)
    dt = time.perf_counter() - t0
    flops = sum(gemm_flops(sub).values())
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {Tc} of {cfg.T} tokens of {cfg.name} (R={Tc * cfg.k} routed rows), "
                      f"full expert weights, forward{'+backward' if cfg.backward else ''}, fp64"
                      + (f", {cfg.gemm.upper()} QDQ of every GEMM operand"
                         if cfg.gemm in ("mxfp8", "mxfp4") else "")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this layer is built for a single MI355X and "
              f"--gpus {args.gpus} is not supported (see the sharding notes in DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibration_copy:
        n = args.calibration_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "launches": 3}), flush=True)
        return
    import synth
    from ragged_grouped_gemm_amd import ops
    from ragged_grouped_gemm_amd.layer import MoEFFN, OpTimer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    log(f"library: {ops.moe_version()}")
    cfg = synth.WORKLOADS[args.workload]
    t0 = time.time()
    inp = synth.make_inputs(cfg)
    log(f"generated inputs for {cfg.name} in {time.time() - t0:.1f}s")
    t = lambda a: synth.to_torch(a, "cuda")
    x, lg, W1, W2 = t(inp["x"]), t(inp["logits"]), t(inp["W1"]), t(inp["W2"])
    b1 = t(inp["b1"]) if cfg.bias else None
    b2 = t(inp["b2"]) if cfg.bias else None
    dout = t(inp["dOut"]) if cfg.backward else None
    if cfg.gated:
        W1p, b1p = ops.moe_repack_glu_weights(W1, b1)
        del W1
    else:
        W1p, b1p = W1, b1
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    mx = cfg.gemm in ("mxfp8", "mxfp4")
    L = MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, dtype=dt, act=cfg.act, score=cfg.score,
               normalize=cfg.normalize, clamp=cfg.clamp, alpha=cfg.alpha, bias=cfg.bias,
               backward=cfg.backward, gemm=cfg.gemm, fuse_permute=args.permute == "fused",
               recompute=args.recompute, mx_dxp=args.mx_dxp,
               transpose_w2=False if args.no_transpose_w2 else None,
               transpose_w1=False if args.no_transpose_w1 else None,
               router=args.router, gate_in_act=args.gate_in_act)
    if args.router:
        lg = t(synth.draw_router_weights(cfg))       # the layer's logits come from x lg^T
    permute = "fused" if L.fuse_permute else "copy"
    if mx:
        # the MXFP8 weight copies are made once, outside the timed steps (the
        # weights do not change between the synthetic steps)
        W1p = MoEFFN.mx_weights(W1p, W2, cfg.gemm)
        W2 = None
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        L.step(x, lg, W1p, W2, dout, b1p, b2)
    torch.cuda.synchronize()
    log(f"counts {torch.bincount(L.topk_idx.flatten().long(), minlength=cfg.E).tolist()}")

    # ---- timed region: K eager steps, HIP events around every library call ----
    timer = OpTimer()
    L.timer = timer
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        L.step(x, lg, W1p, W2, dout, b1p, b2)
    end.record()
    torch.cuda.synchronize()
    L.timer = None
    ms_step = start.elapsed_time(end) / args.steps
    per_op = timer.summary()
    log(f"eager step {ms_step:.3f} ms")

    flops = gemm_flops(cfg)
    total_flops = sum(flops.values())
    kernels = {}
    for name, (n, ms) in per_op.items():
        row = {"launches_per_step": n // args.steps, "ms": round(ms, 4)}
        if name in flops:
            row["tflops"] = round(flops[name] / ms / 1e9, 1)
        hb = hbm_bytes(cfg, L.fuse_permute, args.gate_in_act).get(name)
        if hb:
            row["gbs"] = round(hb / ms / 1e6, 1)
        kernels[name] = row
    gemm_ms = sum(per_op[n][1] for n in flops)
    dom = max(flops, key=lambda n: per_op[n][1])
    peak = (PEAK_F32_TFLOPS if cfg.dtype == "f32" else
            PEAK_FP4_TFLOPS if cfg.gemm == "mxfp4" else
            PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS)
    achieved = flops[dom] / per_op[dom][1] / 1e9
    value = total_flops / ms_step / 1e9

    graph_ms = None
    if not args.no_graph:
        g = L.capture(x, lg, W1p, W2, dout, b1p, b2)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / args.steps
        log(f"graph replay step {graph_ms:.3f} ms")
        del g

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else (cfg.gemm if mx else "bf16"),
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "f": cfg.f, "E": cfg.E,
                   "k": cfg.k, "routed_rows": cfg.R, "score": cfg.score, "act": cfg.act,
                   "permute": "mx_quantize_gather" if mx else permute,
                   "recompute_fc1": bool(args.recompute),
                   "fused_router": bool(args.router),
                   "gate_in_act": bool(args.gate_in_act),
                   "mx_dxp": bool(args.mx_dxp),
                   "dgrad_weights_transposed": [n for n, on in
                                                (("W2", getattr(L, "W2t", None) is not None),
                                                 ("W1p", getattr(L, "W1pt", None) is not None))
                                                if on],
                   "gemm_tflop_per_step": round(total_flops / 1e12, 4)},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "gemm_only_tflops": round(total_flops / gemm_ms / 1e9, 2),
        "graph_ms_per_step": round(graph_ms, 4) if graph_ms else None,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": recorded_traffic(cfg, dom, permute),
                     "flop_per_launch": flops[dom], "ms_per_launch": round(per_op[dom][1], 4)},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        log("running the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
