#!/usr/bin/env python
"""Throughput of the fused MoE layer on one MI355X.

Workload (default): one GPU's share of the hidden-7168 / expert-intermediate-
2048 layer -- T=16384 tokens, 32 experts, top-8 routing with a N(0,1) per-expert
logit bias, weights N(0, 0.02), bf16, minibatches of 2560 tokens.  A step is
one full layer forward (route, layout, dispatch gather, gate|up grouped GEMM
with SwiGLU, down grouped GEMM, combine) over the T tokens, with the inputs
already resident in HBM.  With --pass fwdbwd (the default) a step is the
forward followed by the full backward (reverse-combine, down and gate|up
input-gradient GEMMs, reverse-dispatch with the router term, weight-gradient
GEMMs, router weight gradient) with a N(0,1) upstream gradient.

Prints one JSON line: tokens/s over the timed steps, the roofline position of
the dominant kernel kind (by summed time, timed with HIP events on the stream
it runs on), and the CPU oracle timed on a bounded token sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="h7168_i2048_e32_k8_bf16")
    ap.add_argument("--pass", dest="passes", choices=("fwd", "fwdbwd"), default="fwdbwd")
    ap.add_argument("--minibatch", type=int, default=None)
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer build has no multi-GPU path "
              "(expert parallelism across GPUs is out of scope); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import dispatch_grouped_gemm_moe_amd as moe
    from moe_inputs import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.minibatch is not None:
        w = w.replace(minibatch=args.minibatch)
    log("workload", w)
    t_gen = time.time()
    from moe_inputs import make_inputs
    bwd = args.passes == "fwdbwd"
    inp = make_inputs(w, with_dout=bwd)
    log("inputs drawn in %.1f s" % (time.time() - t_gen))

    flags = moe.MOE_F_SHARED_EXPERT if w.shared_expert else 0
    cfg = moe.make_cfg(w.T, w.H, w.I, w.E, w.k, minibatch=w.minibatch, flags=flags)
    sizes = moe.moe_query_sizes(cfg)
    bufs = moe.alloc_buffers(cfg, with_saved=bwd)
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x, Wr, bias = dev(inp.x), dev(inp.Wr), dev(inp.bias)
    Wg, Wu, Wd = dev(inp.Wg), dev(inp.Wu), dev(inp.Wd)
    moe.moe_prepare_weights(cfg, Wg, Wu, Wd, bufs.packed, dev(inp.Wsg), dev(inp.Wsu), dev(inp.Wsd))
    torch.cuda.synchronize()
    del Wg, Wu, Wd
    out = torch.empty_like(x)
    if bwd:
        T, H, I, E = w.T, w.H, w.I, w.E
        dout = dev(inp.dout)
        dx = torch.empty_like(x)
        dWg = torch.empty(E, H, I, dtype=torch.float32, device="cuda")
        dWu = torch.empty_like(dWg)
        dWd = torch.empty(E, I, H, dtype=torch.float32, device="cuda")
        dWr = torch.empty(H, E, dtype=torch.float32, device="cuda")
        dWs = torch.empty(3 * H * I, dtype=torch.float32, device="cuda") if w.shared_expert else None

    def step():
        moe.moe_layer_fwd(cfg, Wr, bias, bufs.packed, x, out, bufs.ws, saved=bufs.saved)
        if bwd:
            moe.moe_layer_bwd(cfg, Wr, bias, bufs.packed, x, dout, bufs.saved, dx, dWg, dWu, dWd, dWr,
                              bufs.ws, dWs=dWs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    moe.moe_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kt = moe.moe_timing_read()
    moe.moe_timing_enable(False)

    T, H, I, E, k = w.T, w.H, w.I, w.E, w.k
    rows = T * k + (T if w.shared_expert else 0)  # routed (+ shared) rows per step
    hi = float(H) * I * rows  # padding rows excluded from every figure below
    # algorithmic flops per step of each grouped-GEMM kind (forward, plus the
    # backward's input-gradient GEMMs of the same shape and the weight gradients)
    flops = {"gemm_gate_up": 4 * hi * (2 if bwd else 1), "gemm_down": 2 * hi * (2 if bwd else 1),
             "wgrad": 6 * hi if bwd else 0.0}
    ms_step = elapsed * 1e3 / args.steps
    value = T * args.steps / elapsed
    dom = max((kind for kind in flops if flops[kind] > 0), key=lambda kd: kt[kd][1])
    n_dom, ms_dom = kt[dom]
    achieved = flops[dom] * args.steps / (ms_dom / 1e3) / 1e12
    kernel_names = {"gemm_gate_up": "grouped_gemm_kernel<0> gate|up SwiGLU (+ grouped_gemm_kernel<1> gate|up input gradient)",
                    "gemm_down": "grouped_gemm_kernel<1> down (+ grouped_gemm_kernel<2> down input gradient, SwiGLU backward)",
                    "wgrad": "wgrad_kernel (weight gradients)"}
    total_flops = sum(flops.values())
    res = {
        "metric": "MoE layer %s tokens/s at H=7168 I=2048 (bf16) + %% MFMA peak" % ("fwd+bwd" if bwd else "fwd"),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "hidden": H, "intermediate": I, "experts": E,
                   "top_k": k, "minibatch": sizes.minibatch, "minibatches": sizes.num_minibatches,
                   "router_bias": w.router_bias, "shared_expert": w.shared_expert,
                   "pass": "forward+backward" if bwd else "forward"},
        "roofline": {"bound": "mfma", "kernel": kernel_names[dom], "kind": dom,
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "avg_launch_ms": ms_dom / max(n_dom, 1), "launches": n_dom},
        "detail": {
            "layer_mfma_frac": total_flops / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "tflops_by_kind": {kd: flops[kd] * args.steps / (kt[kd][1] / 1e3) / 1e12
                               for kd in flops if flops[kd] > 0 and kt[kd][1] > 0},
            "per_step_ms": {kind: v[1] / args.steps for kind, v in kt.items() if kind != "dropped"},
            "timing_dropped": kt["dropped"],
        },
    }

    if not args.no_cpu_baseline:
        n = args.cpu_sample or (256 if bwd else 2048)
        res["cpu_baseline"] = cpu_baseline(inp, n, bwd)
    print(json.dumps(res), flush=True)


def cpu_baseline(inp, n_tokens: int, bwd: bool) -> dict:
    """The CPU oracle (as it stands) on the first n_tokens tokens of the workload,
    taken as a layer of n_tokens tokens with the same weights."""
    import numpy as np
    import threadpoolctl
    import oracle
    from moe_inputs import LayerInputs

    n = min(n_tokens, inp.w.T)
    sub = LayerInputs(inp.w.replace(T=n), inp.x[:n], inp.Wr, inp.bias, inp.Wg, inp.Wu, inp.Wd,
                      inp.Wsg, inp.Wsu, inp.Wsd, inp.dout[:n] if inp.dout is not None else None)
    oracle.router_logits(np.zeros((1, inp.w.H), np.float32), np.zeros((inp.w.H, 1), np.float32))
    t0 = time.perf_counter()
    fwd = oracle.layer_forward(sub, keep=bwd, mx=False)
    if bwd:
        oracle.layer_backward(sub, fwd=fwd)
    dt = time.perf_counter() - t0
    blas = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    omp = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": n / dt, "unit": "tokens/s", "cores": max(blas, omp), "kind": "oracle",
            "sample": "first %d of %d tokens as a %d-token layer: fixed-order fp32 routing (C, OpenMP) + "
                      "fp64 expert SwiGLU FFN and combine%s (numpy/OpenBLAS); %.1f s"
                      % (n, inp.w.T, n, " + fp64 backward" if bwd else "", dt)}


if __name__ == "__main__":
    main()
