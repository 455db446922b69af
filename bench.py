#!/usr/bin/env python
"""Throughput of the fused MoE layer on one MI355X.

Workload (default): one GPU's share of the hidden-7168 / expert-intermediate-
2048 layer -- T=16384 tokens, 32 experts, top-8 routing with a N(0,1) per-expert
logit bias, weights N(0, 0.02), bf16, minibatches of 2560 tokens.  A step is
one full layer forward (route, layout, dispatch gather, gate|up grouped GEMM
with SwiGLU, down grouped GEMM, combine) over the T tokens, with the inputs
already resident in HBM.

Prints one JSON line: tokens/s over the timed steps, the roofline position of
the dominant kernel (the gate|up grouped GEMM, timed with HIP events on the
stream it runs on), and the CPU oracle timed on a bounded token sample.
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
    ap.add_argument("--minibatch", type=int, default=None)
    ap.add_argument("--cpu-sample", type=int, default=2048, help="tokens the CPU oracle is timed on")
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
    inp = make_inputs(w, with_dout=False)
    log("inputs drawn in %.1f s" % (time.time() - t_gen))

    flags = moe.MOE_F_SHARED_EXPERT if w.shared_expert else 0
    cfg = moe.make_cfg(w.T, w.H, w.I, w.E, w.k, minibatch=w.minibatch, flags=flags)
    sizes = moe.moe_query_sizes(cfg)
    bufs = moe.alloc_buffers(cfg)
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x, Wr, bias = dev(inp.x), dev(inp.Wr), dev(inp.bias)
    Wg, Wu, Wd = dev(inp.Wg), dev(inp.Wu), dev(inp.Wd)
    moe.moe_prepare_weights(cfg, Wg, Wu, Wd, bufs.packed, dev(inp.Wsg), dev(inp.Wsu), dev(inp.Wsd))
    torch.cuda.synchronize()
    del Wg, Wu, Wd
    out = torch.empty_like(x)

    def step():
        moe.moe_layer_fwd(cfg, Wr, bias, bufs.packed, x, out, bufs.ws)

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
    flops_gate_up = 4.0 * H * I * rows  # per step, padding rows excluded
    flops_down = 2.0 * H * I * rows
    n_g1, ms_g1 = kt["gemm_gate_up"]
    n_g2, ms_g2 = kt["gemm_down"]
    n_c, ms_c = kt["combine"]
    achieved_g1 = flops_gate_up * args.steps / (ms_g1 / 1e3) / 1e12
    achieved_g2 = flops_down * args.steps / (ms_g2 / 1e3) / 1e12
    combine_bytes = (T * k * H * 2 + T * H * 2 + T * k * 8) * args.steps
    ms_step = elapsed * 1e3 / args.steps
    value = T * args.steps / elapsed

    res = {
        "metric": "MoE layer fwd tokens/s at H=7168 I=2048 (bf16) + % MFMA peak",
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
                   "router_bias": w.router_bias, "pass": "forward"},
        "roofline": {"bound": "mfma", "kernel": "grouped_gemm_kernel<SwiGLU> (gate|up)",
                     "achieved": achieved_g1, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved_g1 / PEAK_BF16_TFLOPS, "traffic": None,
                     "avg_launch_ms": ms_g1 / max(n_g1, 1), "launches": n_g1},
        "detail": {
            "layer_mfma_frac": (flops_gate_up + flops_down) / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "gemm_down_tflops": achieved_g2,
            "gemm_down_avg_launch_ms": ms_g2 / max(n_g2, 1),
            "combine_gbs": combine_bytes / (ms_c / 1e3) / 1e9 if ms_c > 0 else None,
            "per_step_ms": {kind: v[1] / args.steps for kind, v in kt.items() if kind != "dropped"},
            "timing_dropped": kt["dropped"],
        },
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample)
    print(json.dumps(res), flush=True)


def cpu_baseline(inp, n_tokens: int) -> dict:
    """The CPU oracle (as it stands) on the first n_tokens tokens of the workload."""
    import numpy as np
    import threadpoolctl
    import oracle

    n = min(n_tokens, inp.w.T)
    oracle.router_logits(np.zeros((1, inp.w.H), np.float32), np.zeros((inp.w.H, 1), np.float32))
    t0 = time.perf_counter()
    oracle.layer_forward(inp, tokens=np.arange(n))
    dt = time.perf_counter() - t0
    blas = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    omp = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": n / dt, "unit": "tokens/s", "cores": max(blas, omp), "kind": "oracle",
            "sample": "first %d of %d tokens: fixed-order fp32 routing (C, OpenMP) + fp64 expert "
                      "SwiGLU FFN (numpy/OpenBLAS) + combine; %.1f s" % (n, inp.w.T, dt)}


if __name__ == "__main__":
    main()
