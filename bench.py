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
PEAK_FP8_TFLOPS = 5033.2   # dense MXFP8 / FP8
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
    ap.add_argument("--comm-cus", type=int, default=0, help="combine workgroups of the layer kernel (0 = automatic)")
    ap.add_argument("--ring-slots", type=int, default=0, help="ring slots (0 = automatic)")
    ap.add_argument("--launch-per-gemm", action="store_true",
                    help="forward as one launch per grouped GEMM instead of the persistent layer kernel")
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the main workload (by default the MXFP8 forward, the MXFP8 + shared "
                         "forward + backward with MXFP8 and with bf16 weight gradients, the bf16 forward and "
                         "the per-GEMM bf16 forward are timed as well, into detail.workloads)")
    ap.add_argument("--bf16-wgrad", action="store_true",
                    help="MXFP8 workloads: bf16 weight-gradient operands (MOE_F_BF16_WGRAD)")
    ap.add_argument("--extra-steps", type=int, default=5)
    ap.add_argument("--no-mfma-loop", action="store_true",
                    help="skip the sustained-MFMA measurement (a pure MFMA loop on the layer's own input values)")
    ap.add_argument("--cold-cache", action="store_true",
                    help="write a 512 MiB scratch buffer before every timed step (more than the 256 MB "
                         "Infinity Cache) and time each step alone with HIP events on the stream")
    ap.add_argument("--copy-bandwidth-mib", type=int, default=0,
                    help="first time a plain copy of this many MiB and log its HBM bandwidth")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain elementwise copy (negation) of this many MiB, "
                         "the yardstick for HBM byte counters")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("KERNEL_STATS_CSV", "TITLE", "COMMAND"),
                    help="print a rocprofv3 --stats kernel summary as markdown and exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="fold two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this workload, "
                         "taken with --calibrate-copy-mib, into profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], args.workload,
                          args.calibrate_copy_mib)
        return
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
    if args.copy_bandwidth_mib:
        # a plain elementwise copy, timed (4 repetitions after one warm-up): the
        # HBM bandwidth a streaming kernel reaches on this machine (read + write)
        a = torch.ones(args.copy_bandwidth_mib << 19, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(4):
            torch.neg(a, out=b)
        e1.record()
        torch.cuda.synchronize()
        log("copy of %d MiB: %.2f TB/s (read + write)" % (
            args.copy_bandwidth_mib, 4 * 2 * a.numel() * 2 / (e0.elapsed_time(e1) / 1e3) / 1e12))
        del a, b
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 19  # bf16 elements
        a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    bwd = args.passes == "fwdbwd"
    m = measure(moe, torch, w, bwd, args.steps, args.warmup, comm_cus=args.comm_cus, ring_slots=args.ring_slots,
                launch_per_gemm=args.launch_per_gemm, cold_cache=args.cold_cache,
                mfma_loops=not args.no_mfma_loop, keep_inputs=not args.no_cpu_baseline,
                bf16_wgrad=args.bf16_wgrad)
    inp = m.pop("inputs", None)
    mx = w.prec == "mxfp8"
    res = {
        "metric": "MoE layer %s tokens/s at H=%d I=%d (%s) + %% MFMA peak" % (
            "fwd+bwd" if bwd else "fwd", w.H, w.I, "MXFP8" if mx else "bf16"),
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3" if mx else "bf16",
        "data": "synthetic",
        "config": m["config"],
        "roofline": m["roofline"],
        "detail": m["detail"],
    }
    if not args.no_extra:
        # the other measured workloads of the layer, each timed the same way
        # (inputs resident in HBM, warm-up steps, then timed steps) after the
        # main one's buffers are released
        extras = {}
        for name, e_bwd, flags in (("h7168_i2048_e32_k8_mxfp8_zipf", False, {}),
                                   ("h7168_i2048_e32_k8_mxfp8_shared_fwdbwd", True, {}),
                                   ("h7168_i2048_e32_k8_mxfp8_shared_fwdbwd", True, {"bf16_wgrad": True}),
                                   ("h7168_i2048_e32_k8_bf16", False, {}),
                                   ("h7168_i2048_e32_k8_bf16", False, {"launch_per_gemm": True})):
            key = "%s/%s%s" % (name, "fwdbwd" if e_bwd else "fwd",
                               "".join("/" + {"launch_per_gemm": "per_gemm", "bf16_wgrad": "bf16_wgrad"}[f]
                                       for f in flags))
            log("timing", key)
            r = measure(moe, torch, WORKLOADS[name], e_bwd, args.extra_steps, 2, mfma_loops=False, **flags)
            extras[key] = {"value": r["value"], "unit": "tokens/s", "ms_per_step": r["ms_per_step"],
                           "steps": args.extra_steps, "config": r["config"], "roofline": r["roofline"],
                           "tflops_by_role": r["detail"]["tflops_by_role"],
                           "hbm_gbs_by_role": r["detail"]["hbm_gbs_by_role"],
                           "per_step_ms": r["detail"]["per_step_ms"]}
        res["detail"]["workloads"] = extras
    if not args.no_cpu_baseline:
        n = args.cpu_sample or 2048
        res["cpu_baseline"] = cpu_baseline(inp, n, bwd)
    print(json.dumps(res), flush=True)


def measure(moe, torch, w, bwd: bool, steps: int, warmup: int, comm_cus: int = 0, ring_slots: int = 0,
            launch_per_gemm: bool = False, cold_cache: bool = False, mfma_loops: bool = False,
            keep_inputs: bool = False, bf16_wgrad: bool = False) -> dict:
    """Times `steps` layer steps of workload `w` (forward, or forward + backward)
    after `warmup` untimed ones, with every input already in HBM; returns the
    throughput, the dominant kernel's roofline position and the per-kernel-kind
    breakdown (HIP events recorded by the library on the stream each kernel
    runs on).  Releases every device buffer and the timing events before it
    returns."""
    from moe_inputs import make_inputs
    t_gen = time.time()
    mx = w.prec == "mxfp8"
    inp = make_inputs(w, with_dout=bwd)
    log("%s: inputs drawn in %.1f s" % (w.name, time.time() - t_gen))
    mx_wgrad = mx and not bf16_wgrad
    flags = (moe.MOE_F_SHARED_EXPERT if w.shared_expert else 0) | (moe.MOE_F_LAUNCH_PER_GEMM if launch_per_gemm else 0)
    if mx and bf16_wgrad:
        flags |= moe.MOE_F_BF16_WGRAD
    cfg = moe.make_cfg(w.T, w.H, w.I, w.E, w.k, minibatch=w.minibatch, flags=flags,
                       prec=moe.MOE_PREC_MXFP8 if mx else moe.MOE_PREC_BF16,
                       comm_cus=comm_cus, ring_slots=ring_slots)
    sizes = moe.moe_query_sizes(cfg)
    bufs = moe.alloc_buffers(cfg, with_saved=bwd)
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x, Wr, bias = dev(inp.x), dev(inp.Wr), dev(inp.bias)
    Wg, Wu, Wd = dev(inp.Wg), dev(inp.Wu), dev(inp.Wd)
    moe.moe_prepare_weights(cfg, Wg, Wu, Wd, bufs.packed, dev(inp.Wsg), dev(inp.Wsu), dev(inp.Wsd))
    torch.cuda.synchronize()
    del Wg, Wu, Wd
    out = torch.empty_like(x)
    T, H, I, E, k = w.T, w.H, w.I, w.E, w.k
    grads = {}
    if bwd:
        grads = dict(dout=dev(inp.dout), dx=torch.empty_like(x),
                     dWg=torch.empty(E, H, I, dtype=torch.float32, device="cuda"),
                     dWu=torch.empty(E, H, I, dtype=torch.float32, device="cuda"),
                     dWd=torch.empty(E, I, H, dtype=torch.float32, device="cuda"),
                     dWr=torch.empty(H, E, dtype=torch.float32, device="cuda"),
                     dWs=torch.empty(3 * H * I, dtype=torch.float32, device="cuda") if w.shared_expert else None)

    def step():
        moe.moe_layer_fwd(cfg, Wr, bias, bufs.packed, x, out, bufs.ws, saved=bufs.saved)
        if bwd:
            g = grads
            moe.moe_layer_bwd(cfg, Wr, bias, bufs.packed, x, g["dout"], bufs.saved, g["dx"], g["dWg"], g["dWu"],
                              g["dWd"], g["dWr"], bufs.ws, dWs=g["dWs"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    moe.moe_timing_enable(True)
    torch.cuda.synchronize()
    try:
        if cold_cache:
            # the scratch writes stay outside the timed events (and outside the
            # per-kernel timing, which only sees the library's launches)
            scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps)]
            for i in range(steps):
                scratch.fill_(i & 0xff)
                evs[i][0].record()
                step()
                evs[i][1].record()
            torch.cuda.synchronize()
            elapsed = sum(a.elapsed_time(b) for a, b in evs) / 1e3
            del scratch
        else:
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            elapsed = time.perf_counter() - t0
        kt = moe.moe_timing_read()
    finally:
        moe.moe_timing_enable(False)  # waits for the recorded launches and destroys the events

    layer_kernel = kt["layer"][0] > 0
    flops = role_flops(T, H, I, k, w.shared_expert, mx, bwd, layer_kernel, mx_wgrad)
    symbol = {"gemm_gate_up": "mx_gemm_kernel<0>" if mx else "grouped_gemm_kernel<0>",
              "gemm_down": "mx_gemm_kernel<1>" if mx else "grouped_gemm_kernel<1>",
              "dgrad_down": "mx_gemm_kernel<1>" if mx else "grouped_gemm_kernel<1>",
              "dgrad_gate_up": "mx_gemm_kernel<1>" if mx else "grouped_gemm_kernel<1>",
              # bf16: <1> gate|up (x rows gathered), <2> down (dout rows gathered), one launch each
              "wgrad": "mx_wgrad_kernel" if mx_wgrad else "wgrad_kernel<1|2>",
              "shared_gemm": "grouped_gemm_kernel (bf16 shared expert)",
              # bf16 tiles compiled in: a bf16 layer, or the shared expert's
              # tiles of an MXFP8 inference forward
              "layer": "mega_kernel<%s, %s>" % ("true" if mx else "false",
                                                 "true" if (not mx or (w.shared_expert and not bwd)) else "false")}
    by_sym = {}
    for kd, fl in flops.items():
        n, ms = kt[kd]
        agg = by_sym.setdefault(symbol[kd], [0.0, 0.0, 0, []])
        agg[0] += fl * steps
        agg[1] += ms
        agg[2] += n
        agg[3].append(kd)
    ms_step = elapsed * 1e3 / steps
    dom = max(by_sym, key=lambda sy: by_sym[sy][1])
    dom_flops, ms_dom, n_dom, dom_roles = by_sym[dom]
    achieved = dom_flops / (ms_dom / 1e3) / 1e12
    # the scaled-MFMA kernels (and the MXFP8 layer kernel) are priced at the FP8 peak
    peak = PEAK_FP8_TFLOPS if (mx and (dom.startswith("mx_") or dom.startswith("mega_kernel<true"))) else PEAK_BF16_TFLOPS
    nbytes = role_bytes(T, H, I, k, E, w.shared_expert, mx, bwd, layer_kernel, mx_wgrad)
    res = {
        "value": T * steps / elapsed,
        "ms_per_step": ms_step,
        "config": {"workload": w.name, "tokens": T, "hidden": H, "intermediate": I, "experts": E,
                   "top_k": k, "minibatch": sizes.minibatch, "minibatches": sizes.num_minibatches,
                   "router_bias": w.router_bias, "shared_expert": w.shared_expert, "precision": w.prec,
                   "ring_slots": sizes.ring_slots, "comm_cus": sizes.comm_cus,
                   "forward": "persistent layer kernel" if layer_kernel else "per-GEMM launches",
                   "pass": "forward+backward" if bwd else "forward",
                   "weight_gradients": ("mxfp8" if mx_wgrad else "bf16") if bwd else None,
                   "cache": "cold: 512 MiB written before each step" if cold_cache else "warm"},
        "roofline": {"bound": "mfma", "kernel": "moe::" + dom, "roles": dom_roles,
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic_for(dom, w.name),
                     "avg_launch_ms": ms_dom / max(n_dom, 1), "launches": n_dom},
        "detail": {
            "layer_mfma_frac": sum(flops.values()) / (ms_step / 1e3) / 1e12 / (PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS),
            "tflops_by_role": {kd: flops[kd] * steps / (kt[kd][1] / 1e3) / 1e12 for kd in flops if kt[kd][1] > 0},
            # algorithmic bytes (padding rows excluded) over the kind's event time
            "hbm_gbs_by_role": {kd: b * steps / (kt[kd][1] / 1e3) / 1e9 for kd, b in nbytes.items() if kt[kd][1] > 0},
            "per_step_ms": {kind: v[1] / steps for kind, v in kt.items() if kind != "dropped"},
            "timing_dropped": kt["dropped"],
        },
    }
    if mfma_loops:
        loops = {"bf16": mfma_loop(moe, torch, x, inp.Wg, False)}
        if mx:
            loops["mxfp8"] = mfma_loop(moe, torch, x, inp.Wg, True)
        res["detail"]["mfma_loop"] = loops
        loop = loops["mxfp8" if peak == PEAK_FP8_TFLOPS else "bf16"]
        res["roofline"]["sustained_peak"] = loop["tflops"]
        res["roofline"]["frac_of_sustained"] = achieved / loop["tflops"]
    if keep_inputs:
        res["inputs"] = inp
    del bufs, x, Wr, bias, out, grads
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def role_bytes(T: int, H: int, I: int, k: int, E: int, shared: bool, mx: bool, bwd: bool, layer_kernel: bool,
               mx_wgrad: bool = False) -> dict:
    """Algorithmic HBM bytes per step of the data-movement kernel kinds (routed
    and shared rows; padding rows excluded):
      route: x read once, router weight, indices and weights written (MXFP8:
        the dispatch-side E4M3 codes and E8M0 scales of every token row);
      combine (per-GEMM forward): k (+1 shared) expert-output rows read and one
        output row written per token; in a backward step the kind is the
        reverse-dispatch: k (+1) input-gradient rows read, dx written;
      gather (backward): reverse-combine (dout rows read, and Y rows of the
        routed rows; MXFP8 codes + scales of dY) and SwiGLU backward (dH and
        g|u read, fp32 under MXFP8; row-major dG|dU and w*h written for the
        rows whose weight gradients take bf16 operands, MXFP8 codes + scales
        of dG|dU for the MXFP8 input gradient).  With MXFP8 weight gradients
        (mx_wgrad) the routed rows' x rows are read too, and their dY, x,
        dG|dU and h are written transposed as codes + scales."""
    ks = k + (1 if shared else 0)
    R, Rr = T * ks, T * k  # rows (routed + shared), routed rows
    q = 1.0 + 1.0 / 32  # MXFP8 code + scale bytes per element
    b = {"route": T * H * 2 + H * E * 4 + T * k * 8 + (T * H * q if mx else 0.0)}
    if bwd:
        b["combine"] = T * (ks * H * 2 + H * 2)
        rows_mx = Rr if mx else 0
        rows_w = Rr if (mx and mx_wgrad) else 0  # quantised weight-gradient operands
        f = 4 if mx else 2
        rcomb = R * H * 2 + Rr * H * 2 + rows_w * H * 2 + rows_w * 2 * H * q + rows_mx * H * q
        swiglu = R * 3 * I * f + (R - rows_w) * 3 * I * 2 + rows_w * 3 * I * q + rows_mx * 2 * I * q
        b["gather"] = rcomb + swiglu
    elif not layer_kernel:
        b["combine"] = T * (ks * H * 2 + H * 2)
    return b


def mfma_loop(moe, torch, x, w, mx: bool) -> dict:
    """Sustained MFMA rate of the chip: a pure MFMA loop (one 8-wave workgroup
    per CU, no memory traffic) whose two operands are the layer's own values
    (one from x, one from the gate weights; bf16, or their MXFP8 E4M3 codes),
    then zeros.  Under this load the chip lowers its shader clock to its power
    budget, further for random mantissas than for zeros; the loop's rate is
    the ceiling a GEMM of that precision on such operands can reach here."""
    blocks = 256
    iters = 4096 if mx else 16384
    flops = blocks * 8.0 * iters * 32 * (131072 if mx else 32768)
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    xs = x.reshape(-1)[:16384].contiguous()
    ws = w.reshape(-1)[:16384].to("cuda").contiguous()
    if mx:
        def codes_of(v):
            c = torch.empty(v.numel(), dtype=torch.uint8, device="cuda")
            sc = torch.empty(v.numel() // 32, dtype=torch.uint8, device="cuda")
            moe.moe_mx_quantize(v.view(1, -1), c.view(1, -1), sc.view(1, -1))
            return c
        xs, ws = codes_of(xs), codes_of(ws)
    # lane t takes its first operand from piece 2t and its second from piece
    # 2t+1 (16 bytes per bf16 operand, 32 per E4M3 one): interleave x and W
    piece = 32 if mx else 8
    src = torch.stack([xs.view(-1, piece), ws.view(-1, piece)], 1).reshape(-1).contiguous()
    out = {"kind": "MXFP8 (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 codes of x and Wg)" if mx else
           "bf16 (v_mfma_f32_32x32x16_bf16, values of x and Wg)", "workgroups": blocks, "mfma_per_wave": iters * 32}
    for name, ops in (("", src), ("zeros_", torch.zeros_like(src))):
        moe.moe_diag_mfma_loop(1 if mx else 0, ops, blocks, 64, clocks, sink)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.moe_diag_mfma_loop(1 if mx else 0, ops, blocks, iters, clocks, sink)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        cyc, ref = clocks.tolist()
        out[name + "tflops"] = flops / (ms / 1e3) / 1e12
        out[name + "clock_ghz"] = cyc / (ref / 100e6) / 1e9
        out[name + "ms"] = ms
    return out


def role_flops(T: int, H: int, I: int, k: int, shared: bool, mx: bool, bwd: bool, layer_kernel: bool,
               mx_wgrad: bool = False) -> dict:
    """Algorithmic flops per step of each timing kind of the grouped GEMMs
    (padding rows excluded): 6*H*I per routed or shared row and pass (gate|up
    4*H*I, down 2*H*I), for the forward, the input gradients and the weight
    gradients.  MXFP8 runs the routed experts on the scaled-MFMA kernels and
    the shared expert in bf16: its backward input-gradient launches are their
    own kind, and so are its forward GEMMs, except in an inference forward
    through the persistent layer kernel, which runs them as tiles of its own
    (a training forward runs them as two launches before the layer kernel).  With MXFP8 weight gradients
    (mx_wgrad) the weight-gradient kind is the routed experts' scaled-MFMA
    launches and the shared expert's bf16 weight gradients join its kind.
    bf16 runs both in the same launches."""
    shared_rows = T if shared else 0
    hi = float(H) * I * (T * k + shared_rows)
    hr = float(H) * I * (T * k if mx else T * k + shared_rows)
    flops = {"gemm_gate_up": 4 * hr, "gemm_down": 2 * hr}
    if bwd:
        flops.update({"dgrad_down": 2 * hr, "dgrad_gate_up": 4 * hr,
                      "wgrad": 6 * (float(H) * I * T * k if (mx and mx_wgrad) else hi)})
    shared_fwd = 6.0 * H * I * shared_rows if mx else 0.0
    if mx and shared_rows and bwd:  # the shared expert's bf16 input-gradient (and weight-gradient) GEMMs
        flops["shared_gemm"] = 6.0 * H * I * shared_rows * (2 if mx_wgrad else 1)
    if layer_kernel:
        # the persistent layer kernel runs both forward GEMMs (and combine);
        # under MXFP8 the shared expert's bf16 tiles run in it for inference
        # and as launches of their own before it in training
        in_layer = shared_fwd if not bwd else 0.0
        flops["layer"] = flops.pop("gemm_gate_up") + flops.pop("gemm_down") + in_layer
        if shared_fwd and bwd:
            flops["shared_gemm"] = flops.get("shared_gemm", 0.0) + shared_fwd
    elif shared_fwd:  # per-GEMM forward: the shared expert's launches are timed as their own kind
        flops["shared_gemm"] = flops.get("shared_gemm", 0.0) + shared_fwd
    return flops


def traffic_for(symbol: str, workload: str):
    """HBM bytes per launch of `symbol` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or
    None when there is none for this workload or the kernel source changed
    since the counters were taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    # "name<a|b>": the mean over the instances name<a> and name<b>
    names = [symbol]
    if "|" in symbol and symbol.endswith(">"):
        base, inner = symbol[:-1].split("<", 1)
        names = ["%s<%s>" % (base, v) for v in inner.split("|")]
    vals = []
    for nm in names:
        ent = rec.get("kernels", {}).get("moe::%s@%s" % (nm, workload))
        if not ent or ent.get("source_sha256") != _source_sha():
            return None
        vals.append(ent["hbm_bytes_per_launch"])
    return sum(vals) / len(vals)


def _kernel_symbol(name: str) -> str:
    return name.split("(")[0].replace("void ", "").strip()


def _source_sha() -> str:
    """Hash of every kernel source: counter figures go stale with any change."""
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dispatch_grouped_gemm_moe_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def summarize_stats(path: str, title: str, cmd: str):
    import csv
    rows = list(csv.DictReader(open(path)))
    print("# %s\n" % title)
    print("Command (run from the repository root on one MI355X):\n\n```\n%s\n```\n" % cmd)
    print("| kernel | calls | total ms | avg us | min us | max us | % |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        print("| %s | %s | %.3f | %.1f | %.1f | %.1f | %.2f |" % (
            _kernel_symbol(r["Name"])[:90], r["Calls"], int(r["TotalDurationNs"]) / 1e6,
            float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["Percentage"])))


def summarize_traffic(fetch_csv: str, write_csv: str, workload: str, copy_mib: int):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each moe:: kernel, scaled so
    that the plain copy of copy_mib MiB reads and writes exactly that much."""
    import csv
    from collections import defaultdict
    if not copy_mib:
        sys.exit("--summarize-traffic needs the --calibrate-copy-mib the runs were taken with")

    def per_symbol(path, counter):
        acc = defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                acc[_kernel_symbol(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        return acc

    fetch, write = per_symbol(fetch_csv, "FETCH_SIZE"), per_symbol(write_csv, "WRITE_SIZE")
    copy = [s for s in fetch if "neg_kernel" in s]
    if len(copy) != 1 or len(fetch[copy[0]]) != 1:
        sys.exit("expected exactly one copy (negation) dispatch in %s" % fetch_csv)
    kib = copy_mib * 1024.0
    f_fac, w_fac = kib / fetch[copy[0]][0], kib / write[copy[0]][0]
    here = os.path.dirname(os.path.abspath(__file__))
    out = os.path.join(here, "profiles", "traffic.json")
    rec = json.load(open(out)) if os.path.exists(out) else {"kernels": {}}
    sha = _source_sha()  # entries taken on other sources are stale: drop them
    rec["kernels"] = {k: v for k, v in rec.get("kernels", {}).items() if v.get("source_sha256") == sha}
    rec["note"] = ("HBM bytes per launch = mean FETCH_SIZE * fetch_factor + mean WRITE_SIZE * write_factor "
                   "(KiB -> bytes); the factors make a plain %d MiB elementwise copy read and write "
                   "exactly %d MiB" % (copy_mib, copy_mib))
    for sym in fetch:
        if not sym.startswith("moe::") or sym not in write:
            continue
        fk = sum(fetch[sym]) / len(fetch[sym])
        wk = sum(write[sym]) / len(write[sym])
        rec["kernels"]["%s@%s" % (sym, workload)] = {
            "dispatches": len(fetch[sym]), "fetch_kib": fk, "write_kib": wk,
            "fetch_factor": f_fac, "write_factor": w_fac,
            "hbm_bytes_per_launch": (fk * f_fac + wk * w_fac) * 1024.0,
            "source_sha256": sha}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps({k: v["hbm_bytes_per_launch"] for k, v in rec["kernels"].items()}, indent=1))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, n_tokens: int, bwd: bool) -> dict:
    """The CPU oracle (as it stands) on the first n_tokens tokens of the workload,
    taken as a layer of n_tokens tokens with the same weights.  The oracle
    widens every expert's bf16 weights to fp64 (a cost independent of the
    token count), timed on its own as well so that the sample's share of it is
    visible."""
    import numpy as np
    import threadpoolctl
    import oracle
    from moe_inputs import LayerInputs

    n = min(n_tokens, inp.w.T)
    sub = LayerInputs(inp.w.replace(T=n), inp.x[:n], inp.Wr, inp.bias, inp.Wg, inp.Wu, inp.Wd,
                      inp.Wsg, inp.Wsu, inp.Wsd, inp.dout[:n] if inp.dout is not None else None)
    oracle.router_logits(np.zeros((1, inp.w.H), np.float32), np.zeros((inp.w.H, 1), np.float32))
    mx = inp.w.prec == "mxfp8"
    t0 = time.perf_counter()
    fwd = oracle.layer_forward(sub, keep=bwd)
    if bwd:  # MXFP8: the weight gradients' row quantisation too, as the library runs it by default
        oracle.layer_backward(sub, fwd=fwd, mx_wgrad_minibatch=inp.w.minibatch if mx else None)
    dt = time.perf_counter() - t0
    t0 = time.perf_counter()
    for e in range(inp.w.E):  # the per-expert fp64 widening alone
        for t in (inp.Wg, inp.Wu, inp.Wd):
            oracle.as_f64(t[e])
    dt_w = time.perf_counter() - t0
    blas = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    omp = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": n / dt, "unit": "tokens/s", "cores": max(blas, omp), "kind": "oracle",
            "cpu": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "first %d of %d tokens as a %d-token layer: fixed-order fp32 routing (C, OpenMP) + "
                      "fp64 expert SwiGLU FFN and combine%s%s (numpy/OpenBLAS, fp64 throughout, not tuned); "
                      "%.1f s, of which about %.1f s widen the expert weights to fp64 %s"
                      % (n, inp.w.T, n, " + fp64 backward" if bwd else "",
                         " with the MXFP8 quantisation points (C quantiser)" if mx else "", dt, dt_w,
                         "(twice: forward and backward)" if bwd else "(once)")}


if __name__ == "__main__":
    main()
