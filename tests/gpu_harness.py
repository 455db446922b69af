"""Helpers of the GPU tests: upload a workload's inputs, run the library
through its binding, read results back.  No layer arithmetic here."""
import torch

import dispatch_grouped_gemm_moe_amd as moe


def cfg_of(w, minibatch=None, flags=0, T=None):
    if w.shared_expert:
        flags |= moe.MOE_F_SHARED_EXPERT
    return moe.make_cfg(T or w.T, w.H, w.I, w.E, w.k,
                        minibatch=w.minibatch if minibatch is None else minibatch,
                        prec=moe.MOE_PREC_MXFP8 if w.prec == "mxfp8" else moe.MOE_PREC_BF16,
                        flags=flags)


class Layer:
    """One layer's device tensors and packed weights."""

    def __init__(self, inp, minibatch=None, flags=0, device="cuda", ring_slots=0, comm_cus=0):
        w = inp.w
        self.inp, self.cfg = inp, cfg_of(w, minibatch, flags)
        self.cfg.ring_slots, self.cfg.comm_cus = ring_slots, comm_cus
        self.bufs = moe.alloc_buffers(self.cfg, device=device, with_saved=True)
        dev = lambda t: None if t is None else t.to(device).contiguous()
        self.x, self.Wr, self.bias = dev(inp.x), dev(inp.Wr), dev(inp.bias)
        Wg, Wu, Wd = dev(inp.Wg), dev(inp.Wu), dev(inp.Wd)
        moe.moe_prepare_weights(self.cfg, Wg, Wu, Wd, self.bufs.packed,
                                dev(inp.Wsg), dev(inp.Wsu), dev(inp.Wsd))
        torch.cuda.synchronize()
        del Wg, Wu, Wd
        self.out = torch.empty_like(self.x)

    def forward(self, keep=True):
        """keep=False runs the inference forward (nothing saved for a backward)."""
        moe.moe_layer_fwd(self.cfg, self.Wr, self.bias, self.bufs.packed, self.x, self.out,
                          self.bufs.ws, saved=self.bufs.saved if keep else None)
        return self.out

    def forward_path(self, keep=True):
        """Runs forward(keep) and reports which path it took: "layer kernel" if
        the persistent layer kernel was launched (once), "per-GEMM" if the
        forward ran one launch per grouped GEMM (the library's launch timing)."""
        torch.cuda.synchronize()
        moe.moe_timing_enable(True)
        try:
            self.forward(keep)
            kt = moe.moe_timing_read()
        finally:
            moe.moe_timing_enable(False)
        layer, per_gemm = kt["layer"][0], kt["gemm_gate_up"][0] + kt["shared_gemm"][0] + kt["gather"][0]
        assert layer in (0, 1), kt
        return "layer kernel" if layer == 1 else ("per-GEMM" if per_gemm else "none")

    def device_status(self):
        return moe.moe_read_device_status(self.bufs.ws)

    def backward(self, dout, with_dgate=True, to_cpu=True):
        """Gradients of sum(out * dout); returns a dict of CPU float tensors, or
        of the device tensors themselves with to_cpu=False."""
        w = self.inp.w
        dev = self.x.device
        T, H, I, E, k = w.T, w.H, w.I, w.E, w.k
        g = {
            "dx": torch.empty(T, H, dtype=torch.bfloat16, device=dev),
            "dWg": torch.empty(E, H, I, dtype=torch.float32, device=dev),
            "dWu": torch.empty(E, H, I, dtype=torch.float32, device=dev),
            "dWd": torch.empty(E, I, H, dtype=torch.float32, device=dev),
            "dWr": torch.empty(H, E, dtype=torch.float32, device=dev),
        }
        dWs = torch.empty(2 * H * I + I * H, dtype=torch.float32, device=dev) if w.shared_expert else None
        dgate = torch.empty(T, k, dtype=torch.float32, device=dev) if with_dgate else None
        moe.moe_layer_bwd(self.cfg, self.Wr, self.bias, self.bufs.packed, self.x, dout.to(dev).contiguous(),
                          self.bufs.saved, g["dx"], g["dWg"], g["dWu"], g["dWd"], g["dWr"], self.bufs.ws,
                          dWs=dWs, dgate=dgate)
        torch.cuda.synchronize()
        host = (lambda t: t.float().cpu()) if to_cpu else (lambda t: t)
        res = {n: host(t) for n, t in g.items()}
        if dgate is not None:
            res["dgate"] = host(dgate)
        if dWs is not None:
            res["dWsg"] = host(dWs[:H * I].view(H, I))
            res["dWsu"] = host(dWs[H * I:2 * H * I].view(H, I))
            res["dWsd"] = host(dWs[2 * H * I:].view(I, H))
        return res

    def saved_routing(self):
        T, k = self.cfg.T, self.cfg.k
        n = T * k * 4
        off = (n + 255) // 256 * 256
        raw = self.bufs.saved
        idx = raw[:n].view(torch.int32).view(T, k)
        w = raw[off:off + n].view(torch.float32).view(T, k)
        return idx, w
