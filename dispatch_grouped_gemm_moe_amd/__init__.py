"""Python binding of the MI355X fused MoE layer library (include/moe.h).

Argument marshalling only: every entry point below forwards torch tensors'
device pointers and the caller's current HIP stream to the C ABI function of
the same name in ``_lib/libmoe_mi355x.so``.  All computation happens in the
library's HIP kernels; there is no CPU or PyTorch fallback.  Importing this
package fails loudly if the library has not been built
(``python -m dispatch_grouped_gemm_moe_amd.build``).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

from .build import lib_path

MOE_OK, MOE_E_INVALID, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_HIP, MOE_E_DEVICE = range(6)
MOE_PREC_BF16, MOE_PREC_MXFP8 = 0, 1
MOE_F_SHARED_EXPERT = 1 << 0
MOE_F_IDENTITY_EXPERTS = 1 << 1
MOE_F_LAUNCH_PER_GEMM = 1 << 2
MOE_F_DEBUG_DROP_SIGNAL = 1 << 3
MOE_F_BF16_WGRAD = 1 << 4
MOE_DEV_OK, MOE_DEV_WAIT_TIMEOUT = 0, 1

# every symbol include/moe.h declares
EXPORTS = ("moe_status_string", "moe_abi_version", "moe_validate_cfg", "moe_query_sizes",
           "moe_prepare_weights", "moe_route", "moe_dispatch_layout", "moe_layer_fwd",
           "moe_layer_bwd", "moe_read_device_status", "moe_mx_quantize", "moe_timing_enable",
           "moe_timing_read", "moe_diag_mfma_loop", "moe_layer_fwd_static")
MOE_STATIC_WORKSPACE_BYTES = 256 << 20
KERNEL_KINDS = ("route", "layout", "gemm_gate_up", "gemm_down", "combine", "gather", "other", "wgrad",
                "dgrad_down", "dgrad_gate_up", "shared_gemm", "layer")


class moe_cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("minibatch", ctypes.c_int32),
                ("ring_slots", ctypes.c_int32), ("comm_cus", ctypes.c_int32),
                ("prec", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class moe_sizes(ctypes.Structure):
    _fields_ = [("packed_weights", ctypes.c_size_t), ("workspace_fwd", ctypes.c_size_t),
                ("saved", ctypes.c_size_t), ("workspace_bwd", ctypes.c_size_t),
                ("minibatch", ctypes.c_int32), ("ring_slots", ctypes.c_int32),
                ("num_minibatches", ctypes.c_int32), ("comm_cus", ctypes.c_int32)]


class moe_weights(ctypes.Structure):
    _fields_ = [("Wr", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("packed", ctypes.c_void_p),
                ("packed_bytes", ctypes.c_size_t)]


class moe_kernel_times(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int32 * 12), ("ms", ctypes.c_double * 12), ("dropped", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s: %s (status %d)" % (fn, _load().moe_status_string(status).decode(), status))


_LIB = None


def _load():
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError("HIP library %s is missing: build it with "
                              "`python -m dispatch_grouped_gemm_moe_amd.build`" % path)
        lib = ctypes.CDLL(path)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cfgp = ctypes.POINTER(moe_cfg)
        sig = {
            "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_abi_version": (I32, []),
            "moe_validate_cfg": (ctypes.c_int, [cfgp]),
            "moe_query_sizes": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_sizes)]),
            "moe_prepare_weights": (ctypes.c_int, [cfgp, P, P, P, P, P, P, P, SZ, P]),
            "moe_route": (ctypes.c_int, [cfgp, P, P, P, P, P, P, P, P, P]),
            "moe_dispatch_layout": (ctypes.c_int, [cfgp, P, P, P, P, P, P]),
            "moe_layer_fwd": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_weights), P, P, P, SZ, P, SZ, P]),
            "moe_layer_bwd": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_weights), P, P, P, SZ, P, P, P,
                                             P, P, P, P, P, SZ, P]),
            "moe_read_device_status": (ctypes.c_int, [P, P, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
            "moe_mx_quantize": (ctypes.c_int, [P, ctypes.c_int64, I32, P, P, P]),
            "moe_timing_enable": (ctypes.c_int, [I32]),
            "moe_timing_read": (ctypes.c_int, [ctypes.POINTER(moe_kernel_times)]),
            "moe_diag_mfma_loop": (ctypes.c_int, [I32, P, ctypes.c_int64, I32, I32, P, P, P]),
            "moe_layer_fwd_static": (ctypes.c_int, [cfgp, ctypes.POINTER(moe_weights), P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (loads it on first use)."""
    return _load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st)


def make_cfg(T, H, I, E, k, minibatch=0, ring_slots=0, comm_cus=0, prec=MOE_PREC_BF16, flags=0) -> moe_cfg:
    return moe_cfg(T, H, I, E, k, minibatch, ring_slots, comm_cus, prec, flags)


# ---------------------------------------------------------------- entry points

def moe_abi_version() -> int:
    return _load().moe_abi_version()


def moe_validate_cfg(cfg: moe_cfg) -> int:
    return _load().moe_validate_cfg(ctypes.byref(cfg))


def moe_query_sizes(cfg: moe_cfg) -> moe_sizes:
    s = moe_sizes()
    _check("moe_query_sizes", _load().moe_query_sizes(ctypes.byref(cfg), ctypes.byref(s)))
    return s


def moe_prepare_weights(cfg, Wg, Wu, Wd, packed, Wsg=None, Wsu=None, Wsd=None, stream=None):
    _check("moe_prepare_weights", _load().moe_prepare_weights(
        ctypes.byref(cfg), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(Wsg), _ptr(Wsu), _ptr(Wsd),
        _ptr(packed), packed.numel() * packed.element_size(), _stream(stream)))


def moe_route(cfg, x, Wr, bias, topk_idx, topk_w, logits=None, x_codes=None, x_scales=None, stream=None):
    _check("moe_route", _load().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(Wr), _ptr(bias),
                                          _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(x_codes),
                                          _ptr(x_scales), _stream(stream)))


def moe_dispatch_layout(cfg, topk_idx, counts, offsets, row_token, tok_row, stream=None):
    _check("moe_dispatch_layout", _load().moe_dispatch_layout(
        ctypes.byref(cfg), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(row_token),
        _ptr(tok_row), _stream(stream)))


def _weights(Wr, bias, packed) -> moe_weights:
    return moe_weights(Wr.data_ptr(), bias.data_ptr() if bias is not None else None,
                       packed.data_ptr(), packed.numel() * packed.element_size())


def moe_layer_fwd(cfg, Wr, bias, packed, x, out, ws, saved=None, stream=None):
    w = _weights(Wr, bias, packed)
    _check("moe_layer_fwd", _load().moe_layer_fwd(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), _ptr(saved),
        0 if saved is None else saved.numel() * saved.element_size(), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_fwd_static(cfg, Wr, bias, packed, x, out, status=None, stream=None):
    """Forward on the library's static workspace (allocates nothing); status: an
    int32 device tensor of 2 elements that receives the device status word."""
    w = _weights(Wr, bias, packed)
    _check("moe_layer_fwd_static", _load().moe_layer_fwd_static(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(out), _ptr(status), _stream(stream)))


def moe_layer_bwd(cfg, Wr, bias, packed, x, dout, saved, dx, dWg, dWu, dWd, dWr, ws,
                  dWs=None, dgate=None, stream=None):
    w = _weights(Wr, bias, packed)
    _check("moe_layer_bwd", _load().moe_layer_bwd(
        ctypes.byref(cfg), ctypes.byref(w), _ptr(x), _ptr(dout), _ptr(saved),
        saved.numel() * saved.element_size(), _ptr(dx), _ptr(dWg), _ptr(dWu), _ptr(dWd), _ptr(dWr),
        _ptr(dWs), _ptr(dgate), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_read_device_status(ws, stream=None):
    code, detail = ctypes.c_int32(0), ctypes.c_int32(0)
    st = _load().moe_read_device_status(_ptr(ws), _stream(stream), ctypes.byref(code), ctypes.byref(detail))
    return st, code.value, detail.value


def moe_mx_quantize(src, codes, scales, stream=None):
    rows, cols = src.shape
    _check("moe_mx_quantize", _load().moe_mx_quantize(_ptr(src), rows, cols, _ptr(codes), _ptr(scales),
                                                      _stream(stream)))


def moe_diag_mfma_loop(kind, operands, blocks, iters, clocks, sink, stream=None):
    """Sustained-MFMA diagnostic: kind 0 = bf16, 1 = MXFP8 (E4M3 codes); operands
    >= 16 KiB, clocks int64 [2], sink fp32 [blocks*512]."""
    _check("moe_diag_mfma_loop", _load().moe_diag_mfma_loop(kind, _ptr(operands),
                                                            operands.numel() * operands.element_size(), blocks,
                                                            iters, _ptr(clocks), _ptr(sink), _stream(stream)))


def moe_timing_enable(on: bool):
    _check("moe_timing_enable", _load().moe_timing_enable(1 if on else 0))


def moe_timing_read() -> dict:
    """{kind: (launches, total_ms)} since the last moe_timing_enable(True)."""
    t = moe_kernel_times()
    _check("moe_timing_read", _load().moe_timing_read(ctypes.byref(t)))
    res = {n: (t.launches[i], t.ms[i]) for i, n in enumerate(KERNEL_KINDS)}
    res["dropped"] = t.dropped
    return res


# ---------------------------------------------------------------- buffers

@dataclasses.dataclass
class LayerBuffers:
    """Device buffers of one layer configuration, allocated with torch."""

    cfg: moe_cfg
    sizes: moe_sizes
    packed: object
    ws: object
    saved: object | None


def alloc_buffers(cfg: moe_cfg, device="cuda", with_saved=False) -> LayerBuffers:
    import torch
    s = moe_query_sizes(cfg)
    packed = torch.empty(s.packed_weights, dtype=torch.uint8, device=device)
    ws = torch.zeros(max(s.workspace_fwd, s.workspace_bwd) if with_saved else s.workspace_fwd,
                     dtype=torch.uint8, device=device)
    saved = torch.empty(s.saved, dtype=torch.uint8, device=device) if with_saved else None
    return LayerBuffers(cfg, s, packed, ws, saved)
