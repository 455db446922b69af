"""CPU oracle of the fused MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call or link anything in this
package.  It shares no code with the GPU library: no kernels, headers, helpers
or tables.  Inputs come from ``moe_inputs`` (seeded draws, no layer math).

What the layer computes, as the pages describe it:

* a router picks several experts for every token, re-deciding at every step
  (KuCoin flash "Cursor's MoK achieves 2.37x performance boost on NVIDIA GB300
  NVL72", section 01);
* the tokens of each expert are counted and placed next to each other so that
  one grouped GEMM can run every expert's FFN (same page, section 01);
* the expert FFN is SwiGLU (same page, section 02, on fusing MXFP8 into the
  dispatch / grouped GEMM / SwiGLU data path);
* combine returns every expert result to its token's position and a final
  weighted sum forms the layer output (same page, sections 02 and 03);
* the backward pass runs the exchanges in reverse (section 01);
* MoK supports BF16 and MXFP8 and keeps the shared expert in BF16
  (RuntimeWire "Cursor open-sources MoK", section "Rebuilding the MoE layer
  around communication").

Readings taken where the pages are silent (each is listed in the design
notes): softmax over the top-k logits (the renormalised top-k softmax);
logits summed in the fixed fp32 order of ``router_logits.c``; ties go to the
lower expert index; slots of a token ordered by descending logit; rows of an
expert ordered by ascending token; SwiGLU is silu(x Wg) * (x Wu) then Wd, no
biases; the shared expert is ungated with weight 1; MXFP8 follows the OCP
Microscaling v1.0 formats (E4M3 elements, E8M0 scale per 32 elements along
the contraction axis) with the scale chosen as the smallest power of two that
keeps the block maximum within 448.

Floating-point policy: routing logits are fp32 in the fixed order (they decide
integers, so both sides decide in the kernel's precision).  Gate weights, the
FFN, combine and the backward pass are fp64 on the exact values of the bf16
inputs, so the oracle is as close to the exact result as fp64 allows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "router_logits.c"), os.path.join(_HERE, "mx_quant.c")]
_BUILD = os.path.join(_HERE, "_build")
_SO = os.path.join(_BUILD, "liboracle_router.so")
_lib_handle = None


# --------------------------------------------------------------------------
# build / load the C part
# --------------------------------------------------------------------------

def build() -> str:
    """Compile the C part of the oracle (gcc, OpenMP).  Returns the .so path."""
    os.makedirs(_BUILD, exist_ok=True)
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", *_SRCS, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < max(os.path.getmtime(f) for f in _SRCS):
            build()
        lib = ctypes.CDLL(_SO)
        fp = ctypes.POINTER(ctypes.c_float)
        lib.oracle_router_logits.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             fp, fp, fp, fp]
        lib.oracle_router_logits.restype = ctypes.c_int
        u8 = ctypes.POINTER(ctypes.c_uint8)
        lib.oracle_mx_quantize.argtypes = [ctypes.c_int64, ctypes.c_int, fp, u8, u8]
        lib.oracle_mx_quantize.restype = None
        _lib_handle = lib
    return _lib_handle


def as_f32(a) -> np.ndarray:
    """torch tensor (bf16/fp32) or array -> contiguous float32 numpy (bf16 widens exactly)."""
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu", torch.float32).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def as_f64(a) -> np.ndarray:
    """torch tensor or array -> contiguous float64 numpy (no fp32 detour for fp64 input)."""
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


# --------------------------------------------------------------------------
# routing (section 01: the router picks experts for every token)
# --------------------------------------------------------------------------

def router_logits(x, Wr, bias=None) -> np.ndarray:
    """fp32 logits [T, E] in the fixed summation order of router_logits.c."""
    x32, W32 = as_f32(x), as_f32(Wr)
    T, H = x32.shape
    E = W32.shape[1]
    assert W32.shape[0] == H
    out = np.empty((T, E), dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    b32 = as_f32(bias) if bias is not None else None
    rc = _lib().oracle_router_logits(
        T, H, E, x32.ctypes.data_as(fp), W32.ctypes.data_as(fp),
        b32.ctypes.data_as(fp) if b32 is not None else None, out.ctypes.data_as(fp))
    if rc != 0:
        raise ValueError("router logits need H to be a multiple of 64 (got H=%d)" % H)
    return out


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """The k experts of largest logit per token, in descending-logit order.

    Equal logits (IEEE equality, so -0 == +0) keep the lower expert index first.
    """
    assert np.isfinite(logits).all(), "router logits must be finite"
    order = np.argsort(-logits, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k].astype(np.int32))


def gate_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over each token's k selected logits (fp64).

    Equal to the full softmax over all experts renormalised over the selection.
    """
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def route(x, Wr, bias, k: int):
    """(logits fp32 [T,E], idx int32 [T,k], w fp64 [T,k])."""
    logits = router_logits(x, Wr, bias)
    idx = topk_select(logits, k)
    return logits, idx, gate_weights(logits, idx)


# --------------------------------------------------------------------------
# dispatch layout (section 01: count per expert, place each expert's tokens
# next to each other for the grouped GEMM)
# --------------------------------------------------------------------------

def dispatch_layout(idx: np.ndarray, E: int):
    """counts [E], offsets [E+1], row_token [T*k], tok_row [T,k] (all int32).

    Rows of expert e occupy offsets[e] .. offsets[e+1]-1, in ascending token
    order.  row_token[r] is the token of row r; tok_row[t,j] is the row that
    holds slot j of token t.  Plain counting placement, token by token.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for e in idx.ravel():
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    row_token = np.empty(T * k, dtype=np.int32)
    tok_row = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            r = fill[e]
            fill[e] += 1
            row_token[r] = t
            tok_row[t, j] = r
    return counts.astype(np.int32), offsets.astype(np.int32), row_token, tok_row


def minibatch_layouts(idx: np.ndarray, E: int, minibatch: int):
    """dispatch_layout of every minibatch slice [b*M, min(T,(b+1)*M)); rows and
    tokens are relative to the slice."""
    T = idx.shape[0]
    return [dispatch_layout(idx[t0:min(T, t0 + minibatch)], E) for t0 in range(0, T, minibatch)]


# --------------------------------------------------------------------------
# MXFP8 (OCP Microscaling v1.0: E4M3 elements, E8M0 scale per 32 elements)
# --------------------------------------------------------------------------

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_value(code: int) -> float:
    """Decode one OCP E4M3 ("FN") byte: bias 7, 3 mantissa bits, no infinities,
    S.1111.111 is NaN."""
    s = -1.0 if code & 0x80 else 1.0
    ex = (code >> 3) & 0xF
    m = code & 0x7
    if ex == 0xF and m == 0x7:
        return float("nan")
    if ex == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (ex - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes 0x00..0x7E in increasing value order
_POS_VALUES = E4M3_TABLE[:0x7F]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round fp values to the nearest E4M3 code, ties to the even code, saturating
    at +-448 (values must be finite)."""
    v = np.asarray(v, dtype=np.float64)
    assert np.isfinite(v).all()
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS_VALUES[hi], hi, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def e8m0_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127]; 0 for
    an all-zero block (its E8M0 byte is then 127, a scale of 1)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, p = np.frexp(amax)  # amax = m * 2^p, m in [0.5, 1)
    # 448 = 0.875 * 2^9: m <= 0.875 needs e = p - 9, larger m one more.
    e = p - 9 + (m > 0.875)
    e = np.where(amax == 0, 0, e)
    return np.clip(e, -127, 127).astype(np.int64)


def mx_quantize(a, axis: int):
    """Quantise along `axis` in blocks of 32: (codes uint8 same shape, scale bytes
    uint8 with that axis divided by 32).  The input is taken in fp32; the work
    is done by oracle_mx_quantize (mx_quant.c), the same rules as e4m3_encode
    and e8m0_scale_exponent above."""
    a32 = np.moveaxis(as_f32(a), axis, -1)
    shape = a32.shape
    n = shape[-1]
    assert n % MX_BLOCK == 0
    flat = np.ascontiguousarray(a32.reshape(-1, n))
    assert np.isfinite(flat).all()
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty((flat.shape[0], n // MX_BLOCK), dtype=np.uint8)
    u8 = ctypes.POINTER(ctypes.c_uint8)
    _lib().oracle_mx_quantize(flat.shape[0], n, flat.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                              codes.ctypes.data_as(u8), scales.ctypes.data_as(u8))
    codes = np.moveaxis(codes.reshape(shape), -1, axis)
    scales = np.moveaxis(scales.reshape(shape[:-1] + (n // MX_BLOCK,)), -1, axis)
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)


def mx_quantize_reference(a, axis: int):
    """The same quantisation written with the Python helpers (slow; used to
    check the C quantiser)."""
    a32 = as_f32(a).astype(np.float64)
    a32 = np.moveaxis(a32, axis, -1)
    n = a32.shape[-1]
    blk = a32.reshape(a32.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    e = e8m0_scale_exponent(np.abs(blk).max(axis=-1))
    codes = e4m3_encode(blk / np.ldexp(1.0, e)[..., None])
    codes = np.moveaxis(codes.reshape(a32.shape), -1, axis)
    scales = np.moveaxis((e + 127).astype(np.uint8), -1, axis)
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, axis: int) -> np.ndarray:
    c = np.moveaxis(codes, axis, -1)
    s = np.moveaxis(scales, axis, -1).astype(np.int64) - 127
    v = E4M3_TABLE[c].reshape(c.shape[:-1] + (c.shape[-1] // MX_BLOCK, MX_BLOCK))
    v = v * np.ldexp(1.0, s)[..., None]
    return np.moveaxis(v.reshape(c.shape), -1, axis)


def mx_roundtrip(a, axis: int) -> np.ndarray:
    """Dequantised value of the MXFP8 quantisation of `a` along `axis` (fp64)."""
    return mx_dequantize(*mx_quantize(a, axis), axis=axis)


# --------------------------------------------------------------------------
# expert FFN, combine, layer forward
# --------------------------------------------------------------------------

def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def silu_grad(z):
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def expert_ffn(X, Wg, Wu, Wd, mx: bool = False):
    """SwiGLU FFN of one expert on rows X (fp64): returns y, g, u, h.

    With `mx`, h is rounded to fp32 and taken through the MXFP8 quantiser along
    its contraction axis before the down projection (the quantisation point of
    the SwiGLU epilogue); X and the weights are expected already dequantised.
    """
    g = X @ Wg
    u = X @ Wu
    h = silu(g) * u
    hq = mx_roundtrip(h.astype(np.float32), axis=1) if mx else h
    return hq @ Wd, g, u, h


class Weights:
    """fp64 views of one layer's parameters (exact values of the bf16 inputs),
    converted one expert at a time to bound memory."""

    def __init__(self, inp, mx: bool = False):
        self.inp = inp
        self.mx = mx
        self.E = inp.Wg.shape[0]

    def expert(self, e: int):
        Wg, Wu, Wd = (as_f64(t[e]) for t in (self.inp.Wg, self.inp.Wu, self.inp.Wd))
        if self.mx:  # forward quantisation axis = the contraction axis of each GEMM
            Wg, Wu, Wd = mx_roundtrip(Wg, 0), mx_roundtrip(Wu, 0), mx_roundtrip(Wd, 0)
        return Wg, Wu, Wd

    def expert_dgrad(self, e: int, quantizer=None):
        """Operands of the backward input-gradient GEMMs: Wg, Wu [H,I] and Wd [I,H]
        taken through `quantizer` along their contraction axis there (I for Wg and
        Wu, H for Wd: axis 1 each), or unquantised."""
        Wg, Wu, Wd = (as_f64(t[e]) for t in (self.inp.Wg, self.inp.Wu, self.inp.Wd))
        if quantizer is not None:
            Wg, Wu, Wd = quantizer(Wg, 1), quantizer(Wu, 1), quantizer(Wd, 1)
        return Wg, Wu, Wd

    def shared(self):
        return tuple(as_f64(t) for t in (self.inp.Wsg, self.inp.Wsu, self.inp.Wsd))


def layer_forward(inp, tokens=None, *, identity_experts: bool = False, mx: bool | None = None,
                  shared: bool | None = None, keep: bool = False, logits64: bool = False):
    """Forward of the MoE layer on `inp` (a moe_inputs.LayerInputs).

    tokens: optional array of token indices to evaluate (routing and the FFN are
    per token, so a subset gives exactly those tokens' outputs).
    Returns a dict with out [n,H] fp64, logits, idx, w, and with `keep` the
    per-slot expert outputs Y [n,k,H] and FFN intermediates for the backward.
    logits64: take the logits as the fp64 product x Wr (+ bias) instead of the
    fixed-order fp32 sum, which makes the forward a smooth function of x and Wr
    for finite-difference checks of the backward.
    """
    w_ = inp.w
    mx = (w_.prec == "mxfp8") if mx is None else mx
    shared = w_.shared_expert if shared is None else shared
    x64 = as_f64(inp.x)
    if tokens is not None:
        x64 = x64[np.asarray(tokens)]
    n, H = x64.shape
    k, E = w_.k, w_.E
    if logits64:
        logits = x64 @ as_f64(inp.Wr)
        if inp.bias is not None:
            logits = logits + as_f64(inp.bias)
        idx = topk_select(logits, k)
        gw = gate_weights(logits, idx)
    else:
        logits, idx, gw = route(x64.astype(np.float32), inp.Wr, inp.bias, k)
    xin = mx_roundtrip(x64, axis=1) if (mx and not identity_experts) else x64
    W = Weights(inp, mx=mx)
    Y = np.zeros((n, k, H), dtype=np.float64)
    saved = {}
    for e in range(E):
        t_sel, j_sel = np.nonzero(idx == e)  # a direct scan of the selection
        if t_sel.size == 0:
            continue
        if identity_experts:
            Y[t_sel, j_sel] = x64[t_sel]
            continue
        y, g, u, h = expert_ffn(xin[t_sel], *W.expert(e), mx=mx)
        Y[t_sel, j_sel] = y
        if keep:
            saved[e] = (t_sel, j_sel, g, u, h)
    out = np.zeros((n, H), dtype=np.float64)
    for j in range(k):  # final weighted sum, slots in order
        out += gw[:, j:j + 1] * Y[:, j, :]
    res = {"out": out, "logits": logits, "idx": idx, "w": gw, "x": x64, "xin": xin}
    if shared and not identity_experts:
        ys, gs, us, hs = expert_ffn(x64, *W.shared())
        out += ys
        res["shared"] = (gs, us, hs)
    if keep:
        res["Y"] = Y
        res["saved"] = saved
    return res


# --------------------------------------------------------------------------
# backward (section 01: the backward pass runs the exchanges in reverse)
# --------------------------------------------------------------------------

def mx_point(a, axis: int) -> np.ndarray:
    """A quantisation point of the MXFP8 layer: the value is rounded to fp32 (the
    precision it is produced in) and taken through the MXFP8 quantiser."""
    return mx_roundtrip(np.asarray(a, dtype=np.float64).astype(np.float32), axis)


def segment_rows_product(t_sel, A, B, minibatch, q):
    """sum over minibatches b of q(A_b)^T q(B_b), where A_b, B_b are the rows of
    A, B whose token t_sel lies in minibatch b ([b*minibatch, (b+1)*minibatch))
    and q quantises along the rows (axis 0), each segment on its own.  With
    q = None: A^T B."""
    if q is None:
        return A.T @ B
    out = np.zeros((A.shape[1], B.shape[1]))
    seg = np.asarray(t_sel) // minibatch
    for b in np.unique(seg):
        r = seg == b
        out += q(A[r], 0).T @ q(B[r], 0)
    return out


def mx_rows_point(a, axis: int) -> np.ndarray:
    """A weight-gradient quantisation point: the values, rounded to fp32, are
    quantised along `axis` (the token rows) in blocks of 32 rows from the
    segment's first row; a last partial block is padded with zeros, which
    leave its scale unchanged."""
    a = np.asarray(a, dtype=np.float64)
    assert axis == 0
    n = a.shape[0]
    pad = (-n) % MX_BLOCK
    if pad:
        a = np.concatenate([a, np.zeros((pad,) + a.shape[1:])], axis=0)
    return mx_point(a, 0)[:n]


def layer_backward(inp, dout=None, fwd=None, *, mx: bool | None = None, quantizer=None,
                   weight_grads: bool = True, mx_wgrad_minibatch: int | None = None):
    """Gradients of sum(out * dout) for the layer (fp64, routing frozen at the
    forward's selection).

    Returns dict: dx [T,H], dWg/dWu [E,H,I], dWd [E,I,H], dWr [H,E], dgate [T,k]
    (d/dw of the slot weights), and dWsg/dWsu/dWsd with a shared expert.
    The router bias is an input, not a parameter: it gets no gradient.

    MXFP8 (`mx`, default from the workload): the routed experts' two
    input-gradient GEMMs take MXFP8 operands, quantised along their contraction
    axis -- dY and Wd along H for dH = dY Wd^T, dG | dU and Wg | Wu along I for
    dX = dG Wg^T + dU Wu^T -- and the weight-gradient GEMMs take the unquantised
    operands (x rows, h = silu(g) u, dY, dG, dU).  The shared expert is bf16
    throughout.  `fwd` must then be the MXFP8 forward (its g, u, Y include the
    forward's quantisation).  `quantizer(a, axis)` replaces `mx_point`.
    weight_grads=False leaves out the expert weight gradients (dWg, dWu, dWd and
    the shared expert's); every other result is unchanged.
    mx_wgrad_minibatch (MXFP8 only): the routed experts' weight-gradient GEMMs
    take MXFP8 operands too, quantised along their contraction axis, the
    token rows: within each (minibatch of that many tokens, expert) segment,
    in blocks of 32 rows in token order (x rows, h, dY, dG, dU; zero padding
    past the segment's last row).  The shared expert stays bf16.
    """
    w_ = inp.w
    mx = (w_.prec == "mxfp8") if mx is None else mx
    if fwd is None:
        fwd = layer_forward(inp, keep=True, mx=mx)
    q = (quantizer or mx_point) if mx else None
    qw = mx_rows_point if (mx and mx_wgrad_minibatch) else None
    dout = as_f64(inp.dout if dout is None else dout)
    x64, idx, gw, Y = fwd["x"], fwd["idx"], fwd["w"], fwd["Y"]
    T, H = x64.shape
    assert dout.shape == (T, H), "the backward needs the forward of every token"
    E, k, I = w_.E, w_.k, w_.I
    # reverse combine: d out / d Y[t,j] = w[t,j] * dout[t]; d out / d w[t,j] = <dout[t], Y[t,j]>
    dgate = np.einsum("th,tjh->tj", dout, Y)
    dx = np.zeros((T, H), dtype=np.float64)
    if weight_grads:
        dWg = np.zeros((E, H, I)); dWu = np.zeros((E, H, I)); dWd = np.zeros((E, I, H))
    W = Weights(inp, mx=False)
    for e, (t_sel, j_sel, g, u, h) in fwd["saved"].items():
        Wg, Wu, Wd = W.expert_dgrad(e, q)
        dy = gw[t_sel, j_sel][:, None] * dout[t_sel]
        X = x64[t_sel]
        dh = (q(dy, 1) if q else dy) @ Wd.T
        du = dh * silu(g)
        dg = dh * u * silu_grad(g)
        if weight_grads:
            dWd[e] = segment_rows_product(t_sel, h, dy, mx_wgrad_minibatch, qw)
            dWg[e] = segment_rows_product(t_sel, X, dg, mx_wgrad_minibatch, qw)
            dWu[e] = segment_rows_product(t_sel, X, du, mx_wgrad_minibatch, qw)
        if q:
            dxe = q(dg, 1) @ Wg.T + q(du, 1) @ Wu.T
        else:
            dxe = dg @ Wg.T + du @ Wu.T
        np.add.at(dx, t_sel, dxe)
    # router: gate weights are the softmax of the selected logits
    dsel = gw * (dgate - (gw * dgate).sum(axis=1, keepdims=True))
    dlogits = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(dlogits, idx.astype(np.int64), dsel, axis=1)
    Wr64 = as_f64(inp.Wr)
    dx += dlogits @ Wr64.T
    dWr = x64.T @ dlogits
    res = {"dx": dx, "dWr": dWr, "dgate": dgate, "dlogits": dlogits}
    if weight_grads:
        res.update(dWg=dWg, dWu=dWu, dWd=dWd)
    if "shared" in fwd:
        gs, us, hs = fwd["shared"]
        Wsg, Wsu, Wsd = W.shared()
        dhs = dout @ Wsd.T
        dus = dhs * silu(gs)
        dgs = dhs * us * silu_grad(gs)
        if weight_grads:
            res["dWsd"] = hs.T @ dout
            res["dWsg"] = x64.T @ dgs
            res["dWsu"] = x64.T @ dus
        dx += dgs @ Wsg.T + dus @ Wsu.T
    return res


def weight_grad_columns(inp, e: int, cols, dout=None, *, mx: bool | None = None, routing=None,
                        mx_wgrad_minibatch: int | None = None):
    """Columns `cols` of one expert's weight gradients over all of its tokens:
    dWg[:, cols] and dWu[:, cols] [H, n], dWd[cols, :] [n, H] (e >= 0, routing
    frozen at the forward's selection), or the shared expert's dWsg, dWsu, dWsd
    under the same keys (e = -1, every token, bf16 throughout).

    Column i of the gate and up gradients and row i of the down gradient
    involve only column i of the expert's gate/up activations and of dH, so the
    products of `layer_backward` are taken here on those weight columns alone.
    Every MXFP8 block of a forward weight lies inside one column of Wg / Wu
    (blocks run along H) and every block of the backward's Wd inside one row
    (blocks run along H), so restricting to the columns commutes with the
    quantiser.  Same quantisation points as `layer_backward`: forward on the
    MXFP8 x rows and weights, dH from MXFP8 dY and Wd, weight gradients on the
    unquantised x, h and dY.
    routing: (idx, w) of every token, from `route`, to reuse across calls.
    mx_wgrad_minibatch: as in `layer_backward` (routed experts, MXFP8): the
    weight-gradient operands are quantised along the token rows per
    (minibatch, expert) segment; a block of 32 rows of one column lies inside
    that column, so restricting to the columns commutes with it too.
    """
    w_ = inp.w
    mx = (w_.prec == "mxfp8") if mx is None else mx
    cols = np.asarray(cols, dtype=np.int64)
    dout = inp.dout if dout is None else dout
    if e < 0:
        Wsg, Wsu, Wsd = (as_f64(t) for t in (inp.Wsg, inp.Wsu, inp.Wsd))
        X, dy = as_f64(inp.x), as_f64(dout)
        g, u = X @ Wsg[:, cols], X @ Wsu[:, cols]
        dh = dy @ Wsd[cols, :].T
    else:
        if routing is None:
            _, idx, gw = route(as_f32(inp.x), inp.Wr, inp.bias, w_.k)
        else:
            idx, gw = routing
        t_sel, j_sel = np.nonzero(idx == e)
        X = as_f64(inp.x[t_sel])  # rows picked before widening: same values, less memory
        dy = gw[t_sel, j_sel][:, None] * as_f64(dout[t_sel])
        Wg, Wu, Wd = (as_f64(t[e]) for t in (inp.Wg, inp.Wu, inp.Wd))
        Wg, Wu, Wd = Wg[:, cols], Wu[:, cols], Wd[cols, :]
        if mx:
            xin = mx_roundtrip(X, axis=1)
            g, u = xin @ mx_roundtrip(Wg, 0), xin @ mx_roundtrip(Wu, 0)
            dh = mx_point(dy, 1) @ mx_point(Wd, 1).T
        else:
            g, u = X @ Wg, X @ Wu
            dh = dy @ Wd.T
    h = silu(g) * u
    du = dh * silu(g)
    dg = dh * u * silu_grad(g)
    if e >= 0 and mx and mx_wgrad_minibatch:
        return {"dWg": segment_rows_product(t_sel, X, dg, mx_wgrad_minibatch, mx_rows_point),
                "dWu": segment_rows_product(t_sel, X, du, mx_wgrad_minibatch, mx_rows_point),
                "dWd": segment_rows_product(t_sel, h, dy, mx_wgrad_minibatch, mx_rows_point)}
    return {"dWg": X.T @ dg, "dWu": X.T @ du, "dWd": h.T @ dy}


def rel_inf_err(got, ref) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (the layer's max relative error)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))
