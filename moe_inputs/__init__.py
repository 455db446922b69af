"""Seeded synthetic inputs for the fused MoE layer workloads.

This module holds workload shapes and random draws only.  It contains none of
the layer's arithmetic (no routing, no dispatch, no FFN, no quantisation), so
both the CPU oracle and the GPU path may use it without sharing any of the
method.

Every tensor is drawn on the CPU from its own torch generator, seeded from a
master seed and a per-(workload, tensor) stream id, then scaled and rounded
(bf16 tensors use round-to-nearest-even through torch's cast).  The layer
itself (Cursor's "Mixture-of-Kittens" write-ups, section 02) names only the
shape hidden 7168 / expert intermediate 2048; the remaining sizes, the weight
and input distributions and the load skews are the synthetic stand-ins stated
in each workload below.
"""
from __future__ import annotations

import dataclasses
import math

import torch

MASTER_SEED = 20261202

# tensor ids inside a workload's stream space
_X, _WR, _BIAS, _WG, _WU, _WD, _WSG, _WSU, _WSD, _DOUT, _PERM, _WIDE = range(1, 13)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one synthetic MoE layer workload."""

    name: str
    T: int  # tokens
    H: int  # hidden size
    I: int  # expert intermediate size
    E: int  # experts on this GPU
    k: int  # experts per token
    minibatch: int = 0  # tokens per ring slot, 0 = automatic
    router_bias: str = "none"  # "none" | "normal" | "zipf"
    shared_expert: bool = False
    prec: str = "bf16"  # "bf16" | "mxfp8"
    backward: bool = False
    stream: int = 0  # stream-id base for this workload's tensors
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    zipf_s: float = 1.1
    # scale every row and column of x, dout and the expert weights by its own
    # power of two in 2^-3 .. 2^3 (exact in bf16), so 32-element blocks mix
    # magnitudes along one axis only
    wide_range: bool = False

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the measured layer, plus smaller parity shapes.
TINY = Workload("tiny", T=64, H=128, I=64, E=8, k=2, minibatch=64, stream=100)
SMALL = Workload("small", T=4096, H=2048, I=1024, E=64, k=6, stream=200)
KIMI_BF16 = Workload("h7168_i2048_e32_k8_bf16", T=16384, H=7168, I=2048, E=32, k=8,
                     minibatch=2560, router_bias="normal", stream=300)
KIMI_MXFP8 = Workload("h7168_i2048_e32_k8_mxfp8_zipf", T=16384, H=7168, I=2048, E=32, k=8,
                      minibatch=2560, router_bias="zipf", prec="mxfp8", stream=400)
KIMI_FWD_BWD = Workload("h7168_i2048_e32_k8_mxfp8_shared_fwdbwd", T=16384, H=7168, I=2048,
                        E=32, k=8, minibatch=2560, router_bias="normal", prec="mxfp8",
                        shared_expert=True, backward=True, stream=500)

WORKLOADS = {w.name: w for w in (TINY, SMALL, KIMI_BF16, KIMI_MXFP8, KIMI_FWD_BWD)}


def _gen(w: Workload, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(MASTER_SEED * 4096 + w.stream * 16 + tensor_id)
    return g


def _normal(w: Workload, tensor_id: int, shape, sigma: float, chunk_dim0: bool = False):
    """N(0, sigma^2) draws in fp32 on the CPU."""
    g = _gen(w, tensor_id)
    if not chunk_dim0:
        return torch.randn(shape, generator=g, dtype=torch.float32) * sigma
    out = torch.empty(shape, dtype=torch.bfloat16)
    for i in range(shape[0]):  # bounds peak memory for multi-GB weight stacks
        out[i] = (torch.randn(shape[1:], generator=g, dtype=torch.float32) * sigma).to(torch.bfloat16)
    return out


def zipf_shares(E: int, s: float) -> list[float]:
    """p_r = r^-s / sum_q q^-s for ranks r = 1..E (a distribution, not layer math)."""
    z = sum(q ** -s for q in range(1, E + 1))
    return [(r ** -s) / z for r in range(1, E + 1)]


@dataclasses.dataclass
class LayerInputs:
    """CPU tensors of one workload.  bf16 tensors are the layer's exact values."""

    w: Workload
    x: torch.Tensor  # [T, H] bf16
    Wr: torch.Tensor  # [H, E] fp32 router weight
    bias: torch.Tensor | None  # [E] fp32 router logit bias or None
    Wg: torch.Tensor  # [E, H, I] bf16 gate projection
    Wu: torch.Tensor  # [E, H, I] bf16 up projection
    Wd: torch.Tensor  # [E, I, H] bf16 down projection
    Wsg: torch.Tensor | None = None  # [H, I] bf16 shared-expert gate
    Wsu: torch.Tensor | None = None  # [H, I] bf16 shared-expert up
    Wsd: torch.Tensor | None = None  # [I, H] bf16 shared-expert down
    dout: torch.Tensor | None = None  # [T, H] bf16 upstream gradient


def make_inputs(w: Workload, with_dout: bool | None = None) -> LayerInputs:
    """Draw every input tensor of workload `w` (deterministic in the seed)."""
    T, H, I, E = w.T, w.H, w.I, w.E
    big = E * H * I > (1 << 26)
    x = _normal(w, _X, (T, H), w.x_sigma).to(torch.bfloat16)
    Wr = _normal(w, _WR, (H, E), w.w_sigma)
    bias = None
    if w.router_bias == "normal":
        bias = _normal(w, _BIAS, (E,), 1.0)
    elif w.router_bias == "zipf":
        # Expert e gets the log-share of Zipf rank perm[e]+1 as a logit bias,
        # so selection frequency falls off with the rank.
        perm = torch.randperm(E, generator=_gen(w, _PERM))
        p = zipf_shares(E, w.zipf_s)
        bias = torch.tensor([math.log(p[int(perm[e])]) for e in range(E)], dtype=torch.float32)
    Wg = _normal(w, _WG, (E, H, I), w.w_sigma, chunk_dim0=big)
    Wu = _normal(w, _WU, (E, H, I), w.w_sigma, chunk_dim0=big)
    Wd = _normal(w, _WD, (E, I, H), w.w_sigma, chunk_dim0=big)
    if not big:
        Wg, Wu, Wd = (t.to(torch.bfloat16) for t in (Wg, Wu, Wd))
    li = LayerInputs(w, x, Wr, bias, Wg, Wu, Wd)
    if w.shared_expert:
        li.Wsg = _normal(w, _WSG, (H, I), w.w_sigma).to(torch.bfloat16)
        li.Wsu = _normal(w, _WSU, (H, I), w.w_sigma).to(torch.bfloat16)
        li.Wsd = _normal(w, _WSD, (I, H), w.w_sigma).to(torch.bfloat16)
    if with_dout if with_dout is not None else w.backward:
        li.dout = _normal(w, _DOUT, (T, H), 1.0).to(torch.bfloat16)
    if w.wide_range:
        g = _gen(w, _WIDE)

        def scale(t, *axes):
            f = torch.ones(t.shape, dtype=torch.float64)
            for ax in axes:
                shp = [1] * t.dim()
                shp[ax] = t.shape[ax]
                f = f * torch.pow(2.0, torch.randint(-3, 4, shp, generator=g).double())
            return (t.double() * f).to(t.dtype)

        li.x = scale(li.x, 0, 1)
        li.Wg, li.Wu, li.Wd = scale(li.Wg, 1, 2), scale(li.Wu, 1, 2), scale(li.Wd, 1, 2)
        if li.dout is not None:
            li.dout = scale(li.dout, 0, 1)
    return li
