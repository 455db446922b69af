"""GPU parity of the MXFP8 layer forward.

The dispatch-side quantiser must produce the oracle's E4M3 codes and E8M0
scales bit for bit.  The layer output is compared with the quantisation-aware
oracle (the same quantisation points, fp64 elsewhere) within max relative
error 5e-2; the error against the unquantised oracle is printed as context.
"""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu

MX_TOL = 5e-2


def _wl(name, **kw):
    return Workload(name, stream=6000 + (sum(map(ord, name)) % 997), prec="mxfp8", **kw)


def test_mx_quantiser_is_bit_exact(gpu_lib):
    moe = gpu_lib
    g = torch.Generator().manual_seed(5)
    rows = [torch.randn(300, 512, generator=g),
            torch.randn(40, 512, generator=g) * 1e-20,
            torch.randn(40, 512, generator=g) * 1e20,
            torch.zeros(4, 512)]
    a = torch.cat(rows).to(torch.bfloat16)
    a[2, 7] = -0.0
    a[5, :32] = 448.0 / 8  # block maximum exactly at a scale boundary
    src = a.cuda()
    codes = torch.empty(a.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(a.shape[0], a.shape[1] // 32, dtype=torch.uint8, device="cuda")
    moe.moe_mx_quantize(src, codes, scales)
    torch.cuda.synchronize()
    rc, rs = O.mx_quantize(a, axis=1)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


MX_CASES = [
    _wl("mx_tiny", T=64, H=128, I=64, E=8, k=2, minibatch=64),
    _wl("mx_tiles", T=900, H=512, I=256, E=4, k=2, minibatch=400, router_bias="zipf"),
    _wl("mx_shared", T=300, H=384, I=192, E=6, k=2, minibatch=128, shared_expert=True),
    # one 64-deep K step per GEMM: every ring stage is a half stage
    _wl("mx_k64", T=200, H=64, I=64, E=4, k=2, minibatch=128, shared_expert=True),
]


@pytest.mark.parametrize("w", MX_CASES, ids=lambda w: w.name)
def test_mx_forward_matches_quantisation_aware_oracle(gpu_lib, w):
    from gpu_harness import Layer
    inp = make_inputs(w)
    layer = Layer(inp)
    out = layer.forward().float().cpu().numpy()
    idx, _ = layer.saved_routing()
    ref = O.layer_forward(inp, mx=True)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    err = O.rel_inf_err(out, ref["out"])
    plain = O.rel_inf_err(out, O.layer_forward(inp, mx=False)["out"])
    print("%s: max rel err %.3e vs quantisation-aware oracle, %.3e vs unquantised" % (w.name, err, plain))
    assert err <= MX_TOL


def test_mx_forward_bitwise_repeatable_and_minibatch_invariant(gpu_lib):
    from gpu_harness import Layer
    w = _wl("mx_det", T=1000, H=512, I=256, E=8, k=2, minibatch=512)
    inp = make_inputs(w)
    a = Layer(inp, minibatch=512)
    o1 = a.forward().clone()
    o2 = a.forward().clone()
    o3 = Layer(inp, minibatch=256).forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


@pytest.mark.parametrize("T,H,scale", [(300, 7168, 1.0), (77, 192, 1e-3), (33, 448, 1e4)])
def test_dispatch_quantisation_in_the_router_is_bit_exact(gpu_lib, T, H, scale):
    """The router's fused MXFP8 quantisation of x (what the MXFP8 forward's
    gate|up GEMM reads) against the oracle's quantiser: codes and E8M0 scales
    bit for bit, including an odd number of 64-wide chunks per row (H = 192,
    448), tiny and large magnitudes, an all-zero row and signed zeros."""
    moe = gpu_lib
    g = torch.Generator().manual_seed(T + H)
    x = (torch.randn(T, H, generator=g) * scale).to(torch.bfloat16)
    x[1] = 0.0
    x[2, 5] = -0.0
    x[3, :32] = 448.0 * scale  # a block maximum exactly at a scale boundary
    E, k = 8, 2
    Wr = torch.randn(H, E, generator=g) * 0.02
    cfg = moe.make_cfg(T, H, 64, E, k)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gw = torch.empty(T, k, dtype=torch.float32, device="cuda")
    ng = (H + 127) // 128
    codes = torch.full((T, H), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((ng, T, 4), 0x5A, dtype=torch.uint8, device="cuda")
    moe.moe_route(cfg, x.cuda(), Wr.cuda(), None, idx, gw, x_codes=codes, x_scales=scales)
    torch.cuda.synchronize()
    rc, rs = O.mx_quantize(x, axis=1)  # [T, H], [T, H/32]
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    # operand layout -> [T, H/32]: byte b of dword (g, t) is block 4g + b; bytes past the row's end are zero
    sc = scales.cpu().numpy().transpose(1, 0, 2).reshape(T, ng * 4)
    np.testing.assert_array_equal(sc[:, :H // 32], rs)
    assert not sc[:, H // 32:].any()
    _, ref_idx, _ = O.route(x, Wr, None, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
