"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Routing indices, logits and the dispatch layout must match bit for bit; the
layer output must be within max relative error 1e-2 (bf16) of the fp64
oracle; the identity-expert combine must return the input bitwise; repeated
runs and different minibatch sizes must give bitwise-identical outputs.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import Workload, make_inputs, TINY, SMALL

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2


def _wl(name, **kw):
    # a stable digest of the name (Python's str hash is salted per process)
    return Workload(name, stream=7000 + zlib.crc32(name.encode()) % 997, **kw)


def _np(t):
    return t.detach().cpu().numpy()


# ---------------------------------------------------------------- route

@pytest.mark.parametrize("w", [
    TINY,
    _wl("route_h7168", T=300, H=7168, I=64, E=32, k=8, router_bias="normal"),
    _wl("route_e256", T=130, H=256, I=64, E=256, k=16),
    _wl("route_e5", T=77, H=192, I=64, E=5, k=5),
])
def test_route_is_bit_exact(gpu_lib, w):
    moe = gpu_lib
    inp = make_inputs(w)
    cfg = moe.make_cfg(w.T, w.H, w.I, w.E, w.k)
    x, Wr = inp.x.cuda(), inp.Wr.cuda()
    bias = inp.bias.cuda() if inp.bias is not None else None
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device="cuda")
    gw = torch.empty(w.T, w.k, dtype=torch.float32, device="cuda")
    logits = torch.empty(w.T, w.E, dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, x, Wr, bias, idx, gw, logits)
    torch.cuda.synchronize()
    ref_logits, ref_idx, ref_w = O.route(inp.x, inp.Wr, inp.bias, w.k)
    np.testing.assert_array_equal(_np(logits).view(np.uint32), ref_logits.view(np.uint32))
    np.testing.assert_array_equal(_np(idx), ref_idx)
    np.testing.assert_allclose(_np(gw), ref_w, rtol=2e-6, atol=1e-7)


# ---------------------------------------------------------------- layout

def _random_idx(T, E, k, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    p = np.exp(-skew * np.arange(E)); p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k,skew", [(64, 8, 2, 0.0), (16384, 32, 8, 0.1), (3001, 256, 16, 0.02),
                                         (1, 4, 4, 0.0), (1000, 64, 6, 0.5)])
def test_dispatch_layout_is_bit_exact(gpu_lib, T, E, k, skew):
    moe = gpu_lib
    idx = _random_idx(T, E, k, seed=T + E, skew=skew)
    cfg = moe.make_cfg(T, 64, 64, E, k)
    d = lambda n: torch.full((n,), -7, dtype=torch.int32, device="cuda")
    counts, offsets, row_token, tok_row = d(E), d(E + 1), d(T * k), d(T * k)
    moe.moe_dispatch_layout(cfg, torch.from_numpy(idx).cuda(), counts, offsets, row_token, tok_row)
    torch.cuda.synchronize()
    rc, ro, rr, rt = O.dispatch_layout(idx, E)
    np.testing.assert_array_equal(_np(counts), rc)
    np.testing.assert_array_equal(_np(offsets), ro)
    np.testing.assert_array_equal(_np(row_token), rr)
    np.testing.assert_array_equal(_np(tok_row).reshape(T, k), rt)


def test_dispatch_layout_flags_bad_indices(gpu_lib):
    moe = gpu_lib
    for bad in ([[0, 9]], [[3, 3]]):  # out of range; repeated within a token
        idx = torch.tensor([[0, 1], [2, 3]] + bad, dtype=torch.int32, device="cuda")
        cfg = moe.make_cfg(3, 64, 64, 8, 2)
        offsets = torch.zeros(9, dtype=torch.int32, device="cuda")
        z = lambda n: torch.zeros(n, dtype=torch.int32, device="cuda")
        moe.moe_dispatch_layout(cfg, idx, z(8), offsets, z(6), z(6))
        torch.cuda.synchronize()
        assert int(offsets[8]) == -1


# ---------------------------------------------------------------- forward

FWD_CASES = [
    TINY,
    # several M, N and K tiles per GEMM, three minibatches with a ragged last one
    _wl("fwd_tiles", T=1200, H=512, I=256, E=4, k=2, minibatch=500),
    # many experts with few rows, one expert likely empty, bias skew
    _wl("fwd_skew", T=333, H=256, I=128, E=16, k=3, minibatch=0, router_bias="normal"),
    _wl("fwd_shared", T=200, H=384, I=192, E=6, k=2, minibatch=128, shared_expert=True),
    _wl("fwd_k1", T=96, H=128, I=64, E=3, k=1),
    _wl("fwd_k64", T=200, H=64, I=64, E=4, k=2, minibatch=128, shared_expert=True),  # one K stage per GEMM
    _wl("fwd_e256", T=300, H=128, I=64, E=256, k=16, minibatch=150, shared_expert=True),  # top-16 of 256
]


@pytest.mark.parametrize("w", FWD_CASES, ids=lambda w: w.name)
def test_forward_matches_oracle(gpu_lib, w):
    from gpu_harness import Layer
    inp = make_inputs(w)
    layer = Layer(inp)
    out = layer.forward().float().cpu().numpy()
    idx, gw = layer.saved_routing()
    ref = O.layer_forward(inp)
    np.testing.assert_array_equal(_np(idx), ref["idx"])
    np.testing.assert_allclose(_np(gw), ref["w"], rtol=2e-6, atol=1e-7)
    err = O.rel_inf_err(out, ref["out"])
    print("%s: max rel err %.3e" % (w.name, err))
    assert err <= BF16_TOL


def test_identity_experts_return_input_bitwise(gpu_lib):
    moe = gpu_lib
    from gpu_harness import Layer
    w = _wl("identity", T=700, H=256, I=64, E=8, k=4, minibatch=256)
    inp = make_inputs(w)
    layer = Layer(inp, flags=moe.MOE_F_IDENTITY_EXPERTS)
    out = layer.forward()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), layer.x.view(torch.int16))


def test_forward_bitwise_repeatable_and_minibatch_invariant(gpu_lib):
    from gpu_harness import Layer
    w = _wl("determinism", T=1000, H=512, I=256, E=8, k=2, minibatch=512, router_bias="normal")
    inp = make_inputs(w)
    a = Layer(inp, minibatch=512)
    o1 = a.forward().clone()
    o2 = a.forward().clone()
    b = Layer(inp, minibatch=128)
    o3 = b.forward().clone()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_forward_small_config_covering_sample(gpu_lib):
    """Config 2 (T=4096, H=2048, I=1024, E=64, k=6, automatic minibatch): the
    oracle on tokens that put a checked row in every 128-row block of every
    (minibatch, expert) segment; routing of every token bit-exact."""
    from gpu_harness import Layer
    from sampling import covering_tokens
    w = SMALL
    inp = make_inputs(w)
    layer = Layer(inp)
    assert layer.forward_path() == "layer kernel"
    out = layer.out.float().cpu().numpy()
    idx, _ = layer.saved_routing()
    _, ref_idx, _ = O.route(inp.x, inp.Wr, inp.bias, w.k)
    np.testing.assert_array_equal(_np(idx), ref_idx)
    sample = covering_tokens(ref_idx, layer.bufs.sizes.minibatch)
    ref = O.layer_forward(inp, tokens=sample)["out"]
    err = O.rel_inf_err(out[sample], ref)
    print("%s (minibatch %d): max rel err on %d covering tokens %.3e"
          % (w.name, layer.bufs.sizes.minibatch, len(sample), err))
    assert err <= BF16_TOL
