"""Full-size forward parity at H=7168, I=2048, E=32, k=8 and 16384 tokens,
through the C ABI, against the CPU oracle on a token sample that holds a
checked row in every 128-row block of every (minibatch, expert) segment of the
layouts being run (and each segment's first and last row): every M tile of
every grouped GEMM launch, and every N tile of it through the whole output
rows.

bf16, minibatches of 2560 (a ragged last one): the default launch, then the
ring token buffer made smaller than the minibatch count (slots reused as soon
as combine has drained them), the CU split with dedicated combine workgroups,
and the one-launch-per-GEMM forward; each must be bitwise equal to the
default output and within max relative error 1e-2 of the oracle.

MXFP8 with the Zipf-skewed router, over the minibatch sizes 512, 1024, 2560
and 4096: bitwise equal across sizes (every output row is computed by the same
per-row arithmetic) and within 5e-2 of the quantisation-aware oracle on the
union of the four sizes' covering samples.
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import dispatch_grouped_gemm_moe_amd as moe
import oracle as O
from moe_inputs import KIMI_BF16, KIMI_MXFP8, make_inputs
from sampling import covering_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

BF16_TOL, MX_TOL = 1e-2, 5e-2
MX_SWEEP = (2560, 512, 1024, 4096)


def _host(t):
    return t.float().cpu().numpy()


@pytest.fixture(scope="module")
def bf16_full(gpu_lib):
    w = KIMI_BF16
    inp = make_inputs(w)
    _, idx, _ = O.route(inp.x, inp.Wr, inp.bias, w.k)
    S = covering_tokens(idx, w.minibatch)
    print("%s: oracle on %d covering tokens" % (w.name, len(S)), flush=True)
    ref = O.layer_forward(inp, tokens=S)
    yield SimpleNamespace(w=w, inp=inp, idx=idx, S=S, ref=ref, default=None)
    torch.cuda.empty_cache()


def _run(inp, flags=0, ring_slots=0, comm_cus=0, keep=False, minibatch=None):
    from gpu_harness import Layer
    layer = Layer(inp, flags=flags, ring_slots=ring_slots, comm_cus=comm_cus, minibatch=minibatch)
    path = layer.forward_path(keep=keep)
    out = layer.out.clone()
    st, code, detail = layer.device_status()
    assert st == moe.MOE_OK and code == 0, ("device status", code, detail)
    idx, _ = layer.saved_routing() if keep else (None, None)
    sizes = layer.bufs.sizes
    del layer
    torch.cuda.empty_cache()
    return out, path, sizes, idx


def test_bf16_full_size_default_launch(bf16_full):
    f = bf16_full
    out, path, sizes, idx = _run(f.inp, keep=True)
    assert path == "layer kernel"
    np.testing.assert_array_equal(idx.cpu().numpy(), f.idx)
    err = O.rel_inf_err(_host(out)[f.S], f.ref["out"])
    print("%s: default (ring %d slots for %d minibatches): max rel err %.3e on %d tokens"
          % (f.w.name, sizes.ring_slots, sizes.num_minibatches, err, len(f.S)))
    assert err <= BF16_TOL
    f.default = out


@pytest.mark.parametrize("ring_slots,comm_cus,keep,flags", [
    (3, 0, False, 0),   # one minibatch per phase, 3 slots for 7 minibatches
    (6, 0, False, 0),   # two minibatches per phase, 3 slot groups for 4 groups
    (3, 0, True, 0),    # training forward: h in the ring, Y saved
    (0, 8, False, 0),   # 8 dedicated combine workgroups
    (0, 16, False, 0),  # 16 dedicated combine workgroups
    (2, 16, False, 0),  # combine workgroups and 2 slots for 7 minibatches
    (0, 0, False, moe.MOE_F_LAUNCH_PER_GEMM),
], ids=["ring3", "ring6", "ring3_saved", "comm8", "comm16", "ring2_comm16", "per_gemm"])
def test_bf16_full_size_ring_reuse_and_cu_split(bf16_full, ring_slots, comm_cus, keep, flags):
    f = bf16_full
    if f.default is None:
        pytest.skip("needs the default launch's output")
    out, path, sizes, _ = _run(f.inp, flags=flags, ring_slots=ring_slots, comm_cus=comm_cus, keep=keep)
    assert path == ("per-GEMM" if flags else "layer kernel")
    if not flags:
        assert sizes.comm_cus == comm_cus
        if ring_slots:
            assert sizes.ring_slots == ring_slots < sizes.num_minibatches
    err = O.rel_inf_err(_host(out)[f.S], f.ref["out"])
    print("ring %d comm %d keep %s flags %d: max rel err %.3e" % (sizes.ring_slots, sizes.comm_cus, keep, flags, err))
    assert err <= BF16_TOL
    assert torch.equal(out.view(torch.int16), f.default.view(torch.int16))


@pytest.fixture(scope="module")
def mx_full(gpu_lib):
    w = KIMI_MXFP8
    inp = make_inputs(w)
    _, idx, _ = O.route(inp.x, inp.Wr, inp.bias, w.k)
    S = np.unique(np.concatenate([covering_tokens(idx, mb) for mb in MX_SWEEP]))
    print("%s: quantisation-aware oracle on %d tokens" % (w.name, len(S)), flush=True)
    ref = O.layer_forward(inp, tokens=S, mx=True)
    yield SimpleNamespace(w=w, inp=inp, idx=idx, S=S, ref=ref, outs={})
    torch.cuda.empty_cache()


def test_mx_full_size_routing_is_bit_exact(mx_full):
    f = mx_full
    w = f.w
    cfg = moe.make_cfg(w.T, w.H, w.I, w.E, w.k)
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device="cuda")
    gw = torch.empty(w.T, w.k, dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, f.inp.x.cuda(), f.inp.Wr.cuda(), f.inp.bias.cuda(), idx, gw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), f.idx)


@pytest.mark.parametrize("minibatch", MX_SWEEP)
def test_mx_full_size_minibatch_sweep(mx_full, minibatch):
    """The inference forward (nothing saved), as the benchmark runs it."""
    f = mx_full
    out, path, sizes, _ = _run(f.inp, keep=False, minibatch=minibatch)
    assert path == "layer kernel" and sizes.minibatch == minibatch
    err = O.rel_inf_err(_host(out)[f.S], f.ref["out"])
    print("%s minibatch %d (%d minibatches, ring %d): max rel err %.3e on %d tokens"
          % (f.w.name, minibatch, sizes.num_minibatches, sizes.ring_slots, err, len(f.S)))
    assert err <= MX_TOL
    f.outs[minibatch] = out
    first = f.outs[MX_SWEEP[0]] if MX_SWEEP[0] in f.outs else None
    if first is not None:
        assert torch.equal(out.view(torch.int16), first.view(torch.int16))
