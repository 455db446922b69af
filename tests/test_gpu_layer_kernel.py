"""The persistent layer kernel (every forward expert GEMM and the combine in
one cooperative launch, combine workgroups and GEMM workgroups signalling
through device counters, a ring of minibatch slots) against the
one-launch-per-GEMM forward: outputs must agree bit for bit, for several
minibatches, ring sizes and numbers of combine workgroups, with and without
the saved outputs of a training forward, in bf16 and MXFP8; the device status
word must stay clear (no wait expired)."""
import pytest
import torch

import dispatch_grouped_gemm_moe_amd as moe
import oracle as O
from moe_inputs import Workload, make_inputs, KIMI_BF16, KIMI_FWD_BWD

pytestmark = pytest.mark.gpu


def _wl(name, **kw):
    return Workload(name, stream=5000 + (sum(map(ord, name)) % 997), **kw)


CASES = [
    # (workload, ring_slots, comm_cus, keep)
    (_wl("lk_one_mb", T=64, H=128, I=64, E=8, k=2, minibatch=64), 0, 0, True),
    (_wl("lk_many_mb", T=1500, H=256, I=128, E=8, k=2, minibatch=256, router_bias="normal"), 0, 0, False),
    (_wl("lk_many_mb_saved", T=1500, H=256, I=128, E=8, k=2, minibatch=256, router_bias="normal"), 0, 0, True),
    (_wl("lk_two_slots", T=1500, H=256, I=128, E=8, k=2, minibatch=192), 2, 0, False),
    (_wl("lk_comm16", T=1100, H=256, I=192, E=6, k=3, minibatch=128), 3, 16, False),
    (_wl("lk_comm8_two_slots", T=1100, H=256, I=192, E=6, k=3, minibatch=128), 2, 8, False),
    (_wl("lk_tiles_two_slots_saved", T=1500, H=256, I=128, E=8, k=2, minibatch=192), 2, 0, True),
    (_wl("lk_shared", T=700, H=384, I=192, E=6, k=2, minibatch=128, shared_expert=True), 0, 0, False),
    (_wl("lk_mx", T=900, H=512, I=256, E=4, k=2, minibatch=160, router_bias="zipf", prec="mxfp8"), 0, 0, False),
    (_wl("lk_mx_saved", T=900, H=512, I=256, E=4, k=2, minibatch=160, prec="mxfp8"), 3, 8, True),
    (_wl("lk_mx_tiles", T=900, H=512, I=256, E=4, k=2, minibatch=128, prec="mxfp8"), 0, 0, False),
    # minibatches grouped into phases (ring slots = 3 groups; ragged last group)
    (_wl("lk_group2", T=1500, H=256, I=128, E=8, k=2, minibatch=192, router_bias="normal"), 6, 0, False),
    (_wl("lk_group3_saved", T=1500, H=256, I=128, E=8, k=2, minibatch=160), 9, 0, True),
    (_wl("lk_group2_comm8", T=1500, H=256, I=128, E=8, k=2, minibatch=192), 6, 8, False),
    (_wl("lk_group_auto", T=2000, H=256, I=192, E=6, k=3, minibatch=256), 0, 0, False),
    (_wl("lk_mx_group2", T=1200, H=512, I=256, E=4, k=2, minibatch=128, prec="mxfp8"), 6, 0, False),
    # MXFP8 routed experts with the bf16 shared expert's tiles in the same launch
    (_wl("lk_mx_shared", T=700, H=384, I=192, E=6, k=2, minibatch=128, shared_expert=True, prec="mxfp8"), 0, 0, False),
    (_wl("lk_mx_shared_saved", T=700, H=384, I=192, E=6, k=2, minibatch=128, shared_expert=True, prec="mxfp8",
         router_bias="normal"), 3, 8, True),
    (_wl("lk_mx_shared_group", T=1200, H=512, I=256, E=4, k=2, minibatch=128, shared_expert=True, prec="mxfp8"),
     6, 0, True),
]


def _forward(inp, flags, ring_slots, comm_cus, keep):
    from gpu_harness import Layer
    layer = Layer(inp, flags=flags, ring_slots=ring_slots, comm_cus=comm_cus)
    out = layer.forward(keep=keep).clone()
    st, code, detail = layer.device_status()
    assert st == moe.MOE_OK and code == 0, ("device status", code, detail)
    return out


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].name)
def test_layer_kernel_matches_per_gemm_launches(gpu_lib, case):
    w, ring_slots, comm_cus, keep = case
    inp = make_inputs(w)
    print(w.name, flush=True)
    a = _forward(inp, 0, ring_slots, comm_cus, keep)
    b = _forward(inp, moe.MOE_F_LAUNCH_PER_GEMM, ring_slots, comm_cus, keep)
    assert torch.equal(a, b)
    if w.name == "lk_many_mb":
        err = O.rel_inf_err(a.float().cpu().numpy(), O.layer_forward(inp, mx=False)["out"])
        assert err <= 1e-2, err


@pytest.mark.parametrize("w", [KIMI_BF16, KIMI_FWD_BWD], ids=lambda w: w.name)
def test_layer_kernel_full_size_matches_per_gemm_launches(gpu_lib, w):
    inp = make_inputs(w)
    print(w.name, flush=True)
    a = _forward(inp, 0, 0, 0, w.backward)
    b = _forward(inp, moe.MOE_F_LAUNCH_PER_GEMM, 0, 0, w.backward)
    assert torch.equal(a, b)
