"""The persistent layer kernel (every forward expert GEMM and the combine in
one cooperative launch, combine workgroups and GEMM workgroups signalling
through device counters, a ring of minibatch slots reused as soon as combine
has drained them) against the one-launch-per-GEMM forward and the oracle.

Every case checks which path ran, that the two paths agree bit for bit, that
the output is within the stated tolerance of the CPU oracle (1e-2 bf16, 5e-2
MXFP8 against the quantisation-aware oracle), and that the device status word
stays clear (no wait expired).  Cases span several minibatches, rings smaller
than the minibatch count (slot reuse), dedicated combine workgroups, grouped
phases, the saved outputs of a training forward, bf16 and MXFP8, and the
shared expert.  A forced dropped signal must end in the bounded wait's
timeout report, with the next forward on the same workspace clean.
"""
import zlib

import pytest
import torch

import dispatch_grouped_gemm_moe_amd as moe
import oracle as O
from moe_inputs import Workload, make_inputs, KIMI_FWD_BWD

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "mxfp8": 5e-2}


def _wl(name, **kw):
    return Workload(name, stream=5000 + zlib.crc32(name.encode()) % 997, **kw)


LK = "layer kernel"
CASES = [
    # (workload, ring_slots, comm_cus, keep, path the default flags take)
    (_wl("lk_one_mb", T=64, H=128, I=64, E=8, k=2, minibatch=64), 0, 0, True, LK),
    (_wl("lk_many_mb", T=1500, H=256, I=128, E=8, k=2, minibatch=256, router_bias="normal"), 0, 0, False, LK),
    (_wl("lk_many_mb_saved", T=1500, H=256, I=128, E=8, k=2, minibatch=256, router_bias="normal"), 0, 0, True, LK),
    # combine tiles with Y in the ring need three slots: two slots and nothing
    # saved take the one-launch-per-GEMM forward
    (_wl("lk_two_slots_fallback", T=1500, H=256, I=128, E=8, k=2, minibatch=192), 2, 0, False, "per-GEMM"),
    # ring reuse: one minibatch per slot, 3 slots for 8 minibatches
    (_wl("lk_three_slots", T=1500, H=256, I=128, E=8, k=2, minibatch=192, router_bias="normal"), 3, 0, False, LK),
    (_wl("lk_comm16", T=1100, H=256, I=192, E=6, k=3, minibatch=128), 3, 16, False, LK),
    (_wl("lk_comm8_two_slots", T=1100, H=256, I=192, E=6, k=3, minibatch=128), 2, 8, False, LK),
    (_wl("lk_tiles_two_slots_saved", T=1500, H=256, I=128, E=8, k=2, minibatch=192), 2, 0, True, LK),
    (_wl("lk_shared", T=700, H=384, I=192, E=6, k=2, minibatch=128, shared_expert=True), 0, 0, False, LK),
    (_wl("lk_mx", T=900, H=512, I=256, E=4, k=2, minibatch=160, router_bias="zipf", prec="mxfp8"), 0, 0, False, LK),
    (_wl("lk_mx_saved", T=900, H=512, I=256, E=4, k=2, minibatch=160, prec="mxfp8"), 3, 8, True, LK),
    (_wl("lk_mx_tiles", T=900, H=512, I=256, E=4, k=2, minibatch=128, prec="mxfp8"), 0, 0, False, LK),
    (_wl("lk_mx_three_slots", T=1200, H=512, I=256, E=4, k=2, minibatch=128, prec="mxfp8"), 3, 0, False, LK),
    # four one-minibatch slot groups with Y in the ring: down(s-1) runs before
    # combine(s-2), and gate|up waits for the combine four groups back
    (_wl("lk_four_slots", T=1500, H=256, I=128, E=8, k=2, minibatch=192, router_bias="normal"), 4, 0, False, LK),
    (_wl("lk_mx_four_slots", T=1200, H=512, I=256, E=4, k=2, minibatch=128, prec="mxfp8"), 4, 0, False, LK),
    # minibatches grouped into phases (ring slots = 3 groups; ragged last group)
    (_wl("lk_group2", T=1500, H=256, I=128, E=8, k=2, minibatch=192, router_bias="normal"), 6, 0, False, LK),
    (_wl("lk_group3_saved", T=1500, H=256, I=128, E=8, k=2, minibatch=160), 9, 0, True, LK),
    (_wl("lk_group2_comm8", T=1500, H=256, I=128, E=8, k=2, minibatch=192), 6, 8, False, LK),
    (_wl("lk_group_auto", T=2000, H=256, I=192, E=6, k=3, minibatch=256), 0, 0, False, LK),
    (_wl("lk_mx_group2", T=1200, H=512, I=256, E=4, k=2, minibatch=128, prec="mxfp8"), 6, 0, False, LK),
    # MXFP8 routed experts with the bf16 shared expert's tiles in the same launch
    (_wl("lk_mx_shared", T=700, H=384, I=192, E=6, k=2, minibatch=128, shared_expert=True, prec="mxfp8"), 0, 0,
     False, LK),
    (_wl("lk_mx_shared_saved", T=700, H=384, I=192, E=6, k=2, minibatch=128, shared_expert=True, prec="mxfp8",
         router_bias="normal"), 3, 8, True, LK),
    (_wl("lk_mx_shared_group", T=1200, H=512, I=256, E=4, k=2, minibatch=128, shared_expert=True, prec="mxfp8"),
     6, 0, True, LK),
]


def _forward(inp, flags, ring_slots, comm_cus, keep):
    from gpu_harness import Layer
    layer = Layer(inp, flags=flags, ring_slots=ring_slots, comm_cus=comm_cus)
    path = layer.forward_path(keep=keep)
    out = layer.out.clone()
    st, code, detail = layer.device_status()
    assert st == moe.MOE_OK and code == 0, ("device status", code, detail)
    sizes = layer.bufs.sizes
    return out, path, sizes


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].name)
def test_layer_kernel_matches_per_gemm_launches_and_oracle(gpu_lib, case):
    w, ring_slots, comm_cus, keep, want_path = case
    inp = make_inputs(w)
    print(w.name, flush=True)
    a, path, sizes = _forward(inp, 0, ring_slots, comm_cus, keep)
    assert path == want_path
    b, path_b, _ = _forward(inp, moe.MOE_F_LAUNCH_PER_GEMM, ring_slots, comm_cus, keep)
    assert path_b == "per-GEMM"
    assert torch.equal(a, b)
    err = O.rel_inf_err(a.float().cpu().numpy(), O.layer_forward(inp)["out"])
    print("%s: %s, %d minibatches, ring %d, comm %d: max rel err %.3e"
          % (w.name, path, sizes.num_minibatches, sizes.ring_slots, sizes.comm_cus, err))
    assert err <= TOL[w.prec]


def test_layer_kernel_full_size_mx_shared_matches_per_gemm_launches(gpu_lib):
    """MXFP8 routed experts with the bf16 shared expert at full size, training
    forward (the backward benchmark's launch); the oracle side of this workload
    is checked through the full-size backward tests."""
    w = KIMI_FWD_BWD
    inp = make_inputs(w)
    print(w.name, flush=True)
    a, path, _ = _forward(inp, 0, 0, 0, True)
    assert path == LK
    b, _, _ = _forward(inp, moe.MOE_F_LAUNCH_PER_GEMM, 0, 0, True)
    assert torch.equal(a, b)


def test_dropped_signal_expires_the_bounded_wait_then_next_forward_is_clean(gpu_lib):
    """MOE_F_DEBUG_DROP_SIGNAL: GEMM workgroup 0 never signals the end of the
    first gate|up phase, so every wait on it (the down tiles of minibatch
    group 0: wait site 3) runs into its 2 s bound; the launch drains and the
    device status word reports the timeout.  Reading the status clears it, and
    a normal forward on the same workspace and stream then matches the oracle
    with a clear status."""
    from gpu_harness import Layer
    w = _wl("lk_watchdog", T=1500, H=256, I=128, E=8, k=2, minibatch=256, router_bias="normal")
    inp = make_inputs(w)
    layer = Layer(inp, flags=moe.MOE_F_DEBUG_DROP_SIGNAL)
    print("%s: forward with a dropped signal (waits expire after 2 s)" % w.name, flush=True)
    assert layer.forward_path(keep=False) == LK
    st, code, detail = layer.device_status()
    assert (st, code, detail) == (moe.MOE_E_DEVICE, moe.MOE_DEV_WAIT_TIMEOUT, 3)
    assert layer.device_status() == (moe.MOE_OK, 0, 0)
    layer.cfg.flags &= ~moe.MOE_F_DEBUG_DROP_SIGNAL
    assert layer.forward_path(keep=False) == LK
    assert layer.device_status() == (moe.MOE_OK, 0, 0)
    err = O.rel_inf_err(layer.out.float().cpu().numpy(), O.layer_forward(inp)["out"])
    assert err <= TOL["bf16"], err
