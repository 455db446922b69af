"""The allocation-free forward (moe_layer_fwd_static: the workspace is the
library's static device array) against moe_layer_fwd on a caller workspace,
through the C ABI: bitwise-equal outputs on two calls in a row, the second
with fewer tokens; MXFP8 as well; a stale device status word cleared at the
start of the next call; oversized configurations rejected before any device
call."""
import pytest
import torch

import dispatch_grouped_gemm_moe_amd as moe
import oracle as O
from moe_inputs import Workload, make_inputs


def _layer(inp, T, flags=0):
    """Device tensors of the first T tokens of `inp`, packed weights, and the
    reference forward on a caller-owned workspace."""
    from gpu_harness import cfg_of
    w = inp.w
    cfg = cfg_of(w, flags=flags, T=T)
    bufs = moe.alloc_buffers(cfg)
    d = lambda t: None if t is None else t.cuda().contiguous()
    moe.moe_prepare_weights(cfg, d(inp.Wg), d(inp.Wu), d(inp.Wd), bufs.packed, d(inp.Wsg), d(inp.Wsu), d(inp.Wsd))
    x, Wr, bias = d(inp.x[:T]), d(inp.Wr), d(inp.bias)
    ref = torch.empty_like(x)
    moe.moe_layer_fwd(cfg, Wr, bias, bufs.packed, x, ref, bufs.ws)
    return cfg, bufs, x, Wr, bias, ref


def _static(cfg, bufs, x, Wr, bias):
    out = torch.full_like(x, 7)
    status = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    moe.moe_layer_fwd_static(cfg, Wr, bias, bufs.packed, x, out, status)
    torch.cuda.synchronize()
    return out, status.tolist()


@pytest.mark.gpu
@pytest.mark.parametrize("prec,T1,T2", [("bf16", 4096, 1000), ("mxfp8", 700, 129)])
def test_static_forward_matches_workspace_forward_on_two_calls(gpu_lib, prec, T1, T2):
    # config 2's layer shape (H=2048, I=1024, E=64, k=6), one minibatch per call
    w = Workload("static_" + prec, T=T1, H=2048, I=1024, E=64, k=6, prec=prec, stream=8100)
    inp = make_inputs(w)
    for T in (T1, T2):  # the second call with a smaller input
        cfg, bufs, x, Wr, bias, ref = _layer(inp, T)
        assert moe.moe_query_sizes(cfg).workspace_fwd <= moe.MOE_STATIC_WORKSPACE_BYTES
        out, status = _static(cfg, bufs, x, Wr, bias)
        assert status == [0, 0]
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (prec, T)
        sub = inp.__class__(w.replace(T=T), inp.x[:T], inp.Wr, inp.bias, inp.Wg, inp.Wu, inp.Wd)
        err = O.rel_inf_err(out.float().cpu().numpy(), O.layer_forward(sub)["out"])
        print("%s T=%d: bitwise equal to moe_layer_fwd; max rel err %.3e" % (prec, T, err))
        assert err <= (5e-2 if prec == "mxfp8" else 1e-2)


@pytest.mark.gpu
def test_static_forward_clears_a_stale_status_word(gpu_lib):
    """A forced dropped signal leaves a timeout in the static workspace's status
    word; the next call clears it first and reports {0, 0}."""
    w = Workload("static_status", T=1500, H=256, I=128, E=8, k=2, minibatch=256, stream=8200)
    inp = make_inputs(w)
    cfg, bufs, x, Wr, bias, ref = _layer(inp, w.T, flags=moe.MOE_F_DEBUG_DROP_SIGNAL)
    _, status = _static(cfg, bufs, x, Wr, bias)
    assert status[0] == moe.MOE_DEV_WAIT_TIMEOUT
    cfg.flags &= ~moe.MOE_F_DEBUG_DROP_SIGNAL
    out, status = _static(cfg, bufs, x, Wr, bias)
    assert status == [0, 0]
    moe.moe_layer_fwd(cfg, Wr, bias, bufs.packed, x, ref, bufs.ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_static_forward_rejects_configs_beyond_the_static_workspace():
    """Checked on the host before any device call (runs without a GPU)."""
    cfg = moe.make_cfg(16384, 7168, 2048, 32, 8, minibatch=2560)
    assert moe.moe_query_sizes(cfg).workspace_fwd > moe.MOE_STATIC_WORKSPACE_BYTES
    t = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_fwd_static(cfg, t, None, t, t, t, stream=0)
    assert e.value.status == moe.MOE_E_WORKSPACE
