"""GPU parity of the layer backward against the fp64 CPU oracle, through the
C ABI: dx, dWg, dWu, dWd, dWr, the gate gradients and the shared expert's
weight gradients, each within max relative error 1e-2; repeated backward runs
must be bitwise identical."""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2


def _wl(name, **kw):
    return Workload(name, stream=8000 + (sum(map(ord, name)) % 997), **kw)


BWD_CASES = [
    _wl("bwd_tiny", T=64, H=128, I=64, E=8, k=2, minibatch=64),
    # several minibatches (ragged last), M/N/K tiles, partial wgrad tiles (H=384, I=192)
    _wl("bwd_shared", T=300, H=384, I=192, E=6, k=2, minibatch=128, shared_expert=True, router_bias="normal"),
    _wl("bwd_tiles", T=700, H=512, I=256, E=4, k=3, minibatch=256),
    _wl("bwd_k1", T=96, H=256, I=128, E=5, k=1),
    _wl("bwd_k64", T=200, H=64, I=64, E=4, k=2, minibatch=128, shared_expert=True),  # one K stage per GEMM
    # backward chunks (minibatches per input-gradient GEMM launch, about 5120
    # tokens): two chunks of two minibatches, the last minibatch ragged ...
    _wl("bwd_chunks2", T=7000, H=256, I=128, E=8, k=2, minibatch=2000, router_bias="normal"),
    # ... and three chunks of one minibatch
    _wl("bwd_chunks1", T=6000, H=256, I=128, E=8, k=2, minibatch=2600),
    # many experts with few rows each (most segments one half tile or empty)
    _wl("bwd_e64", T=600, H=256, I=128, E=64, k=6, minibatch=256),
    _wl("bwd_e256", T=300, H=128, I=64, E=256, k=16, minibatch=150, shared_expert=True),
]


@pytest.mark.parametrize("w", BWD_CASES, ids=lambda w: w.name)
def test_backward_matches_oracle(gpu_lib, w):
    from gpu_harness import Layer
    inp = make_inputs(w, with_dout=True)
    layer = Layer(inp)
    layer.forward()
    got = layer.backward(inp.dout)
    fwd = O.layer_forward(inp, keep=True, mx=False)
    ref = O.layer_backward(inp, fwd=fwd)
    names = ["dx", "dWg", "dWu", "dWd", "dWr", "dgate"] + (["dWsg", "dWsu", "dWsd"] if w.shared_expert else [])
    errs = {n: O.rel_inf_err(got[n].numpy(), ref[n]) for n in names}
    print(w.name, " ".join("%s %.2e" % kv for kv in errs.items()))
    for n, e in errs.items():
        assert e <= BF16_TOL, (n, e)


def test_backward_bitwise_repeatable(gpu_lib):
    from gpu_harness import Layer
    w = _wl("bwd_repeat", T=500, H=256, I=128, E=8, k=2, minibatch=200, shared_expert=True)
    inp = make_inputs(w, with_dout=True)
    layer = Layer(inp)
    layer.forward()
    a = layer.backward(inp.dout)
    layer.forward()
    b = layer.backward(inp.dout)
    for n in a:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("shared", [False, True], ids=["routed", "shared"])
def test_backward_empty_and_sparse_segments(gpu_lib, shared):
    """Minibatches of 12 tokens over 8 experts (k = 2): most (minibatch,
    expert) segments hold a few rows or none, and the last expert is never
    chosen (its router bias lowered by 1e4).  The weight gradients' K sequence
    then skips empty segments and stops inside ragged ones; the unused
    expert's weight gradients must be exactly zero and every gradient within
    the bf16 tolerance of the oracle."""
    import dispatch_grouped_gemm_moe_amd as moe
    from gpu_harness import Layer
    w = _wl("bwd_sparse" + ("_shared" if shared else ""), T=60, H=256, I=128, E=8, k=2, minibatch=12,
            shared_expert=shared)
    inp = make_inputs(w, with_dout=True)
    inp.bias = torch.zeros(w.E)
    inp.bias[-1] = -1e4
    _, idx, _ = O.route(O.as_f32(inp.x), inp.Wr, inp.bias, w.k)
    assert not (idx == w.E - 1).any()
    seg_rows = [np.bincount(idx[t0:t0 + w.minibatch].ravel(), minlength=w.E) for t0 in range(0, w.T, w.minibatch)]
    assert sum(int((c[:-1] == 0).sum()) for c in seg_rows) > 0, "no empty segment among the used experts"
    layer = Layer(inp)
    assert moe.moe_query_sizes(layer.cfg).minibatch == w.minibatch
    layer.forward()
    got = layer.backward(inp.dout)
    ref = O.layer_backward(inp, fwd=O.layer_forward(inp, keep=True, mx=False))
    for n in ("dWg", "dWu", "dWd"):
        assert not got[n][w.E - 1].any(), n
    names = ["dx", "dWg", "dWu", "dWd", "dWr", "dgate"] + (["dWsg", "dWsu", "dWsd"] if shared else [])
    errs = {n: O.rel_inf_err(got[n].numpy(), ref[n]) for n in names}
    print(w.name, "segment rows per minibatch", [c.tolist() for c in seg_rows], " ".join("%s %.2e" % kv for kv in errs.items()))
    for n, e in errs.items():
        assert e <= BF16_TOL, (n, e)
