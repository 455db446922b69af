"""Full-size backward parity of the layer at H=7168, I=2048, E=32, k=8 and
16384 tokens in minibatches of 2560 (a ragged last one), launched as the
benchmark launches it (same configuration, default ring slots and CU split),
against the fp64 CPU oracle on outputs it can compute one at a time.

With the benchmark's dout:
* dx and the gate gradients of sampled tokens (each token's gradients depend
  on that token alone), chosen so that every 128-row block of every
  (minibatch, expert) segment -- the shared expert's too -- holds a sampled
  row, and so every M tile of every input-gradient GEMM; the first and last
  token among them;
* sampled columns of dWg and dWu and rows of dWd of the most-loaded, the
  least-loaded and the last expert, over all of their tokens, and sampled
  shared-expert columns;
* dWr, which sums over every token, through the invariant that each of its rows
  sums to zero (the gate softmax makes a token's logit gradients sum to zero),
  within 1e-3 of its largest element.

With dout kept only on the sampled tokens, every gradient is the oracle's
backward of those tokens alone: dWr is compared whole, dx and the gate
gradients must be exactly zero off the sample, the weight gradients of experts
that no sampled token reaches exactly zero, and two reached experts' weight
gradients (and the shared expert's) are compared whole.

Under MXFP8 the routed experts' weight gradients take MXFP8 operands quantised
along the token rows of each (minibatch, expert) segment, so a 32-row block
can hold tokens on and off the sample: with dout kept on the sample only, the
oracle's weight gradients then run over every token of the expert (dout zero
off the sample) instead of over the sampled tokens alone.

Tolerances: max relative error 1e-2 for bf16, 5e-2 for MXFP8.
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import KIMI_BF16, KIMI_FWD_BWD, LayerInputs, make_inputs
from sampling import covering_tokens

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

TOL = {"bf16": 1e-2, "mxfp8": 5e-2}


@pytest.fixture(scope="module", params=[KIMI_BF16, KIMI_FWD_BWD], ids=lambda w: w.name)
def full(request, gpu_lib):
    from gpu_harness import Layer
    w = request.param
    inp = make_inputs(w, with_dout=True)
    layer = Layer(inp)
    layer.forward()
    torch.cuda.synchronize()
    _, idx, _ = O.route(O.as_f32(inp.x), inp.Wr, inp.bias, w.k)
    import dispatch_grouped_gemm_moe_amd as moe
    assert moe.moe_query_sizes(layer.cfg).minibatch == w.minibatch
    S = np.union1d(covering_tokens(idx, w.minibatch, shared=w.shared_expert), [0, w.T - 1])
    print("%s: layer forward done; oracle on %d tokens" % (w.name, len(S)), flush=True)
    fwd = O.layer_forward(inp, tokens=S, keep=True)
    ref = O.layer_backward(inp, dout=inp.dout[S], fwd=fwd, weight_grads=False)
    yield SimpleNamespace(w=w, inp=inp, layer=layer, S=S, fwd=fwd, ref=ref)
    del layer
    torch.cuda.empty_cache()


def _host(t):
    return t.float().cpu().numpy()


def _check(errs, tol, label):
    print(label, " ".join("%s %.2e" % kv for kv in errs.items()))
    for n, e in errs.items():
        assert e <= tol, (n, e)


def test_full_size_backward_sampled_outputs(full):
    w, inp, S, ref = full.w, full.inp, full.S, full.ref
    g = full.layer.backward(inp.dout, to_cpu=False)
    Sd = torch.from_numpy(S).to(g["dx"].device)
    errs = {"dx": O.rel_inf_err(_host(g["dx"][Sd]), ref["dx"]),
            "dgate": O.rel_inf_err(_host(g["dgate"][Sd]), ref["dgate"])}
    _, idx, gw = O.route(O.as_f32(inp.x), inp.Wr, inp.bias, w.k)
    counts = np.bincount(idx.ravel(), minlength=w.E)
    experts = sorted({int(counts.argmax()), int(counts.argmin()), w.E - 1})
    cols = [0, 1 + int(np.random.default_rng(18).integers(w.I - 2)), w.I - 1]
    mxw = w.minibatch if w.prec == "mxfp8" else None  # MXFP8 weight gradients: their segments
    for e in experts:
        c = O.weight_grad_columns(inp, e, cols, routing=(idx, gw), mx_wgrad_minibatch=mxw)
        errs["dWg[%d]" % e] = O.rel_inf_err(_host(g["dWg"][e][:, cols]), c["dWg"])
        errs["dWu[%d]" % e] = O.rel_inf_err(_host(g["dWu"][e][:, cols]), c["dWu"])
        errs["dWd[%d]" % e] = O.rel_inf_err(_host(g["dWd"][e][cols, :]), c["dWd"])
    if w.shared_expert:
        c = O.weight_grad_columns(inp, -1, cols)
        errs["dWsg"] = O.rel_inf_err(_host(g["dWsg"][:, cols]), c["dWg"])
        errs["dWsu"] = O.rel_inf_err(_host(g["dWsu"][:, cols]), c["dWu"])
        errs["dWsd"] = O.rel_inf_err(_host(g["dWsd"][cols, :]), c["dWd"])
    dWr = _host(g["dWr"]).astype(np.float64)
    row_sums = float(np.abs(dWr.sum(axis=1)).max() / np.abs(dWr).max())
    _check(errs, TOL[w.prec], "%s (expert rows %s, columns %s; dWr row sums %.2e)"
           % (w.name, counts[experts].tolist(), cols, row_sums))
    # exact in any arithmetic up to the fp32 rounding of the logit gradients
    assert row_sums <= 1e-3, row_sums


def test_full_size_backward_dout_on_sampled_tokens_only(full):
    w, inp, S, ref, fwd = full.w, full.inp, full.S, full.ref, full.fwd
    masked = torch.zeros_like(inp.dout)
    masked[torch.from_numpy(S)] = inp.dout[torch.from_numpy(S)]
    g = full.layer.backward(masked, to_cpu=False)
    dev = g["dx"].device
    Sd = torch.from_numpy(S).to(dev)
    off = torch.ones(w.T, dtype=torch.bool, device=dev)
    off[Sd] = False
    assert not g["dx"][off].any() and not g["dgate"][off].any()
    reached = set(np.unique(fwd["idx"]).tolist())
    for e in sorted(set(range(w.E)) - reached):
        assert not (g["dWg"][e].any() or g["dWu"][e].any() or g["dWd"][e].any()), e
    errs = {"dx": O.rel_inf_err(_host(g["dx"][Sd]), ref["dx"]),
            "dgate": O.rel_inf_err(_host(g["dgate"][Sd]), ref["dgate"]),
            "dWr": O.rel_inf_err(_host(g["dWr"]), ref["dWr"])}
    sub = LayerInputs(w.replace(T=len(S)), inp.x[S], inp.Wr, inp.bias, inp.Wg, inp.Wu, inp.Wd,
                      inp.Wsg, inp.Wsu, inp.Wsd, inp.dout[S])
    every = np.arange(w.I)
    for e in sorted({int(fwd["idx"][0, 0]), int(fwd["idx"][-1, -1])}):
        if w.prec == "mxfp8":  # row blocks span sampled and unsampled tokens: every token, masked dout
            _, idx, gw = O.route(O.as_f32(inp.x), inp.Wr, inp.bias, w.k)
            c = O.weight_grad_columns(inp, e, every, dout=masked, routing=(idx, gw),
                                      mx_wgrad_minibatch=w.minibatch)
        else:
            c = O.weight_grad_columns(sub, e, every, routing=(fwd["idx"], fwd["w"]))
        errs["dWg[%d]" % e] = O.rel_inf_err(_host(g["dWg"][e]), c["dWg"])
        errs["dWu[%d]" % e] = O.rel_inf_err(_host(g["dWu"][e]), c["dWu"])
        errs["dWd[%d]" % e] = O.rel_inf_err(_host(g["dWd"][e]), c["dWd"])
    if w.shared_expert:
        c = O.weight_grad_columns(sub, -1, every)
        errs["dWsg"] = O.rel_inf_err(_host(g["dWsg"]), c["dWg"])
        errs["dWsu"] = O.rel_inf_err(_host(g["dWsu"]), c["dWu"])
        errs["dWsd"] = O.rel_inf_err(_host(g["dWsd"]), c["dWd"])
    _check(errs, TOL[w.prec], "%s dout on %d tokens (%d experts reached)" % (w.name, len(S), len(reached)))


def test_full_size_ten_runs_bitwise_identical(full):
    """Ten forward + backward passes at full size, launched as the benchmark
    launches them, give bitwise-identical outputs and gradients (every sum in
    the layer has a fixed order)."""
    layer, inp = full.layer, full.inp
    first = None
    for run in range(10):
        out = layer.forward().clone()
        g = layer.backward(inp.dout, to_cpu=False)
        g["out"] = out
        if first is None:
            first = g
            continue
        for n in first:
            assert torch.equal(g[n], first[n]), (run, n)
    print("%s: 10 runs bitwise identical (%s)" % (full.w.name, ", ".join(sorted(first))))
