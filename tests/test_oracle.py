"""Pins of the CPU oracle against facts that do not depend on the oracle itself:
exact integer arithmetic, hand-worked rounding cases, textbook error bounds,
brute force on tiny inputs, library routines (torch CPU softmax, SwiGLU and
autograd, torch's float8_e4m3fn cast), closed forms and invariants.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import Workload, make_inputs, LayerInputs


def tiny(T=16, H=64, I=32, E=4, k=2, **kw):
    return Workload("pin", T=T, H=H, I=I, E=E, k=k, stream=9000 + T + H + I + E + k, **kw)


# ---------------------------------------------------------------- logits

def test_logits_integer_inputs_are_exact_dot_products():
    rng = np.random.default_rng(1)
    T, H, E = 5, 256, 7
    x = rng.integers(-8, 9, size=(T, H)).astype(np.float32)
    Wr = rng.integers(-8, 9, size=(H, E)).astype(np.float32)
    bias = rng.integers(-100, 100, size=E).astype(np.float32)
    got = O.router_logits(x, Wr, bias)
    exact = [[sum(int(x[t, h]) * int(Wr[h, e]) for h in range(H)) + int(bias[e]) for e in range(E)]
             for t in range(T)]
    assert (got == np.array(exact, dtype=np.float32)).all()


def _one_hot_dot(H, entries):
    """x = 1 at the given h, Wr[:,0] = value there; all else 0."""
    x = np.zeros((1, H), np.float32)
    Wr = np.zeros((H, 1), np.float32)
    for h, (xv, wv) in entries.items():
        x[0, h] = xv
        Wr[h, 0] = wv
    return O.router_logits(x, Wr)[0, 0]


def test_logits_lane_then_tree_order():
    # lane 0 sums h=0 (2^24) then h=64 (+1): 2^24+1 is a tie, rounds to even 2^24.
    # lane 1 holds -2^24.  Tree merges lanes 0 and 1 last: result 0.
    # Plain left-to-right summation would give 1.
    v = _one_hot_dot(128, {0: (1.0, 2.0 ** 24), 1: (1.0, -2.0 ** 24), 64: (1.0, 1.0)})
    assert v == 0.0
    # lane 32 (+1) merges into lane 0 (2^24) at the first tree level (tie -> 2^24),
    # before lane 1 (-2^24) does at the last: 0.  A pairwise tree of neighbours gives 1.
    v = _one_hot_dot(64, {0: (1.0, 2.0 ** 24), 1: (1.0, -2.0 ** 24), 32: (1.0, 1.0)})
    assert v == 0.0
    # lane 2 (+1) merges into lane 0 at s=2, before lane 1 at s=1: 0 again.
    v = _one_hot_dot(64, {0: (1.0, 2.0 ** 24), 1: (1.0, -2.0 ** 24), 2: (1.0, 1.0)})
    assert v == 0.0
    # lane 1 (-2^24) and lane 33 (+1) merge first: -2^24+1 = -(2^24-1), exact.
    # then lane 0 (2^24) + that = 1.
    v = _one_hot_dot(64, {0: (1.0, 2.0 ** 24), 1: (1.0, -2.0 ** 24), 33: (1.0, 1.0)})
    assert v == 1.0


def test_logits_use_fused_multiply_add():
    # lane 0: first -1, then (1+2^-12)^2 = 1 + 2^-11 + 2^-24 added in one rounding.
    # A separate multiply would round the product to 1 + 2^-11 and give 2^-11.
    a = 1.0 + 2.0 ** -12
    v = _one_hot_dot(128, {0: (-1.0, 1.0), 64: (a, a)})
    assert v == np.float32(2.0 ** -11 + 2.0 ** -24)


def test_logits_within_textbook_bound():
    rng = np.random.default_rng(2)
    T, H, E = 32, 2048, 16
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    Wr = rng.normal(0, 0.02, size=(H, E)).astype(np.float32)
    got = O.router_logits(x, Wr).astype(np.float64)
    x64 = x.double().numpy()
    exact = x64 @ Wr.astype(np.float64)
    # each logit passes through at most H/64 + 6 fp32 roundings
    n = H // 64 + 6
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    bound = gamma * (np.abs(x64) @ np.abs(Wr.astype(np.float64)))
    assert (np.abs(got - exact) <= bound).all()


def test_logits_reject_h_not_multiple_of_64():
    with pytest.raises(ValueError):
        O.router_logits(np.zeros((1, 96), np.float32), np.zeros((96, 2), np.float32))


# ---------------------------------------------------------------- selection

def test_topk_matches_brute_force_sort():
    rng = np.random.default_rng(4)
    logits = rng.normal(size=(50, 9)).astype(np.float32)
    logits[3, 2] = logits[3, 5]  # a tie
    logits[7, :] = 0.0
    logits[8, 1], logits[8, 4] = -0.0, 0.0  # signed zeros compare equal
    for k in (1, 3, 9):
        idx = O.topk_select(logits, k)
        for t in range(logits.shape[0]):
            want = sorted(range(9), key=lambda e: (-float(logits[t, e]), e))[:k]
            assert list(idx[t]) == want


def test_topk_ties_from_identical_router_columns_pick_lower_index():
    w = tiny(T=32, E=6, k=3)
    inp = make_inputs(w)
    Wr = O.as_f32(inp.Wr).copy()
    Wr[:, 4] = Wr[:, 1]  # experts 1 and 4 always tie exactly
    logits, idx, _ = O.route(inp.x, Wr, None, 6)
    for t in range(32):
        row = list(idx[t])
        assert row.index(1) < row.index(4)


def test_gate_weights_closed_forms():
    rng = np.random.default_rng(5)
    logits = rng.normal(size=(40, 8)).astype(np.float32)
    # k=1: a single weight of exactly 1
    idx = O.topk_select(logits, 1)
    assert (O.gate_weights(logits, idx) == 1.0).all()
    # k=E: the full softmax (torch CPU, fp64), reordered by selection
    idx = O.topk_select(logits, 8)
    ref = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    np.testing.assert_allclose(O.gate_weights(logits, idx), np.take_along_axis(ref, idx, 1),
                               rtol=1e-13, atol=0)
    # renormalised top-k softmax: weights sum to one, ratios follow exp(l_i - l_j)
    idx = O.topk_select(logits, 3)
    gw = O.gate_weights(logits, idx)
    np.testing.assert_allclose(gw.sum(1), 1.0, rtol=0, atol=1e-15)
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), 1)
    np.testing.assert_allclose(gw[:, 1] / gw[:, 0], np.exp(sel[:, 1] - sel[:, 0]), rtol=1e-13)


# ---------------------------------------------------------------- layout

def _check_layout(idx, E, counts, offsets, row_token, tok_row):
    T, k = idx.shape
    assert counts.sum() == T * k
    assert offsets[0] == 0 and (np.diff(offsets) == counts).all()
    # brute force: count directly
    for e in range(E):
        assert counts[e] == sum(1 for t in range(T) for j in range(k) if idx[t, j] == e)
    # rows of each expert are contiguous and in ascending token order
    for e in range(E):
        toks = row_token[offsets[e]:offsets[e + 1]]
        assert (np.diff(toks) > 0).all()
        for t in toks:
            assert e in idx[t]
    # tok_row inverts row_token, and is a bijection onto the rows
    assert sorted(tok_row.ravel().tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            r = tok_row[t, j]
            assert row_token[r] == t
            assert offsets[idx[t, j]] <= r < offsets[idx[t, j] + 1]


def test_layout_invariants_and_brute_force():
    for (T, E, k, seed) in [(64, 8, 2, 0), (37, 5, 3, 1), (1, 4, 4, 2), (200, 16, 6, 3)]:
        rng = np.random.default_rng(seed)
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        _check_layout(idx, E, *O.dispatch_layout(idx, E))


def test_layout_empty_experts_and_minibatch_slices():
    idx = np.array([[0, 3], [3, 0], [0, 3]], np.int32)
    counts, offsets, row_token, tok_row = O.dispatch_layout(idx, 5)
    assert counts.tolist() == [3, 0, 0, 3, 0]
    assert offsets.tolist() == [0, 3, 3, 3, 6, 6]
    assert row_token.tolist() == [0, 1, 2, 0, 1, 2]
    assert tok_row.tolist() == [[0, 3], [4, 1], [2, 5]]
    mbs = O.minibatch_layouts(idx, 5, 2)
    assert len(mbs) == 2
    assert mbs[1][0].tolist() == [1, 0, 0, 1, 0] and mbs[1][2].tolist() == [0, 0]


# ---------------------------------------------------------------- FFN / forward

def test_single_expert_top1_is_a_dense_swiglu_ffn_torch():
    w = tiny(T=24, H=128, I=64, E=1, k=1)
    inp = make_inputs(w)
    out = O.layer_forward(inp)["out"]
    x = inp.x.double()
    ref = (torch.nn.functional.silu(x @ inp.Wg[0].double()) * (x @ inp.Wu[0].double())) @ inp.Wd[0].double()
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_forward_matches_pure_python_brute_force():
    w = tiny(T=6, H=64, I=8, E=4, k=2)
    inp = make_inputs(w)
    res = O.layer_forward(inp)
    X = inp.x.double().tolist()
    Wg, Wu, Wd = (t.double().tolist() for t in (inp.Wg, inp.Wu, inp.Wd))
    logits = res["logits"]
    for t in range(w.T):
        # every expert on the token, then keep the top-k by logit
        ys = []
        for e in range(w.E):
            h = []
            for i in range(w.I):
                g = sum(X[t][hh] * Wg[e][hh][i] for hh in range(w.H))
                u = sum(X[t][hh] * Wu[e][hh][i] for hh in range(w.H))
                h.append(g / (1 + math.exp(-g)) * u)
            ys.append([sum(h[i] * Wd[e][i][hh] for i in range(w.I)) for hh in range(w.H)])
        sel = sorted(range(w.E), key=lambda e: (-float(logits[t, e]), e))[:w.k]
        z = [math.exp(float(logits[t, e]) - float(logits[t, sel[0]])) for e in sel]
        ws = [v / sum(z) for v in z]
        want = [sum(ws[j] * ys[sel[j]][hh] for j in range(w.k)) for hh in range(w.H)]
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-11, atol=1e-15)


def test_identity_experts_return_the_input():
    inp = make_inputs(tiny(T=40, E=8, k=3))
    out = O.layer_forward(inp, identity_experts=True)["out"]
    np.testing.assert_allclose(out, inp.x.double().numpy(), rtol=1e-15, atol=0)


def test_top1_combine_returns_the_expert_output():
    w = tiny(T=30, E=5, k=1)
    inp = make_inputs(w)
    res = O.layer_forward(inp, keep=True)
    np.testing.assert_array_equal(res["out"], res["Y"][:, 0, :])


def test_linearity_in_down_projection_is_exact():
    w = tiny(T=20, E=4, k=2)
    inp = make_inputs(w)
    base = O.layer_forward(inp)["out"]
    inp2 = LayerInputs(w, inp.x, inp.Wr, inp.bias, inp.Wg, inp.Wu, inp.Wd * 2)
    np.testing.assert_array_equal(O.layer_forward(inp2)["out"], 2 * base)


def test_token_permutation_equivariance():
    w = tiny(T=33, E=6, k=2)
    inp = make_inputs(w)
    perm = np.random.default_rng(7).permutation(w.T)
    a = O.layer_forward(inp)["out"]
    b = O.layer_forward(inp, tokens=perm)["out"]
    # per-token math; only BLAS blocking (a function of the row count) may differ
    np.testing.assert_allclose(a[perm], b, rtol=1e-12, atol=1e-18)


def test_token_subset_matches_full_forward():
    w = tiny(T=50, E=6, k=3)
    inp = make_inputs(w)
    full = O.layer_forward(inp)["out"]
    sub = O.layer_forward(inp, tokens=[3, 17, 49])["out"]
    np.testing.assert_allclose(full[[3, 17, 49]], sub, rtol=1e-12, atol=1e-18)


def test_shared_expert_adds_a_dense_ffn():
    w = tiny(T=12, E=4, k=2, shared_expert=True)
    inp = make_inputs(w)
    with_s = O.layer_forward(inp)["out"]
    without = O.layer_forward(inp, shared=False)["out"]
    x = inp.x.double()
    s = (torch.nn.functional.silu(x @ inp.Wsg.double()) * (x @ inp.Wsu.double())) @ inp.Wsd.double()
    np.testing.assert_allclose(with_s - without, s.numpy(), rtol=1e-10, atol=1e-14)


# ---------------------------------------------------------------- MXFP8

def test_e4m3_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(codes)
    assert np.isnan(O.E4M3_TABLE[~finite]).all()
    np.testing.assert_array_equal(O.E4M3_TABLE[finite], codes[finite])
    assert O.E4M3_TABLE[0x7E] == 448.0 and O.E4M3_TABLE[0x01] == 2.0 ** -9


def test_e4m3_encode_roundtrips_and_matches_torch_rne():
    finite = [c for c in range(256) if not np.isnan(O.E4M3_TABLE[c])]
    assert O.e4m3_encode(O.E4M3_TABLE[finite]).tolist() == finite
    rng = np.random.default_rng(8)
    v = np.concatenate([rng.normal(0, 60, 20000), rng.normal(0, 0.01, 20000),
                        (O.E4M3_TABLE[1:0x7E] + O.E4M3_TABLE[2:0x7F]) / 2])  # exact midpoints
    v = np.clip(v, -448, 448).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(v), ref)
    # saturation
    assert O.e4m3_encode(np.array([1e4, -1e4, 464.0])).tolist() == [0x7E, 0xFE, 0x7E]


def test_e8m0_scale_is_the_smallest_power_of_two_within_448():
    rng = np.random.default_rng(9)
    amax = np.concatenate([np.abs(rng.normal(0, 1, 2000)) * 10.0 ** rng.integers(-30, 30, 2000),
                           [448.0, 449.0, 1.0, 2.0 ** -140, 896.0, 897.0]])
    e = O.e8m0_scale_exponent(amax)
    for a, ee in zip(amax, e):
        want = next(q for q in range(-200, 200) if a <= 448.0 * 2.0 ** q)
        assert ee == max(-127, min(127, want))
    assert O.e8m0_scale_exponent(np.array([448.0, 449.0, 1.0, 0.0])).tolist() == [0, 1, -8, 0]


def test_mx_quantise_hand_blocks():
    blk = np.zeros((3, 32), np.float32)
    blk[0, 0] = 448.0; blk[0, 1] = -1.0; blk[0, 2] = 2.0 ** -9; blk[0, 3] = 2.0 ** -10
    blk[1, :] = 0.0
    blk[2, 0] = 896.0; blk[2, 1] = 3.0
    codes, scales = O.mx_quantize(blk, axis=1)
    assert scales[:, 0].tolist() == [127, 127, 128]
    assert codes[0, :4].tolist() == [0x7E, 0xB8, 0x01, 0x00]  # 2^-10 is half the step: tie -> 0
    assert (codes[1] == 0).all()
    assert codes[2, :2].tolist() == [0x7E, 0x3C]  # 896/2 = 448 (S.1111.110); 3/2 = 1.5 (S.0111.100)
    np.testing.assert_array_equal(O.mx_dequantize(codes, scales, 1)[2, :2], [896.0, 3.0])


def test_mx_quantiser_c_equals_python_helpers():
    rng = np.random.default_rng(12)
    a = np.concatenate([rng.normal(0, 1, (40, 96)), rng.normal(0, 1e-3, (8, 96)) * 10.0 ** rng.integers(-30, 30, (8, 1)),
                        np.zeros((2, 96))]).astype(np.float32)
    a[3, 5] = -0.0
    a[7, :32] = np.float32(448.0 * 2.0 ** -3)  # exactly at a scale boundary
    c1, s1 = O.mx_quantize(a, 1)
    c2, s2 = O.mx_quantize_reference(a, 1)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)
    c1, s1 = O.mx_quantize(a[:32], 0)
    c2, s2 = O.mx_quantize_reference(a[:32], 0)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)


def test_mx_quantise_axis_and_error_bound():
    rng = np.random.default_rng(10)
    a = rng.normal(size=(64, 96)).astype(np.float32)
    q0 = O.mx_roundtrip(a, 0)
    np.testing.assert_array_equal(q0, O.mx_roundtrip(a.T, 1).T)
    # relative error of E4M3 normal numbers is at most 2^-4 (half of the 3-bit step)
    blk = np.abs(a.reshape(64, 3, 32)).max(-1, keepdims=True)
    err = np.abs(O.mx_roundtrip(a, 1) - a).reshape(64, 3, 32)
    scale = 2.0 ** O.e8m0_scale_exponent(blk)
    assert (err <= np.maximum(np.abs(a.reshape(64, 3, 32)) * 2.0 ** -4, scale * 2.0 ** -10)).all()


def test_mx_forward_equals_plain_forward_on_representable_values():
    # every x, weight and h already on the MXFP8 grid: quantisation is the identity.
    w = tiny(T=8, H=64, I=32, E=2, k=1, prec="mxfp8")
    inp = make_inputs(w)
    x = torch.zeros(8, 64); x[:, 0] = 1.0  # x = e_0 -> g, u = row 0 of the weights
    Wg = torch.zeros(2, 64, 32); Wu = torch.zeros(2, 64, 32); Wd = torch.zeros(2, 32, 64)
    Wg[:, 0, :] = 64.0  # g = 64: silu(64) rounds to exactly 64 in fp64
    Wu[:, 0, :] = 0.5  # u = 0.5, so h = 32 on every i
    Wd[:, :, :] = 0.25  # y = 32 inputs * 32 * 0.25 = 256 on every h
    inp2 = LayerInputs(w, x.to(torch.bfloat16), inp.Wr, None, Wg.to(torch.bfloat16),
                       Wu.to(torch.bfloat16), Wd.to(torch.bfloat16))
    a = O.layer_forward(inp2, mx=True)["out"]
    b = O.layer_forward(inp2, mx=False)["out"]
    np.testing.assert_allclose(a, b, rtol=1e-12)
    np.testing.assert_array_equal(b, np.full_like(b, 256.0))


# ---------------------------------------------------------------- backward

def _fd_inputs(w, seed):
    inp = make_inputs(w, with_dout=True)
    f64 = lambda t: t.double().numpy().copy() if t is not None else None
    return LayerInputs(w, f64(inp.x), f64(inp.Wr), f64(inp.bias), f64(inp.Wg), f64(inp.Wu),
                       f64(inp.Wd), f64(inp.Wsg), f64(inp.Wsu), f64(inp.Wsd), f64(inp.dout))


def _objective(inp):
    return float((O.layer_forward(inp, logits64=True)["out"] * inp.dout).sum())


def test_backward_matches_central_finite_differences():
    w = tiny(T=10, H=64, I=16, E=4, k=2, shared_expert=True, router_bias="normal")
    inp = _fd_inputs(w, 0)
    fwd = O.layer_forward(inp, keep=True, logits64=True)
    g = O.layer_backward(inp, fwd=fwd)
    logits = fwd["logits"]
    srt = np.sort(logits, 1)[:, ::-1]
    assert (srt[:, w.k - 1] - srt[:, w.k] > 1e-4).all()  # no selection flips under +-eps
    rng = np.random.default_rng(11)
    eps = 1e-6
    checks = [("x", "dx"), ("Wr", "dWr"), ("Wg", "dWg"), ("Wu", "dWu"), ("Wd", "dWd"),
              ("Wsg", "dWsg"), ("Wsu", "dWsu"), ("Wsd", "dWsd")]
    for name, gname in checks:
        arr = getattr(inp, name)
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            old = arr[pos]
            arr[pos] = old + eps; fp = _objective(inp)
            arr[pos] = old - eps; fm = _objective(inp)
            arr[pos] = old
            fd = (fp - fm) / (2 * eps)
            assert abs(fd - g[gname][pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, g[gname][pos])


def test_backward_matches_torch_autograd():
    w = tiny(T=20, H=128, I=32, E=6, k=3, router_bias="normal")
    inp = _fd_inputs(w, 1)
    fwd = O.layer_forward(inp, keep=True, logits64=True)
    g = O.layer_backward(inp, fwd=fwd)
    idx = torch.from_numpy(fwd["idx"].astype(np.int64))
    t = {n: torch.tensor(getattr(inp, n), requires_grad=True) for n in ("x", "Wr", "Wg", "Wu", "Wd")}
    logits = t["x"] @ t["Wr"] + torch.from_numpy(inp.bias)
    wsel = torch.softmax(torch.gather(logits, 1, idx), dim=1)
    out = torch.zeros(w.T, w.H, dtype=torch.float64)
    for j in range(w.k):
        e = idx[:, j]
        gg = torch.einsum("th,thi->ti", t["x"], t["Wg"][e])
        uu = torch.einsum("th,thi->ti", t["x"], t["Wu"][e])
        yy = torch.einsum("ti,tih->th", torch.nn.functional.silu(gg) * uu, t["Wd"][e])
        out = out + wsel[:, j:j + 1] * yy
    (out * torch.from_numpy(inp.dout)).sum().backward()
    for n, gn in [("x", "dx"), ("Wr", "dWr"), ("Wg", "dWg"), ("Wu", "dWu"), ("Wd", "dWd")]:
        np.testing.assert_allclose(g[gn], t[n].grad.numpy(), rtol=1e-9, atol=1e-12)


def test_backward_scales_exactly_with_dout():
    w = tiny(T=12, E=4, k=2)
    inp = _fd_inputs(w, 2)
    fwd = O.layer_forward(inp, keep=True)
    g1 = O.layer_backward(inp, fwd=fwd)
    g2 = O.layer_backward(inp, dout=2 * inp.dout, fwd=fwd)
    for n in ("dx", "dWg", "dWu", "dWd", "dWr", "dgate"):
        np.testing.assert_array_equal(g2[n], 2 * g1[n])


def test_weight_grad_columns_match_torch_autograd():
    """Column-restricted weight gradients of every routed expert and of the
    shared expert against autograd of a dense torch formulation (routing and
    gate weights frozen at the oracle forward's)."""
    w = tiny(T=40, H=128, I=64, E=5, k=3, shared_expert=True, router_bias="normal")
    inp = _fd_inputs(w, 3)
    fwd = O.layer_forward(inp, keep=True)
    idx = torch.from_numpy(fwd["idx"].astype(np.int64))
    gw = torch.from_numpy(fwd["w"])
    names = ("Wg", "Wu", "Wd", "Wsg", "Wsu", "Wsd")
    t = {n: torch.tensor(getattr(inp, n), requires_grad=True) for n in names}
    x = torch.from_numpy(inp.x)
    out = torch.zeros(w.T, w.H, dtype=torch.float64)
    for j in range(w.k):
        e = idx[:, j]
        gg = torch.einsum("th,thi->ti", x, t["Wg"][e])
        uu = torch.einsum("th,thi->ti", x, t["Wu"][e])
        out = out + gw[:, j:j + 1] * torch.einsum("ti,tih->th", torch.nn.functional.silu(gg) * uu, t["Wd"][e])
    out = out + (torch.nn.functional.silu(x @ t["Wsg"]) * (x @ t["Wsu"])) @ t["Wsd"]
    (out * torch.from_numpy(inp.dout)).sum().backward()
    cols = [0, 9, 31, 63]
    routing = (fwd["idx"], fwd["w"])
    for e in range(-1, w.E):
        got = O.weight_grad_columns(inp, e, cols, routing=routing)
        pre = "Ws" if e < 0 else "W"
        sel = (lambda a: a) if e < 0 else (lambda a: a[e])
        np.testing.assert_allclose(got["dWg"], sel(t[pre + "g"].grad.numpy())[:, cols], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(got["dWu"], sel(t[pre + "u"].grad.numpy())[:, cols], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(got["dWd"], sel(t[pre + "d"].grad.numpy())[cols, :], rtol=1e-9, atol=1e-12)
    # default routing: the oracle's own fixed-order fp32 route of every token
    got = O.weight_grad_columns(inp, 2, cols)
    np.testing.assert_allclose(got["dWd"], t["Wd"].grad.numpy()[2][cols, :], rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("prec", ["bf16", "mxfp8"])
def test_backward_of_token_subset_equals_backward_with_masked_dout(prec):
    """Gradients are linear in dout and every token's contribution depends on
    that token alone (its MXFP8 blocks run along its own row), so the backward
    with dout zero outside a token subset S equals the backward of the layer
    restricted to S: same weight and router gradients, same dx and gate
    gradients on S, exact zeros elsewhere."""
    w = tiny(T=48, H=128, I=64, E=5, k=3, shared_expert=True, router_bias="normal", prec=prec)
    inp = make_inputs(w, with_dout=True)
    S = np.array([0, 7, 8, 30, 47])
    masked = torch.zeros_like(inp.dout)
    masked[S] = inp.dout[S]
    full = O.layer_backward(inp, dout=masked, fwd=O.layer_forward(inp, keep=True))
    sub = O.layer_backward(inp, dout=inp.dout[S], fwd=O.layer_forward(inp, tokens=S, keep=True))
    rest = np.setdiff1d(np.arange(w.T), S)
    assert (full["dx"][rest] == 0).all() and (full["dgate"][rest] == 0).all()
    for n in ("dx", "dgate"):
        np.testing.assert_allclose(full[n][S], sub[n], rtol=1e-12, atol=1e-15, err_msg=n)
    for n in ("dWg", "dWu", "dWd", "dWr", "dWsg", "dWsu", "dWsd"):
        np.testing.assert_allclose(full[n], sub[n], rtol=1e-12, atol=1e-15, err_msg=n)
    lean = O.layer_backward(inp, dout=inp.dout[S], fwd=O.layer_forward(inp, tokens=S, keep=True),
                            weight_grads=False)
    assert sorted(lean) == ["dWr", "dgate", "dlogits", "dx"]
    for n in lean:
        np.testing.assert_array_equal(lean[n], sub[n], err_msg=n)


# ---------------------------------------------------------------- MXFP8 backward

def _e4m3_positive_values():
    """The 127 finite non-negative E4M3 (OCP, bias 7) values by code, from the
    format definition: exponent field 0 is subnormal (m/8 * 2^-6)."""
    vals = []
    for c in range(127):
        ex, m = c >> 3, c & 7
        vals.append(m / 8 * 2.0 ** -6 if ex == 0 else (1 + m / 8) * 2.0 ** (ex - 7))
    return vals


_E4M3_POS = _e4m3_positive_values()


def _brute_quant_block(vals):
    """Dequantised MXFP8 of one 32-element block by enumeration: the smallest
    scale 2^e (e in [-127, 127]) with amax <= 448 * 2^e (e = 0 for an all-zero
    block), each element / 2^e to the nearest E4M3 value, ties to the even code."""
    vals = [float(np.float32(v)) for v in vals]
    amax = max(abs(v) for v in vals)
    e = 0
    if amax > 0:
        e = -127
        while e < 127 and amax > 448.0 * 2.0 ** e:
            e += 1
    out = []
    for v in vals:
        t = abs(v) / 2.0 ** e
        best = None
        for c, cv in enumerate(_E4M3_POS):
            d = abs(cv - t)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (d, c)
        out.append(math.copysign(_E4M3_POS[best[1]] * 2.0 ** e, v))
    return out


def _brute_quant_rows(M):
    """Quantise every row of the nested list M in 32-element blocks along the row."""
    return [sum((_brute_quant_block(r[b:b + 32]) for b in range(0, len(r), 32)), []) for r in M]


def _T(M):
    return [list(c) for c in zip(*M)]


def _brute_mx_rows(inp, idx, gw):
    """Scalar brute force of the MXFP8 layer for every routed (t, j): the
    forward (x along H; Wg, Wu along H; h along I; Wd along I) and the
    input-gradient GEMMs (dY and Wd along H; dG, dU and Wg, Wu along I).
    Returns {(t, j): dict(x, g, u, h, y, dy, dg, du, dx)} with plain lists."""
    w = inp.w
    T, H, I, E, k = w.T, w.H, w.I, w.E, w.k
    x = inp.x.double().tolist()
    dout = inp.dout.double().tolist()
    sig = lambda z: 1.0 / (1.0 + math.exp(-z)) if z >= 0 else math.exp(z) / (1.0 + math.exp(z))
    xq = _brute_quant_rows(x)
    rows = {}
    for e in range(E):
        Wg, Wu, Wd = (t[e].double().tolist() for t in (inp.Wg, inp.Wu, inp.Wd))  # [H][I], [H][I], [I][H]
        Wgf, Wuf = _T(_brute_quant_rows(_T(Wg))), _T(_brute_quant_rows(_T(Wu)))  # forward: along H
        Wdf = _T(_brute_quant_rows(_T(Wd)))                                      # forward: along I
        Wgb, Wub, Wdb = _brute_quant_rows(Wg), _brute_quant_rows(Wu), _brute_quant_rows(Wd)  # dgrad
        for t in range(T):
            for j in range(k):
                if idx[t, j] != e:
                    continue
                gg = [sum(xq[t][h] * Wgf[h][i] for h in range(H)) for i in range(I)]
                uu = [sum(xq[t][h] * Wuf[h][i] for h in range(H)) for i in range(I)]
                hh = [gg[i] * sig(gg[i]) * uu[i] for i in range(I)]
                hq = _brute_quant_rows([hh])[0]
                y = [sum(hq[i] * Wdf[i][h] for i in range(I)) for h in range(H)]
                dy = [gw[t, j] * dout[t][h] for h in range(H)]
                dyq = _brute_quant_rows([dy])[0]
                dh = [sum(dyq[h] * Wdb[i][h] for h in range(H)) for i in range(I)]
                dg = [dh[i] * uu[i] * sig(gg[i]) * (1 + gg[i] * (1 - sig(gg[i]))) for i in range(I)]
                du = [dh[i] * gg[i] * sig(gg[i]) for i in range(I)]
                dgq, duq = _brute_quant_rows([dg])[0], _brute_quant_rows([du])[0]
                dx = [sum(dgq[i] * Wgb[h][i] + duq[i] * Wub[h][i] for i in range(I)) for h in range(H)]
                rows[(t, j)] = dict(x=x[t], g=gg, u=uu, h=hh, y=y, dy=dy, dg=dg, du=du, dx=dx, e=e)
    return rows


def test_mx_backward_matches_scalar_brute_force():
    """Every MXFP8 quantisation point of the layer, and every contraction, by
    scalar loops on a tiny layer: the forward (x along H; Wg, Wu along H; h
    along I; Wd along I), the input-gradient GEMMs (dY and Wd along H; dG, dU
    and Wg, Wu along I) and the unquantised weight gradients."""
    w = tiny(T=5, H=64, I=64, E=3, k=2, router_bias="normal", prec="mxfp8", wide_range=True)
    inp = make_inputs(w, with_dout=True)
    fwd = O.layer_forward(inp, keep=True)
    g = O.layer_backward(inp, fwd=fwd)
    T, H, I, E, k = w.T, w.H, w.I, w.E, w.k
    x = inp.x.double().tolist()
    dout = inp.dout.double().tolist()
    Wr = inp.Wr.double().tolist()
    idx, gw = fwd["idx"], fwd["w"]
    rows = _brute_mx_rows(inp, idx, gw)
    ref = {"dx": [[0.0] * H for _ in range(T)], "dWg": np.zeros((E, H, I)), "dWu": np.zeros((E, H, I)),
           "dWd": np.zeros((E, I, H)), "dgate": np.zeros((T, k)), "dWr": np.zeros((H, E)), "out": np.zeros((T, H))}
    for (t, j), r in rows.items():
        e = r["e"]
        ref["out"][t] += gw[t, j] * np.array(r["y"])
        ref["dgate"][t, j] = sum(dout[t][h] * r["y"][h] for h in range(H))
        for h in range(H):
            ref["dx"][t][h] += r["dx"][h]
            for i in range(I):
                ref["dWg"][e, h, i] += x[t][h] * r["dg"][i]
                ref["dWu"][e, h, i] += x[t][h] * r["du"][i]
                ref["dWd"][e, i, h] += r["h"][i] * r["dy"][h]
    for t in range(T):  # router: softmax over the selected logits
        s = sum(gw[t, j] * ref["dgate"][t, j] for j in range(k))
        for j in range(k):
            dl = gw[t, j] * (ref["dgate"][t, j] - s)
            e = idx[t, j]
            for h in range(H):
                ref["dx"][t][h] += dl * Wr[h][e]
                ref["dWr"][h, e] += x[t][h] * dl
    np.testing.assert_allclose(fwd["out"], ref["out"], rtol=1e-9, atol=1e-12)
    for n in ("dx", "dWg", "dWu", "dWd", "dgate", "dWr"):
        np.testing.assert_allclose(g[n], np.array(ref[n]), rtol=1e-9, atol=1e-12, err_msg=n)
    cols = [0, 17, 63]
    for e in range(E):
        c = O.weight_grad_columns(inp, e, cols)
        np.testing.assert_allclose(c["dWg"], ref["dWg"][e][:, cols], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(c["dWu"], ref["dWu"][e][:, cols], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(c["dWd"], ref["dWd"][e][cols, :], rtol=1e-9, atol=1e-12)


def _brute_quant_cols(M):
    """Quantise every column of the row list M along the rows, in blocks of 32
    rows from the first, a last partial block padded with zeros."""
    n = len(M)
    out = [[0.0] * len(M[0]) for _ in range(n)]
    for c in range(len(M[0])):
        for b in range(0, n, 32):
            blk = [M[r][c] for r in range(b, min(n, b + 32))]
            q = _brute_quant_block(blk + [0.0] * (32 - len(blk)))
            for r in range(len(blk)):
                out[b + r][c] = q[r]
    return out


def test_mx_weight_gradients_match_scalar_brute_force():
    """The MXFP8 weight-gradient GEMMs (all six routed GEMMs in MXFP8): their
    operands x, h, dY, dG, dU are quantised along the token rows of each
    (minibatch, expert) segment in blocks of 32 rows, zero-padded, by scalar
    loops here.  96 tokens, top-1 over 2 experts, minibatches of 80 and 16:
    the first minibatch's segments span two blocks, the second's one partial
    block; wide-range rows mix magnitudes along the quantised axis."""
    mb = 80
    w = tiny(T=96, H=64, I=64, E=2, k=1, router_bias="normal", prec="mxfp8", wide_range=True)
    inp = make_inputs(w, with_dout=True)
    fwd = O.layer_forward(inp, keep=True)
    g = O.layer_backward(inp, fwd=fwd, mx_wgrad_minibatch=mb)
    T, H, I, E = w.T, w.H, w.I, w.E
    idx, gw = fwd["idx"], fwd["w"]
    rows = _brute_mx_rows(inp, idx, gw)
    ref = {"dWg": np.zeros((E, H, I)), "dWu": np.zeros((E, H, I)), "dWd": np.zeros((E, I, H))}
    longest = 0
    for e in range(E):
        for t0 in range(0, T, mb):
            seg = [rows[(t, 0)] for t in range(t0, min(T, t0 + mb)) if idx[t, 0] == e]
            if not seg:
                continue
            longest = max(longest, len(seg))
            Xq = _brute_quant_cols([r["x"] for r in seg])
            dgq, duq = _brute_quant_cols([r["dg"] for r in seg]), _brute_quant_cols([r["du"] for r in seg])
            hq, dyq = _brute_quant_cols([r["h"] for r in seg]), _brute_quant_cols([r["dy"] for r in seg])
            ref["dWg"][e] += np.array(Xq).T @ np.array(dgq)
            ref["dWu"][e] += np.array(Xq).T @ np.array(duq)
            ref["dWd"][e] += np.array(hq).T @ np.array(dyq)
    assert longest > 32  # a segment spans more than one block
    for n in ref:
        np.testing.assert_allclose(g[n], ref[n], rtol=1e-9, atol=1e-12, err_msg=n)
        # the columns helper takes the same quantisation
    for e in range(E):
        c = O.weight_grad_columns(inp, e, [0, 33, 63], mx_wgrad_minibatch=mb)
        np.testing.assert_allclose(c["dWg"], ref["dWg"][e][:, [0, 33, 63]], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(c["dWd"], ref["dWd"][e][[0, 33, 63], :], rtol=1e-9, atol=1e-12)
    # the check is sensitive to the quantisation and to the segment restarts:
    # unquantised weight gradients, or one segment over all tokens (blocks
    # not restarting at the minibatch boundary), fail the same tolerance
    plain = O.layer_backward(inp, fwd=fwd)
    whole = O.layer_backward(inp, fwd=fwd, mx_wgrad_minibatch=T)
    for n in ref:
        assert O.rel_inf_err(plain[n], ref[n]) > 1e-3, n
        assert not np.allclose(whole[n], ref[n], rtol=1e-9, atol=1e-12), n


def test_mx_backward_with_identity_quantiser_is_the_plain_backward():
    w = tiny(T=24, H=128, I=64, E=4, k=2, shared_expert=True, router_bias="normal", prec="mxfp8")
    inp = make_inputs(w, with_dout=True)
    fwd = O.layer_forward(inp, keep=True, mx=False)
    plain = O.layer_backward(inp, fwd=fwd, mx=False)
    ident = O.layer_backward(inp, fwd=fwd, mx=True, quantizer=lambda a, axis: np.asarray(a, np.float64))
    for n in plain:
        np.testing.assert_array_equal(ident[n], plain[n], err_msg=n)


def test_mx_backward_scales_exactly_with_dout_and_stays_near_plain():
    w = tiny(T=32, H=128, I=64, E=4, k=2, router_bias="normal", prec="mxfp8")
    inp = make_inputs(w, with_dout=True)
    fwd = O.layer_forward(inp, keep=True)
    g1 = O.layer_backward(inp, fwd=fwd)
    g2 = O.layer_backward(inp, dout=2 * inp.dout, fwd=fwd)
    for n in ("dx", "dWg", "dWu", "dWd", "dWr", "dgate"):
        np.testing.assert_array_equal(g2[n], 2 * g1[n], err_msg=n)
    # E4M3 keeps 3 mantissa bits: per-operand relative error <= 2^-4, so the
    # quantised gradients stay within a few per cent of the unquantised ones
    plain = O.layer_backward(inp, fwd=O.layer_forward(inp, keep=True, mx=False), mx=False)
    for n in ("dx", "dWg", "dWu", "dWd"):
        assert 1e-4 < O.rel_inf_err(g1[n], plain[n]) < 0.15, n


# ------------------------------------------------------------ error metric

def test_rel_inf_err_hand_cases():
    """The metric behind every tolerance: max_i |got_i - ref_i| / max_i |ref_i|,
    over the whole tensor.  Each case is worked by hand and fails a plausible
    slip: a missing abs on the difference, a missing abs on the reference, a
    per-row instead of a global maximum, a mean instead of a maximum."""
    # |diff| = [0, 2], max |ref| = 4 (a negative entry): 0.5.  Without the abs
    # on the reference the denominator would be 1 (ratio 2); without the abs on
    # the difference the numerator would be 0.
    assert O.rel_inf_err([1.0, -6.0], [1.0, -4.0]) == 0.5
    # |diff| = [1, 2], max |ref| = 2: 1.0 (max(got - ref) alone would be -1)
    assert O.rel_inf_err([1.0, -3.0], [2.0, -1.0]) == 1.0
    # 2-D: the maxima run over every element, not row by row:
    # |diff| max = 0.5 (row 1), max |ref| = 8 (row 0): 1/16.  Row-wise ratios
    # would give 0.25 for row 1; the mean |diff| (0.125) over 8 would be 1/64.
    got = np.array([[8.0, 1.0], [2.0, 1.5]])
    ref = np.array([[8.0, 1.0], [2.0, 2.0]])
    assert O.rel_inf_err(got, ref) == 1.0 / 16.0
    # an all-zero reference divides by 1: the absolute error itself
    assert O.rel_inf_err([0.0, -0.25], [0.0, 0.0]) == 0.25
    assert O.rel_inf_err(np.zeros(3), np.zeros(3)) == 0.0
    # bf16 and fp32 inputs widen exactly before the difference is taken
    a = torch.tensor([1.0 + 2.0 ** -7], dtype=torch.bfloat16).float().numpy()
    assert O.rel_inf_err(a, np.array([1.0])) == 2.0 ** -7
