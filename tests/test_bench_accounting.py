"""CPU checks of bench.py's algorithmic-flop accounting per timing kind.

A grouped GEMM over M rows with an N x K weight costs 2*M*N*K flops, so one
routed or shared row costs 4*H*I in gate|up (N = 2I, K = H) and 2*H*I in down
(N = H, K = I) per pass; the backward repeats that for the input gradients and
again for the weight gradients.  Whatever kinds the launches are timed under,
every row's flops must be counted once and only once."""
import itertools

import pytest

import bench

T, H, I, K = 1000, 384, 192, 4
HI = float(H) * I


@pytest.mark.parametrize("shared,mx,bwd,layer,mxw", list(itertools.product([False, True], repeat=5)))
def test_every_row_counted_once(shared, mx, bwd, layer, mxw):
    f = bench.role_flops(T, H, I, K, shared, mx, bwd, layer, mxw)
    rows = T * K + (T if shared else 0)
    assert sum(f.values()) == (18 if bwd else 6) * HI * rows
    assert all(v > 0 for v in f.values())
    if layer:
        assert "gemm_gate_up" not in f and "gemm_down" not in f
        # the layer kernel runs every forward GEMM, the shared expert's
        # included, except in MXFP8 training, where the shared expert's two
        # bf16 GEMMs run as launches of their own before it
        assert f["layer"] == 6 * HI * (T * K if (mx and shared and bwd) else rows)
    else:
        assert "layer" not in f
    if bwd:
        # MXFP8 weight gradients: the routed rows on the scaled-MFMA kernel,
        # the shared expert's with its other bf16 GEMMs
        assert f["wgrad"] == 6 * HI * (T * K if (mx and mxw) else rows)


def test_mxfp8_shared_expert_kinds():
    # routed rows on the scaled-MFMA kernels; the shared expert's backward
    # input gradients are their own kind (bf16)
    f = bench.role_flops(T, H, I, K, True, True, True, True)
    assert f["dgrad_down"] == 2 * HI * T * K and f["dgrad_gate_up"] == 4 * HI * T * K
    # training: the shared expert's forward launches and its input gradients
    assert f["shared_gemm"] == 2 * 6 * HI * T
    # forward only, through the layer kernel: no shared-expert launches at all
    assert "shared_gemm" not in bench.role_flops(T, H, I, K, True, True, False, True)
    # forward only, one launch per GEMM: the shared expert's forward launches
    f = bench.role_flops(T, H, I, K, True, True, False, False)
    assert f["shared_gemm"] == 6 * HI * T
    assert f["gemm_gate_up"] == 4 * HI * T * K and f["gemm_down"] == 2 * HI * T * K


def test_bf16_runs_shared_rows_with_the_routed_ones():
    f = bench.role_flops(T, H, I, K, True, False, True, True)
    assert "shared_gemm" not in f
    assert f["dgrad_down"] == 2 * HI * (T * K + T) and f["dgrad_gate_up"] == 4 * HI * (T * K + T)


def test_data_movement_bytes():
    """Per token: combine reads k (+1 shared) bf16 rows of H and writes one;
    route reads the token's bf16 row once (plus the router weight once per
    step) and writes k indices and k weights; under MXFP8 it also writes the
    row's E4M3 codes and one E8M0 scale per 32 elements."""
    E = 8
    b = bench.role_bytes(T, H, I, K, E, False, False, False, False)
    assert b["combine"] == T * (K * H * 2 + H * 2)
    assert b["route"] == T * H * 2 + H * E * 4 + T * K * 8
    bm = bench.role_bytes(T, H, I, K, E, True, True, False, True)
    assert "combine" not in bm  # the layer kernel's combine is not timed on its own
    assert bm["route"] - b["route"] == T * H * (1 + 1 / 32)
    bb = bench.role_bytes(T, H, I, K, E, True, False, True, True)
    assert bb["combine"] == T * ((K + 1) * H * 2 + H * 2) and bb["gather"] > 0


def test_backward_gather_bytes():
    """Reverse-combine reads the dout row of every row and the Y row of every
    routed row; SwiGLU backward reads dH and g|u (fp32 under MXFP8) and writes
    row-major dG|dU and w*h for the rows whose weight gradients are bf16 (x
    and dout reach those GEMMs through the row map, with no copy).  Under
    MXFP8 the input-gradient GEMMs take codes + scales of dY and dG|dU for the
    routed rows (one code byte plus a 32nd of a scale byte per element); with
    MXFP8 weight gradients the routed rows' x rows are read as well, and dY,
    x, dG|dU and h are written transposed as codes + scales instead of the
    bf16 row-major dG|dU and w*h."""
    E, q = 8, 1 + 1 / 32
    R, Rr = T * (K + 1), T * K
    b = bench.role_bytes(T, H, I, K, E, True, False, True, True)
    assert b["gather"] == R * H * 2 + Rr * H * 2 + R * (3 * I * 2 + 3 * I * 2)
    bm = bench.role_bytes(T, H, I, K, E, True, True, True, True)
    assert bm["gather"] == (R * H * 2 + Rr * H * 2 + Rr * H * q
                            + R * (3 * I * 4 + 3 * I * 2) + Rr * 2 * I * q)
    bw = bench.role_bytes(T, H, I, K, E, True, True, True, True, True)
    assert bw["gather"] == (R * H * 2 + Rr * H * 2 + Rr * H * 2 + Rr * 2 * H * q + Rr * H * q
                            + R * 3 * I * 4 + T * 3 * I * 2 + Rr * 3 * I * q + Rr * 2 * I * q)
