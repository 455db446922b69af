"""GPU check of the sustained-MFMA diagnostic (moe_diag_mfma_loop) through the
C ABI: with every operand 1.0 each accumulator element grows by K per matrix
instruction (16 for v_mfma_f32_32x32x16_bf16, 64 for the scaled
v_mfma_scale_f32_32x32x64_f8f6f4 with unit E8M0 scales), so every thread's
sum of its eight 16-element accumulators after iters x 4 instructions each is
the exact integer 8 * 16 * 4 * iters * K; zero operands give exactly zero.
The shader-clock and reference-tick counts must both be positive."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,one,K", [(0, 0x3F80, 16), (1, 0x38, 64)], ids=["bf16", "mxfp8"])
def test_diag_mfma_loop_exact_sums(gpu_lib, kind, one, K):
    moe = gpu_lib
    blocks, iters = 8, 16
    dtype = torch.int16 if kind == 0 else torch.uint8
    n = (1 << 15) if kind == 0 else (1 << 16)  # 64 KiB of operands
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    sink = torch.full((blocks * 512,), -1.0, dtype=torch.float32, device="cuda")
    ones = torch.full((n,), one, dtype=dtype, device="cuda")
    moe.moe_diag_mfma_loop(kind, ones, blocks, iters, clocks, sink)
    torch.cuda.synchronize()
    want = 8.0 * 16 * 4 * iters * K
    assert torch.all(sink == want), (sink.min().item(), sink.max().item(), want)
    cyc, ref = clocks.tolist()
    assert cyc > 0 and ref > 0
    zeros = torch.zeros_like(ones)
    moe.moe_diag_mfma_loop(kind, zeros, blocks, iters, clocks, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 0.0)
