// Sustained matrix-core rate of the chip under a pure MFMA load.
//
// The layer's grouped GEMMs are priced against the published bf16 peak
// (256 CUs x 2.4 GHz x 4096 flop/clk).  Under a dense MFMA load the chip
// lowers its shader clock to stay within its power budget, and how far it
// lowers it depends on the operand bits (random mantissas switch more logic
// than zeros).  This kernel measures that ceiling: one workgroup of eight
// waves per CU, each wave issuing independent v_mfma_f32_32x32x16_bf16 on
// eight accumulators with operands taken from the caller's buffer (so the
// caller chooses the data), no memory traffic inside the loop, and the shader
// clock read with s_memtime against the 100 MHz s_memrealtime over the loop.
#include "common.hpp"

#include "../../include/moe.h"

namespace moe {

constexpr int kDiagThreads = 512;

// MX: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes with unit E8M0 scales
// (131072 flops each) instead of v_mfma_f32_32x32x16_bf16 (32768 flops).
template <bool MX>
__global__ __attribute__((amdgpu_flat_work_group_size(kDiagThreads, kDiagThreads), amdgpu_waves_per_eu(2, 2)))
void mfma_loop_kernel(const intx4* __restrict__ operands, int64_t n16, int iters, uint64_t* clocks, float* sink) {
    // every lane takes four 16-byte pieces of the buffer (n16 >= 1024 entries)
    const int64_t g = ((int64_t)blockIdx.x * kDiagThreads + threadIdx.x) * 4;
    const intx4 p0 = operands[g % n16], p1 = operands[(g + 1) % n16];
    const intx4 p2 = operands[(g + 2) % n16], p3 = operands[(g + 3) % n16];
    floatx16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = floatx16{};
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    if constexpr (MX) {
        const intx8 a = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        const intx8 b = {p2[0], p2[1], p2[2], p2[3], p3[0], p3[1], p3[2], p3[3]};
        const int unit = 0x7f7f7f7f;  // E8M0 127 = 2^0
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, unit, 0, unit);
        }
    } else {
        const bf16x8 a = __builtin_bit_cast(bf16x8, p0), b = __builtin_bit_cast(bf16x8, p1);
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) s += acc[j][q];
    sink[blockIdx.x * kDiagThreads + threadIdx.x] = s;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clocks[0] = t1 - t0;
        clocks[1] = r1 - r0;
    }
}

}  // namespace moe

extern "C" moe_status moe_diag_mfma_loop(int32_t kind, const void* operands, int64_t operand_bytes, int32_t blocks,
                                         int32_t iters, uint64_t* clocks, float* sink, void* stream) {
    if (kind != 0 && kind != 1) return MOE_E_INVALID;
    if (!operands || !clocks || !sink) return MOE_E_INVALID;
    if (((uintptr_t)operands & 15) || ((uintptr_t)clocks & 7) || ((uintptr_t)sink & 3)) return MOE_E_INVALID;
    if (operand_bytes < 16 * 1024 || blocks < 1 || blocks > 65536 || iters < 1) return MOE_E_INVALID;
    const moe::intx4* ops = (const moe::intx4*)operands;
    if (kind == 1)
        hipLaunchKernelGGL(moe::mfma_loop_kernel<true>, dim3(blocks), dim3(moe::kDiagThreads), 0, (hipStream_t)stream,
                           ops, operand_bytes / 16, iters, clocks, sink);
    else
        hipLaunchKernelGGL(moe::mfma_loop_kernel<false>, dim3(blocks), dim3(moe::kDiagThreads), 0, (hipStream_t)stream,
                           ops, operand_bytes / 16, iters, clocks, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}
