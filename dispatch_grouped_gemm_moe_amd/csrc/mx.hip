// MXFP8 path of the MoE layer (gfx950): the quantiser and the scaled-MFMA
// grouped GEMMs.
//
// MoK runs its experts in MXFP8 and moves the quantisation into the dispatch,
// grouped-GEMM and SwiGLU data path instead of a separate quantize kernel
// (KuCoin flash "Cursor's MoK achieves 2.37x performance boost on NVIDIA
// GB300 NVL72", section 02; RuntimeWire "Cursor open-sources MoK",
// "Rebuilding the MoE layer around communication": production uses MXFP8).
// The format follows the OCP Microscaling v1.0 definitions: E4M3 elements and
// one E8M0 scale (bias 127) per 32 consecutive elements along the contraction
// axis; the scale is the smallest power of two 2^e with amax <= 448 * 2^e,
// elements are x / 2^e rounded to nearest even (the hardware conversion
// v_cvt_pk_fp8_f32, which saturates).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 takes, per lane, 32 E4M3 bytes of one row:
// bytes 0..15 are 16 values of the row's first 32-block of the K step and
// bytes 16..31 16 values of its second block (lanes 32..63 hold the other
// halves), and the E8M0 scale of (row m, block b) from lane m + 32 b.
#include "common.hpp"
#include "kernels.hpp"
#include "mxfp8.hpp"
#include "mx_tile.hpp"

namespace moe {


// ---------------------------------------------------------------------------
// quantiser: bf16 rows [rows][cols] -> E4M3 codes [rows][cols] + scales.
// scale layout 0: [rows][cols/32] bytes.  Layout 1: the GEMM operand scale
// layout [mx_groups(cols)][rows][4], byte b of group g the scale of block 4g + b.
// One thread per 32-element block; the thread of a row's last block also
// zeroes the bytes of its group past the row's end.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t* __restrict__ src, int64_t rows, int cols,
                                                       int layout, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, const LayoutHeader* hdr) {
    const int nb = cols / 32;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * nb) return;
    const int64_t r = i / nb;
    const int b = (int)(i - r * nb);
    if (hdr && r >= (int64_t)hdr->prows) return;  // rows past the minibatch's padded rows
    const uint8_t sc = mx_quant_block32(src + r * cols + b * 32, codes + r * cols + b * 32);
    if (layout == 0)
        scales[r * nb + b] = sc;
    else
        mx_store_scale_byte(scales, rows, r, b, nb, sc);
}

void launch_mx_quant(const uint16_t* src, int64_t rows, int cols, int layout, uint8_t* codes, uint8_t* scales,
                     hipStream_t stream, const LayoutHeader* hdr) {
    const int64_t n = rows * (cols / 32);
    hipLaunchKernelGGL(mx_quant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, src, rows, cols,
                       layout, codes, scales, hdr);
}

// ---------------------------------------------------------------------------
// scaled-MFMA grouped GEMM
// ---------------------------------------------------------------------------

template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(kTileThreads, kTileThreads), amdgpu_waves_per_eu(2, 2)))
void mx_gemm_kernel(MxGemmArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kMxSmem];
    const int NT = ceil_div(p.N, BN);
    const int total = launch_tiles(p);
    const int G = gridDim.x, per = G >> 3;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    for (int it = 0;; ++it) {
        int v = it * G + xcd * per + local;
        if (v >= total) break;
        MxGemmArgs q = p;
        if (p.nmb > 1) {
            const int b = minibatch_of_tile(p, v);
            q.mt_start += (int64_t)b * p.mt_ld;
            q.prow_start += (int64_t)b * p.mt_ld;
            if (q.rows_e) q.rows_e += (int64_t)b * p.mt_ld;
            if (!q.a_row_map) q.A += b * p.a_mb;
            q.SA += b * p.sa_mb;
            if (q.C) q.C += b * p.c_mb;
            if (q.Cf) q.Cf += b * p.c_mb;
        }
        int e, ml, ntile;
        tile_coords(q.mt_start, q.e_begin, q.e_end, NT, v, e, ml, ntile);
        mx_gemm_tile<EPI>(q, e, ml, ntile, smem);
    }
}

void launch_mx_gemm(const MxGemmArgs& a, GemmEpilogue epi, int grid, hipStream_t stream) {
    if (epi == kEpiSwiGLU)
        hipLaunchKernelGGL(mx_gemm_kernel<kEpiSwiGLU>, dim3(grid), dim3(kTileThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(mx_gemm_kernel<kEpiStore>, dim3(grid), dim3(kTileThreads), 0, stream, a);
}

}  // namespace moe
