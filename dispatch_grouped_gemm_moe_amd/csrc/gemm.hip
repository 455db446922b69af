// Grouped GEMM (bf16 MFMA), combine, dispatch gather and weight packing.
//
// Every expert's FFN runs as one grouped GEMM over the expert-contiguous rows
// the layout produced (KuCoin flash "Cursor's MoK achieves 2.37x performance
// boost on NVIDIA GB300 NVL72", section 01: grouped GEMM needs each expert's
// tokens adjacent; section 02: the FFN is SwiGLU).  The first GEMM gathers
// its A rows straight from the token matrix into LDS tiles (the dispatch
// gather of the one-GPU layer) and applies SwiGLU in registers; the second is
// the down projection.  Combine then forms the weighted sum of every token's
// expert outputs back in token order (same page, sections 02-03), in slot
// order with fp32 fused multiply-adds, so the result is bitwise reproducible.
#include "common.hpp"
#include "gemm_tile.hpp"
#include "kernels.hpp"

namespace moe {

template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(kTileThreads, kTileThreads), amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kTileSmem];
    const int NT = ceil_div(p.N, BN);
    const int total = launch_tiles(p);
    const int G = gridDim.x, per = G >> 3;
    // Workgroups are dealt to the 8 XCDs round-robin; the 'per' workgroups of
    // one XCD take consecutive tiles so that they share weight and row tiles
    // in that XCD's L2.
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    for (int it = 0;; ++it) {
        int v = it * G + xcd * per + local;
        if (v >= total) break;
        GemmArgs q = p;
        if (p.nmb > 1) {
            const int b = minibatch_of_tile(p, v);
            q.mt_start += (int64_t)b * p.mt_ld;
            q.prow_start += (int64_t)b * p.mt_ld;
            if (q.rows_e) q.rows_e += (int64_t)b * p.mt_ld;
            if (q.a_row_map) q.a_row_map += b * p.map_mb;
            else q.A += b * p.a_mb;
            if (q.row_scale) q.row_scale += b * p.rs_mb;
            if (q.C) q.C += b * p.c_mb;
            if (q.Cf) q.Cf += b * p.c_mb;
        }
        int e, ml, ntile;
        tile_coords(q.mt_start, q.e_begin, q.e_end, NT, v, e, ml, ntile);
        gemm_tile<EPI>(q, e, ml, ntile, smem);
    }
}

// ---------------------------------------------------------------------------
// weight gradients: C[e] = A_e^T-rows x B_e^T-rows over every routed row of
// expert e, minibatch by minibatch in order (a fixed summation order).
// ---------------------------------------------------------------------------

// K sequence of expert e's rows: for each minibatch b its padded rows from
// prs_b[e] on, in 64-row K stages up to the last one holding a routed row
// (the dY-side operand is zero on every padding row, so the padding rows a
// stage takes in add nothing); A and B copies of minibatch b lie a_mb / b_mb
// bytes after minibatch 0's.
struct SegmentK {
    const int32_t* prs;   // [nmb][mt_ld] first padded row of each expert
    const int32_t* rows;  // [nmb][mt_ld]
    int mt_ld, e, nmb;
    int64_t a_mb, b_mb;
    // current minibatch, K step within it, its step count and first row: the
    // tile map is read only when the sequence enters the next minibatch
    int b = -1, step = 0, nsteps = 0;
    int64_t row0 = 0;
    __device__ __forceinline__ void next(int64_t& a_off, int64_t& b_off) {
        while (step >= nsteps && b + 1 < nmb) {
            ++b;
            // the tile map is read-only here: read it through the constant
            // address space (scalar loads, counted by lgkmcnt) so that the
            // ring's vmcnt accounting sees only the ring's own loads
            const __attribute__((address_space(4))) int32_t* cprs =
                (const __attribute__((address_space(4))) int32_t*)prs;
            const __attribute__((address_space(4))) int32_t* crows =
                (const __attribute__((address_space(4))) int32_t*)rows;
            row0 = cprs[(int64_t)b * mt_ld + e];
            nsteps = ceil_div(crows[(int64_t)b * mt_ld + e], kBK8);
            step = 0;
        }
        const int64_t kbyte = (row0 + (int64_t)step * kBK8) * 2;
        a_off = (int64_t)b * a_mb + kbyte;
        b_off = (int64_t)b * b_mb + kbyte;
        ++step;
    }
};

__global__ __attribute__((amdgpu_flat_work_group_size(kTileThreads, kTileThreads), amdgpu_waves_per_eu(2, 2)))
void wgrad_kernel(WgradArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kTileSmem];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const WgradTiles tiles(p.M, p.N, p.mq, p.nq);
    int e, m0, n0;
    for (int it = 0; tiles.get(it, p.Et - p.e_begin, e, m0, n0); ++it) {
        e += p.e_begin;
        int KT = 0;
        for (int b = 0; b < p.nmb; ++b) KT += ceil_div(p.rows[(int64_t)b * p.mt_ld + e], kBK8);
        uint32_t aoff[4], boff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wave * 32 + i * 8 + (lane >> 3);
            const int lchunk = (lane & 7) ^ swz8(r);
            aoff[i] = (uint32_t)(((int64_t)min(m0 + r, p.M - 1) * p.ld + lchunk * 8) * 2);
            boff[i] = (uint32_t)(((int64_t)min(n0 + r, p.N - 1) * p.ld + lchunk * 8) * 2);
        }
        SegmentK kit{p.prs, p.rows, p.mt_ld, e, p.nmb, p.a_mb, p.b_mb};
        floatx16 acc[2][4];
        tile_mainloop8<2>(acc, smem, (const char*)p.A, aoff, (const char*)p.B, boff, KT, kit);
        // columns < n_split go to C0, the rest to C1 (column - n_split); the
        // last expert writes to the shared-expert outputs when they are given
        const bool shared = p.Cs0 && e == p.Et - 1;
        float* c0 = shared ? p.Cs0 : p.C0 + (int64_t)e * p.M * p.n_split;
        float* c1 = shared ? p.Cs1 : (p.C1 ? p.C1 + (int64_t)e * p.M * (p.N - p.n_split) : nullptr);
        wgrad_store(acc, m0, n0, p.M, p.N, p.n_split, c0, c1);
    }
}

void launch_wgrad(const WgradArgs& a, int grid, hipStream_t stream) {
    WgradArgs w = a;
    wgrad_cut(a.M, a.N, w.mq, w.nq);
    hipLaunchKernelGGL(wgrad_kernel, dim3(grid), dim3(kTileThreads), 0, stream, w);
}

void launch_grouped_gemm(const GemmArgs& a, GemmEpilogue epi, int grid, hipStream_t stream) {
    if (epi == kEpiSwiGLU)
        hipLaunchKernelGGL(grouped_gemm_kernel<kEpiSwiGLU>, dim3(grid), dim3(kTileThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(grouped_gemm_kernel<kEpiStore>, dim3(grid), dim3(kTileThreads), 0, stream, a);
}

// ---------------------------------------------------------------------------
// combine: one workgroup per token, 8 hidden elements per thread per step
// ---------------------------------------------------------------------------

constexpr int kCombineThreads = 128;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint16_t* __restrict__ Y, int64_t ldy, const int32_t* __restrict__ tok_prow, int ld,
    const float* __restrict__ w, int k, int with_shared, int H, uint16_t* __restrict__ out) {
    __shared__ int s_row[kMaxTopK + 1];
    __shared__ float s_w[kMaxTopK];
    const int t = blockIdx.x;
    if ((int)threadIdx.x < k + with_shared) s_row[threadIdx.x] = tok_prow[(int64_t)t * ld + threadIdx.x];
    if ((int)threadIdx.x < k) s_w[threadIdx.x] = w[(int64_t)t * k + threadIdx.x];
    __syncthreads();
    combine_token(Y, ldy, s_row, s_w, k, with_shared, H, out + (int64_t)t * H, threadIdx.x, kCombineThreads);
}

void launch_combine(const uint16_t* Y, int64_t ldy, const int32_t* tok_prow, int tok_prow_ld,
                    const float* w, int k, int with_shared, int H, int Tm, uint16_t* out,
                    hipStream_t stream) {
    hipLaunchKernelGGL(combine_kernel, dim3(Tm), dim3(kCombineThreads), 0, stream, Y, ldy, tok_prow,
                       tok_prow_ld, w, k, with_shared, H, out);
}

// ---------------------------------------------------------------------------
// dispatch gather of whole rows (identity-expert mode)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x, int H,
                                                          const int32_t* __restrict__ prow_token,
                                                          const LayoutHeader* __restrict__ hdr,
                                                          uint16_t* __restrict__ Y, int64_t ldy) {
    const int prow = blockIdx.x;
    if (prow >= hdr->prows) return;
    const int64_t src = (int64_t)prow_token[prow] * H;
    for (int c = threadIdx.x; c < H / 8; c += 256)
        *(intx4*)(Y + (int64_t)prow * ldy + c * 8) = *(const intx4*)(x + src + c * 8);
}

void launch_gather_rows(const uint16_t* x, int H, const int32_t* prow_token, const LayoutHeader* hdr,
                        int max_rows, uint16_t* Y, int64_t ldy, hipStream_t stream) {
    hipLaunchKernelGGL(gather_rows_kernel, dim3(max_rows), dim3(256), 0, stream, x, H, prow_token, hdr,
                       Y, ldy);
}

// ---------------------------------------------------------------------------
// weight packing
// ---------------------------------------------------------------------------

// W1t[e][64q + c][h]: c < 32 -> Wg[e][h][32q + c], c >= 32 -> Wu[e][h][32q + c - 32].
// One workgroup moves a 64 (packed rows) x 64 (h) tile through LDS.
__global__ __launch_bounds__(256) void pack_gate_up_kernel(const uint16_t* __restrict__ Wg,
                                                           const uint16_t* __restrict__ Wu, int H, int I,
                                                           uint16_t* __restrict__ W1t) {
    __shared__ uint16_t tile[64][65];
    const int h0 = blockIdx.x * 64, q = blockIdx.y, e = blockIdx.z;
    const int64_t src_e = (int64_t)e * H * I;
    for (int f = threadIdx.x; f < 64 * 64; f += 256) {
        const int hr = f >> 6, c = f & 63;
        const uint16_t* src = (c < 32) ? Wg : Wu;
        tile[hr][c] = src[src_e + (int64_t)(h0 + hr) * I + 32 * q + (c & 31)];
    }
    __syncthreads();
    const int64_t dst_e = (int64_t)e * 2 * I * H;
    for (int f = threadIdx.x; f < 64 * 64; f += 256) {
        const int c = f >> 6, hr = f & 63;
        W1t[dst_e + (int64_t)(64 * q + c) * H + h0 + hr] = tile[hr][c];
    }
}

void launch_pack_gate_up(const uint16_t* Wg, const uint16_t* Wu, int E, int H, int I, uint16_t* W1t,
                         hipStream_t stream) {
    hipLaunchKernelGGL(pack_gate_up_kernel, dim3(H / 64, I / 32, E), dim3(256), 0, stream, Wg, Wu, H, I,
                       W1t);
}

// dst[b][c][r] = src[b][r][c]; rows and cols multiples of 64.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src, int rows,
                                                        int cols, uint16_t* __restrict__ dst) {
    __shared__ uint16_t tile[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const int64_t boff = (int64_t)blockIdx.z * rows * cols;
    for (int f = threadIdx.x; f < 64 * 64; f += 256) {
        const int r = f >> 6, c = f & 63;
        tile[r][c] = src[boff + (int64_t)(r0 + r) * cols + c0 + c];
    }
    __syncthreads();
    for (int f = threadIdx.x; f < 64 * 64; f += 256) {
        const int c = f >> 6, r = f & 63;
        dst[boff + (int64_t)(c0 + c) * rows + r0 + r] = tile[r][c];
    }
}

void launch_transpose(const uint16_t* src, int batches, int rows, int cols, uint16_t* dst,
                      hipStream_t stream) {
    hipLaunchKernelGGL(transpose_kernel, dim3(cols / 64, rows / 64, batches), dim3(256), 0, stream, src,
                       rows, cols, dst);
}

}  // namespace moe
