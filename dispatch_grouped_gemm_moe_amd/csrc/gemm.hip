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
#include "kernels.hpp"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_cvoid;

// LDS of one pipeline stage: A tile [BM][BK] then B tile [BN][BK], bf16.
// A row of a tile is 128 bytes = eight 16-byte chunks; chunk c of row r is
// stored at position c ^ (r & 7), so the 32 rows an MFMA fragment read
// touches spread over all banks.
constexpr int kStageA = BM * BK * 2;
constexpr int kStageBytes = (BM + BN) * BK * 2;
constexpr int kStages = 2;

template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(kGemmThreads, kGemmThreads), amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int NT = ceil_div(p.N, BN);
    const int total = p.hdr->m_tiles * NT;
    const int G = gridDim.x, per = G >> 3;
    // Workgroups are dealt to the 8 XCDs round-robin; the 'per' workgroups of
    // one XCD take consecutive tiles so that they share weight and row tiles
    // in that XCD's L2.
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int KT = p.K / BK;
    const int lchunk = (lane & 7) ^ (lane >> 3);

    for (int it = 0;; ++it) {
        const int v = it * G + xcd * per + local;
        if (v >= total) break;
        // tile order: expert-major, then N tile, then M tile (M fastest)
        int lo = 0, hi = p.Et - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.mt_start[mid] * NT <= v) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int mt0 = p.mt_start[e], mte = p.mt_start[e + 1] - mt0;
        const int loc = v - mt0 * NT;
        const int ntile = loc / mte, ml = loc - ntile * mte;
        const int prow0 = (mt0 + ml) * BM;
        const int n0 = ntile * BN;

        const uint16_t* ga[8];
        const uint16_t* gb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = wave * 64 + i * 8 + (lane >> 3);
            const int prow = prow0 + r;
            const int arow = p.a_row_map ? p.a_row_map[prow] : prow;
            ga[i] = p.A + (int64_t)arow * p.lda + lchunk * 8;
            const int n = min(n0 + r, p.N - 1);
            gb[i] = p.B + (int64_t)e * p.b_stride + (int64_t)n * p.K + lchunk * 8;
        }

        floatx16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};

        auto issue = [&](int kt, int s) {
            const int koff = kt * BK;
            uint8_t* base = smem + s * kStageBytes + (wave * 64) * 128;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                __builtin_amdgcn_global_load_lds((gbl_cvoid*)(ga[i] + koff), (lds_void*)(base + i * 8 * 128), 16, 0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                __builtin_amdgcn_global_load_lds((gbl_cvoid*)(gb[i] + koff), (lds_void*)(base + kStageA + i * 8 * 128), 16, 0, 0);
        };

        __syncthreads();  // every wave is done reading the previous tile's stages
        issue(0, 0);
        for (int kt = 0; kt < KT; ++kt) {
            const int s = kt & 1;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (kt + 1 < KT) issue(kt + 1, s ^ 1);
            const uint8_t* As = smem + s * kStageBytes;
            const uint8_t* Bs = As + kStageA;
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                const int pc = (kk * 2 + (lane >> 5)) ^ (lane & 7);
                bf16x8 a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[i] = *(const bf16x8*)(As + (wm * 128 + i * 32 + (lane & 31)) * 128 + pc * 16);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    b[j] = *(const bf16x8*)(Bs + (wn * 128 + j * 32 + (lane & 31)) * 128 + pc * 16);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }

        // Epilogue.  Fragment element r of lane l sits at row 8*(r/4) + 4*(l/32) + r%4,
        // column l%32 of its 32x32 block.
        const int rbase = prow0 + wm * 128 + 4 * (lane >> 5);
        if (EPI == kEpiSwiGLU) {
            const int I = p.N / 2;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int hcol = n0 / 2 + wn * 64 + jj * 32 + (lane & 31);
                if (hcol < I) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float g = acc[i][2 * jj][r], u = acc[i][2 * jj + 1][r];
                            const float h = g / (1.0f + __expf(-g)) * u;
                            const int row = rbase + i * 32 + (r >> 2) * 8 + (r & 3);
                            p.C[(int64_t)row * p.ldc + hcol] = f32_to_bf16_rne(h);
                        }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn * 128 + j * 32 + (lane & 31);
                if (col < p.N) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int row = rbase + i * 32 + (r >> 2) * 8 + (r & 3);
                            p.C[(int64_t)row * p.ldc + col] = f32_to_bf16_rne(acc[i][j][r]);
                        }
                }
            }
        }
    }
}

void launch_grouped_gemm(const GemmArgs& a, GemmEpilogue epi, int grid, hipStream_t stream) {
    if (epi == kEpiSwiGLU)
        hipLaunchKernelGGL(grouped_gemm_kernel<kEpiSwiGLU>, dim3(grid), dim3(kGemmThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(grouped_gemm_kernel<kEpiStore>, dim3(grid), dim3(kGemmThreads), 0, stream, a);
}

// ---------------------------------------------------------------------------
// combine: one workgroup per token, 8 hidden elements per thread per step
// ---------------------------------------------------------------------------

constexpr int kCombineThreads = 128;

__device__ __forceinline__ void bf16x8_to_f32(const intx4 raw, float* f) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = (uint32_t)raw[q];
        f[2 * q] = __builtin_bit_cast(float, v << 16);
        f[2 * q + 1] = __builtin_bit_cast(float, v & 0xffff0000u);
    }
}

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint16_t* __restrict__ Y, int64_t ldy, const int32_t* __restrict__ tok_prow, int ld,
    const float* __restrict__ w, int k, int with_shared, int H, uint16_t* __restrict__ out) {
    __shared__ int s_row[kMaxTopK + 1];
    __shared__ float s_w[kMaxTopK];
    const int t = blockIdx.x;
    if ((int)threadIdx.x < k + with_shared) s_row[threadIdx.x] = tok_prow[(int64_t)t * ld + threadIdx.x];
    if ((int)threadIdx.x < k) s_w[threadIdx.x] = w[(int64_t)t * k + threadIdx.x];
    __syncthreads();
    for (int c = threadIdx.x; c < H / 8; c += kCombineThreads) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        for (int j = 0; j < k; ++j) {
            float y[8];
            bf16x8_to_f32(*(const intx4*)(Y + (int64_t)s_row[j] * ldy + c * 8), y);
            const float wj = s_w[j];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(wj, y[q], acc[q]);
        }
        if (with_shared) {
            float y[8];
            bf16x8_to_f32(*(const intx4*)(Y + (int64_t)s_row[k] * ldy + c * 8), y);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = acc[q] + y[q];
        }
        intx4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = (int)((uint32_t)f32_to_bf16_rne(acc[2 * q]) | ((uint32_t)f32_to_bf16_rne(acc[2 * q + 1]) << 16));
        *(intx4*)(out + (int64_t)t * H + c * 8) = o;
    }
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
    if (prow >= hdr->m_tiles * BM) return;
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
