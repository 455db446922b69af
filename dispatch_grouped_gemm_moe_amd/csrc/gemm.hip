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

// LDS ring of kStages pipeline stages; a stage holds the A tile [BM][BK] then
// the B tile [BN][BK] (bf16, BK = 32: 64-byte rows of four 16-byte chunks).
// Chunk c of row r sits at position c ^ f(r), f(r) = (r >> 2) & 3.  With this
// swizzle the 128-bit fragment reads (lane l: row l%32, chunk 2*kstep + l/32)
// are free of bank conflicts on gfx950's LDS; swizzles that also mix in row
// bit 1 (or use r & 3) measured 2-way conflicted with rocprofv3's
// SQ_LDS_BANK_CONFLICT, as did unswizzled rows.
constexpr int kBK = 32;
constexpr int kRowBytes = kBK * 2;
constexpr int kStageA = BM * kRowBytes;
constexpr int kStageBytes = (BM + BN) * kRowBytes;
constexpr int kStages = 5;  // 160 KB of LDS: loads run up to 4 K steps ahead

__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ void mfma_block(floatx16 (&acc)[4][4], const bf16x8 (&a)[4], const bf16x8 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// Wait until at most c K steps (8 loads each) of this wave are in flight and
// all of its LDS reads are done.  c is clamped to [0, kStages-1].
__device__ __forceinline__ void wait_vm_steps(int c) {
    switch (c < 0 ? 0 : c) {
        case 0: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(32) lgkmcnt(0)" ::: "memory"); break;
    }
}
static_assert(kStages <= 5, "wait_vm_steps covers at most 4 steps in flight");

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMFMA = 0x008, kSchedVMEM = 0x020, kSchedDSRead = 0x100;

// K sequence of a dense GEMM: K step kt sits kt * 64 bytes into every row.
struct DenseK {
    int kt = 0;
    __device__ __forceinline__ void next(int64_t& a_off, int64_t& b_off) {
        a_off = b_off = (int64_t)kt * kBK * 2;
        ++kt;
    }
};

// One 256 x 256 output tile: acc = A_tile * B_tile^T over KT K steps.
// a_base/b_base + aoff[i]/boff[i] address the 4 A and 4 B rows this lane
// stages (tile rows wave*64 + 16i + lane/4, swizzled chunk); kit.next() gives
// the byte offset of each successive K step, called in K order.
template <class KIt>
__device__ __forceinline__ void tile_mainloop(floatx16 (&acc)[4][4], uint8_t* smem, const char* a_base,
                                              const uint32_t (&aoff)[4], const char* b_base,
                                              const uint32_t (&boff)[4], int KT, KIt kit) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
    if (KT <= 0) return;

    auto issue = [&](int kt) {
        int64_t ka, kb;
        kit.next(ka, kb);
        uint8_t* base = smem + (kt % kStages) * kStageBytes + (wave * 64) * kRowBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((gbl_cvoid*)(a_base + ka + aoff[i]), (lds_void*)(base + i * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((gbl_cvoid*)(b_base + kb + boff[i]), (lds_void*)(base + kStageA + i * 1024), 16, 0, 0);
    };
    // MFMA operand fragments of k-step kk (16 deep) of K step kt.
    const int fr = lane & 31;
    const int arow_b = (wm * 128 + fr) * kRowBytes, brow_b = kStageA + (wn * 128 + fr) * kRowBytes;
    const int fsw = swz(fr);
    auto frags = [&](int kt, int kk, bf16x8 (&a)[4], bf16x8 (&b)[4]) {
        const uint8_t* st = smem + (kt % kStages) * kStageBytes;
        const int pc = ((kk * 2 + (lane >> 5)) ^ fsw) * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(st + arow_b + i * 32 * kRowBytes + pc);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = *(const bf16x8*)(st + brow_b + j * 32 * kRowBytes + pc);
    };

    // Ring protocol (S = kStages slots, K step j lives in slot j % S, each
    // step is 8 direct-to-LDS loads per lane, counted by vmcnt):
    //  - prologue: issue steps 0..min(S,KT)-1, wait for step 0;
    //  - K step kt: before the barrier wait for step kt+1, i.e. allow the
    //    c = min(KT-2-kt, S-2) newer steps in flight (vmcnt(8c)), and for this
    //    wave's own LDS reads of step kt (lgkmcnt(0)); after the barrier no
    //    wave reads step kt any more, so its slot takes step kt+S.
    // First the previous tile's stores leave the vmcnt count and every wave is
    // done reading the previous tile's stages.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kStages; ++j)
        if (j < KT) issue(j);
    wait_vm_steps(KT - 1 < kStages - 1 ? KT - 1 : kStages - 1);
    __syncthreads();
    bf16x8 a0[4], b0[4], a1[4], b1[4];
    frags(0, 0, a0, b0);
    for (int kt = 0; kt < KT; ++kt) {
        // k-step 0 of this K step: read k-step 1's fragments under 16 MFMAs
        frags(kt, 1, a1, b1);
        mfma_block(acc, a0, b0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 8, 0);
        __builtin_amdgcn_sched_barrier(0);
        // Every wave has read step kt (its reads done) and step kt+1 has
        // landed: refill step kt's slot with step kt+kStages and read step
        // kt+1's first fragments under the last 16 MFMAs.
        const int ahead = KT - 2 - kt;
        wait_vm_steps(ahead < kStages - 2 ? ahead : kStages - 2);
        __syncthreads();
        if (kt + kStages < KT) issue(kt + kStages);
        frags(kt + 1, 0, a0, b0);  // a stale but in-bounds read after the last step
        mfma_block(acc, a1, b1);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVMEM, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 8, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Accumulator element r of fragment (i, j) of lane l sits in tile row
// wm*128 + 32i + 8(r/4) + 4(l/32) + r%4 and tile column wn*128 + 32j + l%32.
__device__ __forceinline__ int frag_row(int i, int r) {
    const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) >> 1;
    return wm * 128 + i * 32 + (r >> 2) * 8 + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int frag_col(int j) {
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
    return wn * 128 + j * 32 + (lane & 31);
}

template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(kGemmThreads, kGemmThreads), amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int NT = ceil_div(p.N, BN);
    const int mt_lo = p.mt_start[p.e_begin];
    const int total = (p.mt_start[p.e_end] - mt_lo) * NT;
    const int G = gridDim.x, per = G >> 3;
    // Workgroups are dealt to the 8 XCDs round-robin; the 'per' workgroups of
    // one XCD take consecutive tiles so that they share weight and row tiles
    // in that XCD's L2.
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int KT = p.K / kBK;

    for (int it = 0;; ++it) {
        const int v = it * G + xcd * per + local;
        if (v >= total) break;
        // tile order: expert-major, then N tile, then M tile (M fastest)
        int lo = p.e_begin, hi = p.e_end - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((p.mt_start[mid] - mt_lo) * NT <= v) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int mt0 = p.mt_start[e], mte = p.mt_start[e + 1] - mt0;
        const int loc = v - (mt0 - mt_lo) * NT;
        const int ntile = loc / mte, ml = loc - ntile * mte;
        const int prow0 = (mt0 + ml) * BM;
        const int n0 = ntile * BN;

        // Byte offsets of the 4 A rows and 4 B rows this lane stages per K step:
        // instruction i fills tile rows wave*64 + 16i .. +15 (lane/4 picks the row,
        // lane%4 the fixed LDS chunk; the lane loads the logical chunk stored there).
        uint32_t aoff[4], boff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wave * 64 + i * 16 + (lane >> 2);
            const int lchunk = (lane & 3) ^ swz(r);
            const int prow = prow0 + r;
            const int arow = p.a_row_map ? p.a_row_map[prow] : prow;
            aoff[i] = (uint32_t)(((int64_t)arow * p.lda + lchunk * 8) * 2);
            const int n = min(n0 + r, p.N - 1);
            boff[i] = (uint32_t)(((int64_t)n * p.K + lchunk * 8) * 2);
        }
        floatx16 acc[4][4];
        tile_mainloop(acc, smem, (const char*)p.A, aoff, (const char*)(p.B + (int64_t)e * p.b_stride), boff, KT,
                      DenseK{});

        if (EPI == kEpiSwiGLU) {
            // columns come in 64-wide groups of 32 gate then 32 up columns
            const int I = p.N / 2;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int hcol = n0 / 2 + (wave & 1) * 64 + jj * 32 + (lane & 31);
                if (hcol < I) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float g = acc[i][2 * jj][r], u = acc[i][2 * jj + 1][r];
                            const float h = g / (1.0f + __expf(-g)) * u;
                            const int64_t row = prow0 + frag_row(i, r);
                            p.C[row * p.ldc + hcol] = f32_to_bf16_rne(h);
                            if (p.GUf) {
                                p.GUf[row * 2 * I + hcol] = g;
                                p.GUf[row * 2 * I + I + hcol] = u;
                            } else if (p.GU) {
                                p.GU[row * 2 * I + hcol] = f32_to_bf16_rne(g);
                                p.GU[row * 2 * I + I + hcol] = f32_to_bf16_rne(u);
                            }
                        }
                }
            }
        } else {  // kEpiStore
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + frag_col(j);
                if (col < p.N) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int64_t o = (int64_t)(prow0 + frag_row(i, r)) * p.ldc + col;
                            if (p.Cf)
                                p.Cf[o] = acc[i][j][r];
                            else
                                p.C[o] = f32_to_bf16_rne(acc[i][j][r]);
                        }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// weight gradients: C[e] = A_e^T-rows x B_e^T-rows over every routed row of
// expert e, minibatch by minibatch in order (a fixed summation order).
// ---------------------------------------------------------------------------

// K sequence of expert e's rows: for each minibatch b its padded row range
// [mt_b[e], mt_b[e+1]) x BM, in 32-row K steps; A and B copies of
// minibatch b lie a_mb / b_mb bytes after minibatch 0's.
struct SegmentK {
    const int32_t* mt;  // [nmb][mt_ld]
    int mt_ld, e, nmb;
    int64_t a_mb, b_mb;
    int b = 0, step = 0;
    __device__ __forceinline__ int steps_of(int bb) const {
        return (mt[(int64_t)bb * mt_ld + e + 1] - mt[(int64_t)bb * mt_ld + e]) * (BM / kBK);
    }
    __device__ __forceinline__ void next(int64_t& a_off, int64_t& b_off) {
        while (b < nmb && step >= steps_of(b)) { ++b; step = 0; }
        const int64_t kbyte = ((int64_t)mt[(int64_t)b * mt_ld + e] * BM + (int64_t)step * kBK) * 2;
        a_off = (int64_t)b * a_mb + kbyte;
        b_off = (int64_t)b * b_mb + kbyte;
        ++step;
    }
};

__global__ __attribute__((amdgpu_flat_work_group_size(kGemmThreads, kGemmThreads), amdgpu_waves_per_eu(1, 1)))
void wgrad_kernel(WgradArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int MT = ceil_div(p.M, BM), NT = ceil_div(p.N, BN);
    const int total = p.Et * MT * NT;
    const int G = gridDim.x, per = G >> 3;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    for (int it = 0;; ++it) {
        const int v = it * G + xcd * per + local;
        if (v >= total) break;
        // tile order: expert-major, then M tile, then N tile (N fastest)
        const int e = v / (MT * NT), loc = v - e * MT * NT;
        const int m0 = (loc / NT) * BM, n0 = (loc % NT) * BN;
        int KT = 0;
        for (int b = 0; b < p.nmb; ++b) KT += (p.mt[(int64_t)b * p.mt_ld + e + 1] - p.mt[(int64_t)b * p.mt_ld + e]) * (BM / kBK);
        uint32_t aoff[4], boff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wave * 64 + i * 16 + (lane >> 2);
            const int lchunk = (lane & 3) ^ swz(r);
            aoff[i] = (uint32_t)(((int64_t)min(m0 + r, p.M - 1) * p.ld + lchunk * 8) * 2);
            boff[i] = (uint32_t)(((int64_t)min(n0 + r, p.N - 1) * p.ld + lchunk * 8) * 2);
        }
        SegmentK kit{p.mt, p.mt_ld, e, p.nmb, p.a_mb, p.b_mb};
        floatx16 acc[4][4];
        tile_mainloop(acc, smem, (const char*)p.A, aoff, (const char*)p.B, boff, KT, kit);
        // columns < n_split go to C0, the rest to C1 (column - n_split); the
        // last expert writes to the shared-expert outputs when they are given
        const bool shared = p.Cs0 && e == p.Et - 1;
        float* c0 = shared ? p.Cs0 : p.C0 + (int64_t)e * p.M * p.n_split;
        float* c1 = shared ? p.Cs1 : (p.C1 ? p.C1 + (int64_t)e * p.M * (p.N - p.n_split) : nullptr);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + frag_col(j);
            if (col >= p.N) continue;
            float* dst = col < p.n_split ? c0 + col : c1 + (col - p.n_split);
            const int64_t ldc = col < p.n_split ? p.n_split : p.N - p.n_split;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + frag_row(i, r);
                    if (m < p.M) dst[(int64_t)m * ldc] = acc[i][j][r];
                }
        }
    }
}

void launch_wgrad(const WgradArgs& a, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(wgrad_kernel, dim3(grid), dim3(kGemmThreads), 0, stream, a);
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
