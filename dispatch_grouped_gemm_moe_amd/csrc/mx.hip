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
    // plain-store tiles chain (the ring plus the staging block past it)
    constexpr bool kChain = EPI == kEpiStore;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kChain ? kMxSmem + kMxStgBytes : kMxSmem];
    const int NT = ceil_div(p.N, BN);
    const int total = launch_tiles(p);
    const int G = gridDim.x, per = G >> 3;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    // tile v: its minibatch's arguments and its coordinates
    auto tile_of = [&](int v, MxGemmArgs& q, int& e, int& ml, int& ntile) {
        q = p;
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
        tile_coords(q.mt_start, q.e_begin, q.e_end, NT, v, e, ml, ntile);
    };
    const bool chain = kChain && mx_tiles_chain(p);
    TileEntry en;
    for (int it = 0;; ++it) {
        const int v = it * G + xcd * per + local;
        if (v >= total) break;
        MxGemmArgs q;
        int e, ml, ntile;
        tile_of(v, q, e, ml, ntile);
        if constexpr (kChain) {
            MxLink ln;
            if (chain && v + G < total) {
                MxGemmArgs qn;
                int e2, ml2, nt2;
                tile_of(v + G, qn, e2, ml2, nt2);
                ln = mx_tile_link(q, e, ml, ntile, qn, e2, ml2, nt2);
            }
            mx_gemm_tile<EPI, kPadPerWave, true>(q, e, ml, ntile, smem, &en, &ln);
        } else {
            mx_gemm_tile<EPI>(q, e, ml, ntile, smem);
        }
    }
}

void launch_mx_gemm(const MxGemmArgs& a, GemmEpilogue epi, int grid, hipStream_t stream) {
    if (epi == kEpiSwiGLU)
        hipLaunchKernelGGL(mx_gemm_kernel<kEpiSwiGLU>, dim3(grid), dim3(kTileThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(mx_gemm_kernel<kEpiStore>, dim3(grid), dim3(kTileThreads), 0, stream, a);
}

// ---------------------------------------------------------------------------
// MXFP8 weight gradients: C[e] = A_e^T B_e, the contraction running over the
// padded rows of expert e's segments, minibatch by minibatch in order (a fixed
// summation order).  Both operands are stored transposed ([M][ld] and [N][ld]
// codes, the padded rows along each row), quantised along those rows in
// 32-row blocks, so a 128-row stage is one scale dword per operand row (the
// operand scale layout's group), as in the forward tiles.  Segments start at
// multiples of 128 rows and their padding rows are zero codes, so every stage
// lies inside one segment and its padding adds nothing.
// ---------------------------------------------------------------------------

// Stage sequence of expert e: for each minibatch b the 128-row stages from
// its segment's first padded row up to the last one holding a routed row.
struct MxSegK {
    const int32_t* prs;   // [nmb][mt_ld]
    const int32_t* rows;  // [nmb][mt_ld]
    int mt_ld, e, nmb;
    int b = -1, step = 0, nsteps = 0;
    int64_t row0 = 0;
    __device__ __forceinline__ void next(int& bo, int64_t& r) {
        while (step >= nsteps && b + 1 < nmb) {
            ++b;
            // read through the constant address space (scalar loads, counted by
            // lgkmcnt): the ring's vmcnt accounting sees only its own loads
            const __attribute__((address_space(4))) int32_t* cprs =
                (const __attribute__((address_space(4))) int32_t*)prs;
            const __attribute__((address_space(4))) int32_t* crows =
                (const __attribute__((address_space(4))) int32_t*)rows;
            row0 = cprs[(int64_t)b * mt_ld + e];
            nsteps = ceil_div(crows[(int64_t)b * mt_ld + e], 128);
            step = 0;
        }
        bo = b;
        r = row0 + (int64_t)step * 128;
        ++step;
    }
};

__global__ __attribute__((amdgpu_flat_work_group_size(kTileThreads, kTileThreads), amdgpu_waves_per_eu(2, 2)))
void mx_wgrad_kernel(MxWgradArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kMxSmem];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS bases
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 31, half = lane >> 5;
    const int fsw = swz8(fr);  // a fragment's rows differ from fr by multiples of 32
    const int arow_b = (wm * 32 + fr) * kMxRow, brow_b = kMxStageA + (wn * 128 + fr) * kMxRow;
    const WgradTiles tiles(p.M, p.N, p.mq, p.nq);
    int e, m0, n0;
    for (int it = 0; tiles.get(it, p.E, e, m0, n0); ++it) {
        int KS = 0;
        for (int b = 0; b < p.nmb; ++b) KS += ceil_div(p.rows[(int64_t)b * p.mt_ld + e], 128);
        floatx16 acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
        if (KS > 0) {
            // Code loads: instruction i fills tile rows 32*wave + 8i .. +7 of
            // the A and of the B block (lane/8 the row, lane%8 the fixed LDS
            // chunk, loading the logical chunk stored there; chunks 4..7 hold
            // the stage's second 64-row K step).  Scale load: waves 0..3 take
            // the dwords of A rows 64*wave + lane, waves 4..7 those of B rows
            // 64*(wave-4) + lane, landing as the stage's SA and SB arrays.
            uint32_t aoff[4], boff[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wave * 32 + i * 8 + (lane >> 3);
                const int lchunk = (lane & 7) ^ swz8(r);
                aoff[i] = (uint32_t)((int64_t)min(m0 + r, p.M - 1) * p.ld + lchunk * 16);
                boff[i] = (uint32_t)((int64_t)min(n0 + r, p.N - 1) * p.ld + lchunk * 16);
            }
            // per lane: 32-bit offsets; per stage: uniform bases (minibatch,
            // stage row) in scalar registers
            const int srow = (wave & 3) * 64 + lane;
            const bool bscale = wave >= 4;
            const uint32_t soff = (uint32_t)(bscale ? min(n0 + srow, p.N - 1) : min(m0 + srow, p.M - 1)) * 4;
            const uint8_t* s_ptr = bscale ? p.SB : p.SA;
            const int64_t s_group = (int64_t)(bscale ? p.N : p.M) * 4;  // scale bytes per 128 rows
            const int64_t s_mb = bscale ? p.sb_mb : p.sa_mb;
            MxSegK kit{p.prs, p.rows, p.mt_ld, e, p.nmb};
            const uint8_t* abase = p.A;
            const uint8_t* bbase = p.B;
            const uint8_t* sbase = s_ptr;
            uint32_t kr = 0;
            int issued = 0;
            // stage `issued` into `slot`; past the last stage the loads repeat
            // it into the slot no wave reads any more (constant waits)
            auto issue = [&](int slot) {
                if (issued < KS) {
                    int b;
                    int64_t r;
                    kit.next(b, r);
                    abase = p.A + b * p.a_mb;
                    bbase = p.B + b * p.b_mb;
                    sbase = s_ptr + b * s_mb + (r >> 7) * s_group;
                    kr = (uint32_t)r;
                }
                ++issued;
                uint8_t* st = smem + slot * kMxStageBytes;
                uint8_t* base = st + (wave * 32) * kMxRow;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_global_load_lds((gbl_cvoid*)(abase + (aoff[i] + kr)), (lds_void*)(base + i * 1024),
                                                     16, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_global_load_lds((gbl_cvoid*)(bbase + (boff[i] + kr)),
                                                     (lds_void*)(base + kMxStageA + i * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((gbl_cvoid*)(sbase + soff), (lds_void*)(st + kMxStageSA + wave * 256),
                                                 4, 0, 0);
            };
            // fragments of K step ks of the stage in `slot` (as the forward
            // tiles: bytes 0..15 from the first 32-block of the K step, 16..31
            // from the second; with ks = 0 also the scale dwords, shifted so
            // that byte 2 * ks is this lane's block scale)
            auto read_a = [&](int slot, int ks, int i, intx8& a, int& sa) {
                const uint8_t* st = smem + slot * kMxStageBytes;
                const int pc0 = ((4 * ks + half) ^ fsw) * 16, pc1 = ((4 * ks + 2 + half) ^ fsw) * 16;
                const intx4 lo4 = *(const intx4*)(st + arow_b + i * 128 * kMxRow + pc0);
                const intx4 hi4 = *(const intx4*)(st + arow_b + i * 128 * kMxRow + pc1);
                a = intx8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                if (ks == 0)
                    sa = (int)(*(const uint32_t*)(st + kMxStageSA + (i * 128 + wm * 32 + fr) * 4) >> (8 * half));
            };
            auto read_b = [&](int slot, int ks, int j, intx8& b, int& sb) {
                const uint8_t* st = smem + slot * kMxStageBytes;
                const int pc0 = ((4 * ks + half) ^ fsw) * 16, pc1 = ((4 * ks + 2 + half) ^ fsw) * 16;
                const intx4 lo4 = *(const intx4*)(st + brow_b + j * 32 * kMxRow + pc0);
                const intx4 hi4 = *(const intx4*)(st + brow_b + j * 32 * kMxRow + pc1);
                b = intx8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                if (ks == 0)
                    sb = (int)(*(const uint32_t*)(st + kMxStageSB + (wn * 128 + j * 32 + fr) * 4) >> (8 * half));
            };
            // MFMAs of K step ksc on the fragments in registers, each B
            // fragment's registers taking fragment j of K step rks of the stage
            // in rslot as soon as its last MFMA is issued, the A fragments last
            auto mfmas_then = [&](auto ksc_, int rslot, int rks, intx8(&a)[2], intx8(&b)[4], int(&sa)[2],
                                  int(&sb)[4]) {
                constexpr int sel = 2 * decltype(ksc_)::value;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0, sel,
                                                                                     sb[j], sel, sa[i]);
                    read_b(rslot, rks, j, b[j], sb[j]);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) read_a(rslot, rks, i, a[i], sa[i]);
            };
            // Ring (stage j in slot j % 2, 9 direct-to-LDS loads per lane and
            // stage): the prologue issues stages 0 and 1, waits for stage 0 and
            // reads its first K step.  Stage s runs its first K step while
            // reading its second, waits for stage s+1 and its own LDS reads,
            // barrier, refills its slot with stage s+2 and runs its second K
            // step while reading stage s+1's first.  Every stage is full.
            // (the previous tile's stores may still be in flight: the vmcnt
            // waits count them too, and only ever wait longer for them)
            static_assert(kMxStages == 2, "the vmcnt immediates below assume 2 stages of 9 loads");
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();
            issue(0);
            issue(1);
            asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
            __syncthreads();
            intx8 fa[2], fb[4];
            int fsa[2], fsb[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) read_a(0, 0, i, fa[i], fsa[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j) read_b(0, 0, j, fb[j], fsb[j]);
            int slot = 0;
            for (int s = 0; s < KS; ++s) {
                mfmas_then(std::integral_constant<int, 0>{}, slot, 1, fa, fb, fsa, fsb);
                Interleave<8, 0, 12>::run();
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
                __syncthreads();
                issue(slot);
                // the last stage reads a stale but in-bounds repeat that nothing uses
                mfmas_then(std::integral_constant<int, 1>{}, slot ^ 1, 0, fa, fb, fsa, fsb);
                Interleave<8, 9, 12>::run();
                __builtin_amdgcn_sched_barrier(0);
                slot ^= 1;
            }
        }
        float* c0 = p.C0 + (int64_t)e * p.M * p.n_split;
        float* c1 = p.C1 ? p.C1 + (int64_t)e * p.M * (p.N - p.n_split) : nullptr;
        wgrad_store(acc, m0, n0, p.M, p.N, p.n_split, c0, c1);
    }
}

void launch_mx_wgrad(const MxWgradArgs& a, int grid, hipStream_t stream) {
    MxWgradArgs w = a;
    wgrad_cut(a.M, a.N, w.mq, w.nq);
    hipLaunchKernelGGL(mx_wgrad_kernel, dim3(grid), dim3(kTileThreads), 0, stream, w);
}

}  // namespace moe
