// Tile-level building blocks of the MXFP8 (scaled-MFMA) grouped GEMMs, shared
// by the one-launch-per-GEMM kernels and the persistent layer kernel.
#pragma once

#include "common.hpp"
#include "gemm_tile.hpp"
#include "kernels.hpp"
#include "mxfp8.hpp"

namespace moe {

// LDS stage: A codes [256][64 B], B codes [256][64 B], A scales [256][4 B],
// B scales [256][4 B].  Code rows use the bf16 path's conflict-free swizzle.
constexpr int kMxRow = 64;
constexpr int kMxStageA = BM * kMxRow;
constexpr int kMxStageSA = (BM + BN) * kMxRow;
constexpr int kMxStageSB = kMxStageSA + BM * 4;
constexpr int kMxStageBytes = kMxStageSB + BN * 4;
constexpr int kMxStages = 4;  // 136 KB
constexpr int kMxLoads = 10;  // direct-to-LDS loads per lane per K step
constexpr int kEpiPitch8 = 8 * 16 + 16;  // staged codes: 128 bytes of data per row
static_assert(kEpiRows * (kEpiPitch8 + 2 * kEpiPitch32) <= kMxStages * kMxStageBytes - 4,
              "the staged SwiGLU block must fit the ring (the layer kernel keeps its last dword)");
static_assert(kEpiRows * kEpiPitch64 <= kMxStages * kMxStageBytes, "the staged fp32 block must fit the ring");

__device__ __forceinline__ int mx_swz(int r) { return (r >> 2) & 3; }


// One 256 x 256 output tile (expert e, M tile ml of the expert, N tile ntile)
// of the MXFP8 grouped GEMM with its epilogue; smem is the kMxStages LDS ring.
// Row fragments as in the bf16 tile: fragment i of wave (wm, wn) holds tile
// rows 64i + 32wm .. +31, and only the first NV of them (those holding a valid
// row of the expert's last tile) get MFMAs and fragment reads.
template <int EPI, int NV>
__device__ __forceinline__ void mx_tile_body(const MxGemmArgs p, int e, int ml, int ntile, uint8_t* smem) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS bases
    const int wm = wave >> 1, wn = wave & 1;
    const int KT = p.K / 64;
    const int mt0 = p.mt_start[e];
    const int prow0 = (mt0 + ml) * BM;
    const int n0 = ntile * BN;

    // per-lane staging: code rows wave*64 + 16i + lane/4 (swizzled chunk),
    // scale row wave*64 + lane (one dword per row and K step)
    const char* a_base = (const char*)p.A;
    const char* b_base = (const char*)(p.B + (int64_t)e * p.b_stride);
    const char* sa_base = (const char*)p.SA;
    const char* sb_base = (const char*)(p.SB + (int64_t)e * p.sb_stride);
    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wave * 64 + i * 16 + (lane >> 2);
        const int lchunk = (lane & 3) ^ mx_swz(r);
        const int prow = prow0 + r;
        const int arow = p.a_row_map ? p.a_row_map[prow] : prow;
        aoff[i] = (uint32_t)((int64_t)arow * p.lda + lchunk * 16);
        boff[i] = (uint32_t)((int64_t)min(n0 + r, p.N - 1) * p.K + lchunk * 16);
    }
    const int srow = wave * 64 + lane;
    const int sarow = p.a_row_map ? p.a_row_map[prow0 + srow] : prow0 + srow;
    const uint32_t saoff = (uint32_t)sarow * 4, sboff = (uint32_t)min(n0 + srow, p.N - 1) * 4;

    // Loads past the last K step repeat it (into the slot of a step every wave
    // has finished with), so they need no branch and the waits are constants.
    auto issue = [&](int kt_, int slot) {
        const int kt = kt_ < KT ? kt_ : KT - 1;
        uint8_t* st = smem + slot * kMxStageBytes;
        uint8_t* base = st + (wave * 64) * kMxRow;
        const uint32_t kb = (uint32_t)kt * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((gbl_cvoid*)(a_base + aoff[i] + kb), (lds_void*)(base + i * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((gbl_cvoid*)(b_base + boff[i] + kb), (lds_void*)(base + kMxStageA + i * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_cvoid*)(sa_base + (int64_t)kt * p.sa_kstride + saoff),
                                         (lds_void*)(st + kMxStageSA + wave * 256), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_cvoid*)(sb_base + (int64_t)kt * p.sb_kstride + sboff),
                                         (lds_void*)(st + kMxStageSB + wave * 256), 4, 0, 0);
    };
    const int fr = lane & 31, half = lane >> 5;
    const int fsw = mx_swz(fr);
    const int pc0 = (half ^ fsw) * 16, pc1 = ((2 + half) ^ fsw) * 16;
    const int arow_b = (wm * 32 + fr) * kMxRow, brow_b = kMxStageA + (wn * 128 + fr) * kMxRow;
    auto frags = [&](int slot, intx8 (&a)[4], intx8 (&b)[4], int (&sa)[4], int (&sb)[4]) {
        const uint8_t* st = smem + slot * kMxStageBytes;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const intx4 lo4 = *(const intx4*)(st + arow_b + i * 64 * kMxRow + pc0);
            const intx4 hi4 = *(const intx4*)(st + arow_b + i * 64 * kMxRow + pc1);
            a[i] = intx8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            sa[i] = st[kMxStageSA + (i * 64 + wm * 32 + fr) * 4 + half];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const intx4 lo4 = *(const intx4*)(st + brow_b + j * 32 * kMxRow + pc0);
            const intx4 hi4 = *(const intx4*)(st + brow_b + j * 32 * kMxRow + pc1);
            b[j] = intx8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            sb[j] = st[kMxStageSB + (wn * 128 + j * 32 + fr) * 4 + half];
        }
    };
    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
    // B is the first operand (with its scales), so each accumulator holds the
    // transposed block: element 4q + s of fragment (i, j) of lane l sits in
    // tile row 64i + 32wm + l%32 and column wn*128 + 32j + 8q + 4(l/32) + s.
    auto mfmas = [&](const intx8 (&a)[4], const intx8 (&b)[4], const int (&sa)[4], const int (&sb)[4]) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, sb[j], 0,
                                                                             sa[i]);
    };

    // Ring protocol as in the bf16 path, with 10 loads per K step and every
    // slot always in flight: before computing step kt, wait until step kt+1
    // has landed (the 2 newer steps stay in flight: vmcnt(20)) and this wave's
    // reads of step kt are done, barrier, refill step kt's slot with step
    // kt + kMxStages, and read step kt+1's fragments under step kt's MFMAs.
    static_assert(kMxStages == 4, "the vmcnt immediates below assume 4 stages of 10 loads");
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMxStages; ++j) issue(j, j);
    asm volatile("s_waitcnt vmcnt(30)" ::: "memory");
    __syncthreads();
    intx8 a0[4], b0[4], a1[4], b1[4];
    int s0a[4], s0b[4], s1a[4], s1b[4];
    frags(0, a0, b0, s0a, s0b);
    int slot = 0;  // slot of step kt
    auto step = [&](int kt, intx8 (&ac)[4], intx8 (&bc)[4], int (&sac)[4], int (&sbc)[4], intx8 (&an)[4],
                    intx8 (&bn)[4], int (&san)[4], int (&sbn)[4]) {
        const int next_slot = slot + 1 == kMxStages ? 0 : slot + 1;
        asm volatile("s_waitcnt vmcnt(20) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        issue(kt + kMxStages, slot);
        frags(next_slot, an, bn, san, sbn);  // stale but in-bounds on the last step
        mfmas(ac, bc, sac, sbc);
        // 4NV MFMAs, 10 loads, 3 LDS reads per fragment (two code halves, one scale)
        Interleave<4 * NV, 10, 3 * (NV + 4)>::run();
        __builtin_amdgcn_sched_barrier(0);
        slot = next_slot;
    };
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
        step(kt, a0, b0, s0a, s0b, a1, b1, s1a, s1b);
        step(kt + 1, a1, b1, s1a, s1b, a0, b0, s0a, s0b);
    }
    if (kt < KT) step(kt, a0, b0, s0a, s0b, a1, b1, s1a, s1b);

    // The tile leaves through LDS, 64 rows at a time (whole-line stores): block
    // i (tile rows 64i .. 64i+63) is fragment i of every wave, this lane's row
    // in it wm*32 + lane%32.  N is a multiple of 64, so a 4-column run, and a
    // 16-byte chunk, lies wholly inside or outside the matrix.
    epi_begin();
    const int rl = wm * 32 + fr;
    if (EPI == kEpiSwiGLU) {
        // h = silu(g) * u, then MXFP8 along I in 32-column blocks: a block of a
        // row is lanes l and l+32 of one fragment (16 values each).  Routed
        // and padding rows alike (the padding rows' codes are never read).
        const int I = p.N / 2, hc0 = n0 / 2;
        const bool live = hc0 + wn * 64 < I;  // I is a multiple of 64: both blocks of the pair alike
        uint8_t* qb = smem;                                 // [64][128] codes
        uint8_t* gb = smem + kEpiRows * kEpiPitch8;         // [64][128] fp32 g
        uint8_t* ub = gb + kEpiRows * kEpiPitch32;          // [64][128] fp32 u
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t sdw = 0;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float g[16], u[16], h[16];
                float m = 0.0f;
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    g[c] = acc[i][2 * jj][c];
                    u[c] = acc[i][2 * jj + 1][c];
                    h[c] = swiglu(g[c], u[c]);
                    m = fmaxf(m, fabsf(h[c]));
                }
                m = fmaxf(m, __shfl_xor(m, 32, kWave));
                const int ex = mx_scale_exp(m);
                sdw |= (uint32_t)(ex + 127) << (8 * jj);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int hc = wn * 64 + jj * 32 + q * 8 + 4 * half;
                    *(uint32_t*)(qb + rl * kEpiPitch8 + hc) = fp8x4(ldexpf(h[4 * q], -ex), ldexpf(h[4 * q + 1], -ex),
                                                                   ldexpf(h[4 * q + 2], -ex), ldexpf(h[4 * q + 3], -ex));
                    if (p.GU) {
                        *(floatx4*)(gb + rl * kEpiPitch32 + hc * 4) = floatx4{g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]};
                        *(floatx4*)(ub + rl * kEpiPitch32 + hc * 4) = floatx4{u[4 * q], u[4 * q + 1], u[4 * q + 2], u[4 * q + 3]};
                    }
                }
            }
            // the row's two block scales of this 64-column pair, as the GEMM
            // operand layout's dword {block 0, block 1, 0, 0}; lanes 0..31 hold
            // 32 consecutive rows, so the stores are one 128-byte run
            const int64_t row = prow0 + i * 64 + rl;
            if (live && half == 0) *(uint32_t*)(p.Cs + ((int64_t)((hc0 + wn * 64) >> 6) * p.cs_rows + row) * 4) = sdw;
            __syncthreads();
            const int64_t row0 = prow0 + i * 64;
            const int lim = I - hc0;
            epi_copy_out<8, kGemmThreads>(qb, kEpiPitch8, (char*)(p.Cq + row0 * I + hc0), (int64_t)I, lim);
            if (p.GU) {
                epi_copy_out<32, kGemmThreads>(gb, kEpiPitch32, (char*)(p.GU + row0 * p.N + hc0), (int64_t)p.N * 4,
                                               lim * 4);
                epi_copy_out<32, kGemmThreads>(ub, kEpiPitch32, (char*)(p.GU + row0 * p.N + I + hc0),
                                               (int64_t)p.N * 4, lim * 4);
            }
            __syncthreads();
        }
    } else if (p.Cf) {  // fp32 output
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(floatx4*)(smem + rl * kEpiPitch64 + frag_col(j, q) * 4) =
                        floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            __syncthreads();
            epi_copy_out<64, kGemmThreads>(smem, kEpiPitch64, (char*)(p.Cf + (int64_t)(prow0 + i * 64) * p.ldc + n0),
                                           (int64_t)p.ldc * 4, (p.N - n0) * 4);
            __syncthreads();
        }
    } else {  // bf16 output
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(uint2*)(smem + rl * kEpiPitch32 + frag_col(j, q) * 2) = pack_bf16x4(
                        acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            __syncthreads();
            epi_copy_out<32, kGemmThreads>(smem, kEpiPitch32, (char*)(p.C + (int64_t)(prow0 + i * 64) * p.ldc + n0),
                                           (int64_t)p.ldc * 2, (p.N - n0) * 2);
            __syncthreads();
        }
    }
}


// One 256 x 256 output tile (expert e, M tile ml, N tile ntile) of the MXFP8
// grouped GEMM; with p.rows_e and kSkipPadding the padding fragments of an
// expert's last tile get no MFMAs (the layer kernel compiles the full loop).
template <int EPI, bool kSkipPadding = true>
__device__ __forceinline__ void mx_gemm_tile(const MxGemmArgs p, int e, int ml, int ntile, uint8_t* smem) {
    if (!kSkipPadding || !p.rows_e) {
        mx_tile_body<EPI, 4>(p, e, ml, ntile, smem);
        return;
    }
    switch (valid_frags(p.rows_e[e] - ml * BM)) {
        case 4: mx_tile_body<EPI, 4>(p, e, ml, ntile, smem); break;
        case 3: mx_tile_body<EPI, 3>(p, e, ml, ntile, smem); break;
        case 2: mx_tile_body<EPI, 2>(p, e, ml, ntile, smem); break;
        case 1: mx_tile_body<EPI, 1>(p, e, ml, ntile, smem); break;
        default: mx_tile_body<EPI, 0>(p, e, ml, ntile, smem); break;
    }
}

}  // namespace moe
