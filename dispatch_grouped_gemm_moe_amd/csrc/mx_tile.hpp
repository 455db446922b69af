// Tile-level building blocks of the MXFP8 (scaled-MFMA) grouped GEMMs, shared
// by the one-launch-per-GEMM kernels and the persistent layer kernel.
#pragma once

#include "common.hpp"
#include "gemm_tile.hpp"
#include "kernels.hpp"
#include "mxfp8.hpp"

namespace moe {

// Eight-wave MXFP8 tile: 256 x 256 output per workgroup of 512 threads, two
// waves per SIMD, each wave a 64 x 128 block of 2 x 4 fragments of
// v_mfma_scale_f32_32x32x64_f8f6f4 (as the bf16 tile).  A stage holds two
// 64-deep K steps: A and B codes as 128-byte rows (whole-line loads, 8 lanes
// per row), then one scale dword per A row and per B row (the operand scale
// layout's group: the four E8M0 block scales of the stage's 128 columns);
// two stages (132 KB).  An odd number of K steps ends on a half stage whose
// second K step repeats the last one in LDS and gets no MFMAs.
constexpr int kMxRow = 128;                               // code bytes of a row per stage
constexpr int kMxStageA = BM * kMxRow;                    // 32 KB
constexpr int kMxStageSA = (BM + BN) * kMxRow;            // scales: [256 A rows] dwords
constexpr int kMxStageSB = kMxStageSA + BM * 4;           //         [256 B rows] dwords
constexpr int kMxStageBytes = kMxStageSB + BN * 4;        // 66 KB
constexpr int kMxStages = 2;
constexpr int kMxSmem = kMxStages * kMxStageBytes;
constexpr int kEpiPitch8 = 8 * 16 + 16;  // staged codes: 128 bytes of data per row
static_assert(kEpiRows * (kEpiPitch8 + 2 * kEpiPitch32) <= kMxSmem - 4,
              "the staged SwiGLU block must fit the ring (the layer kernel keeps its last dword)");
static_assert(kEpiRows * kEpiPitch64 <= kMxSmem, "the staged fp32 block must fit the ring");

// Chained MXFP8 tiles (as the bf16 ones, gemm_tile.hpp): the staging block of
// a chained tile's bf16 output sits past the ring, 32 rows of 512 bytes (the
// ring leaves 28 KB of LDS).  MxLink carries the successor's load addresses as
// differences from this tile's, per wave: A code rows, B code rows and this
// lane's scale dwords.
constexpr int kMxStgRows = 32;
constexpr int kMxStgBytes = kMxStgRows * kStgPitch;
static_assert(kMxSmem + kMxStgBytes <= 160 * 1024, "ring and staging block fit the LDS");
struct MxLink {
    int64_t da = 0, db = 0, ds = 0;  // successor minus this tile: A codes, B codes, scale source
    bool next = false;
};

// One 256 x 256 output tile (expert e, M tile ml of the expert, N tile ntile)
// of the MXFP8 grouped GEMM with its epilogue, by 512 threads; smem is the
// kMxSmem LDS ring.  Wave w (wm = w/2, wn = w%2) owns fragments i = 0, 1 at
// tile rows 128i + 32wm .. +31 and j = 0..3 at columns 128wn + 32j .. +31;
// only the first NV row fragments (those holding a valid row of the expert's
// last tile) get MFMAs and fragment reads.
// kChain: the tile starts as en says, loads its successor's stages 0 and 1
// with the two loads past its last stage when ln.next, and (bf16 output)
// stages its output past the ring; smem then holds kMxSmem + kMxStgBytes.
template <int EPI, int NV, bool kChain = false>
__device__ __forceinline__ void mx_tile_body(const MxGemmArgs p, int e, int ml, int ntile, uint8_t* smem,
                                             TileEntry en = {}, MxLink ln = {}) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS bases
    const int wm = wave >> 1, wn = wave & 1;
    const int KT = p.K / 64, KS = (KT + 1) / 2;
    auto lay = [&](const int32_t* q) -> int { return kChain ? ld_layout(q) : *q; };
    const int seg0 = lay(p.prow_start + e);
    const int prow0 = seg0 + ml * BM;
    // BM rows, or kSegRows for an expert's last tile when it is a half tile
    // (NV is then at most 1); rows past it load the tile's own rows again
    const int trows = tile_rows_of(seg0, lay(p.prow_start + e + 1), ml);
    const int n0 = ntile * BN;

    // Code loads: instruction i fills tile rows 32*wave + 8i .. +7 (lane/8 the
    // row, lane%8 the fixed LDS chunk, loading the logical chunk stored there;
    // chunks 4..7 hold the stage's second K step).  Scale load: waves 0..3
    // take the dwords of A rows 64*wave + lane, waves 4..7 those of B rows
    // 64*(wave-4) + lane, which land as the stage's SA and SB arrays.
    const char* a_base = (const char*)p.A;
    const char* b_base = (const char*)(p.B + (int64_t)e * p.b_stride);
    uint32_t aoff[4], boff[4];
    int himask = 0;  // bit i: this lane's chunk of instruction i belongs to the stage's second K step
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wave * 32 + i * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ swz8(r);
        himask |= (lchunk >> 2) << i;
        const int prow = prow0 + (r & (trows - 1));
        const int arow = p.a_row_map ? p.a_row_map[prow] : prow;
        aoff[i] = (uint32_t)((int64_t)arow * p.lda + lchunk * 16);
        boff[i] = (uint32_t)((int64_t)min(n0 + r, p.N - 1) * p.K + lchunk * 16);
    }
    const int srow = (wave & 3) * 64 + lane;
    const char* s_lane;
    int64_t s_kstride;
    if (wave >= 4) {
        s_lane = (const char*)(p.SB + (int64_t)e * p.sb_stride) + (int64_t)min(n0 + srow, p.N - 1) * 4;
        s_kstride = p.sb_kstride;
    } else {
        const int sprow = prow0 + (srow & (trows - 1));
        const int sarow = p.a_row_map ? p.a_row_map[sprow] : sprow;
        s_lane = (const char*)p.SA + (int64_t)sarow * 4;
        s_kstride = p.sa_kstride;
    }

    // Loads past the last stage repeat it (into the slot no wave reads any
    // more), so they need no branch and the waits are constants.  On a half
    // stage (odd K steps) the second K step's code chunks repeat the first's
    // and the upper half of the stage's scale dwords is zero; neither is used.
    auto issue = [&](int s_, int slot) {
        uint8_t* st = smem + slot * kMxStageBytes;
        uint8_t* base = st + (wave * 32) * kMxRow;
        if constexpr (kChain) {
            // past the last stage, the successor's stage s_ - KS (a full
            // stage); one load sequence, its bases picked by scalar selects
            // (a branch to a second sequence costs vector registers)
            const bool nx = ln.next && s_ >= KS;
            const int s = nx ? s_ - KS : (s_ < KS ? s_ : KS - 1);
            const int back = !nx && 2 * s + 1 >= KT ? himask : 0;
            const char* ab = a_base + (nx ? ln.da : 0);
            const char* bb = b_base + (nx ? ln.db : 0);
            const int64_t so = (int64_t)s * s_kstride + (nx ? ln.ds : 0);
            const uint32_t kb = (uint32_t)s * 128;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_global_load_lds((gbl_cvoid*)(ab + aoff[i] + kb - ((back >> i) & 1) * 64),
                                                 (lds_void*)(base + i * 1024), 16, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_global_load_lds((gbl_cvoid*)(bb + boff[i] + kb - ((back >> i) & 1) * 64),
                                                 (lds_void*)(base + kMxStageA + i * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_cvoid*)(s_lane + so), (lds_void*)(st + kMxStageSA + wave * 256), 4,
                                             0, 0);
        } else {
            const int s = s_ < KS ? s_ : KS - 1;
            // a half stage's second K step repeats the first: the lanes of the
            // upper chunks step back 64 bytes
            const int back = 2 * s + 1 >= KT ? himask : 0;
            const uint32_t kb = (uint32_t)s * 128;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_global_load_lds((gbl_cvoid*)(a_base + aoff[i] + kb - ((back >> i) & 1) * 64),
                                                 (lds_void*)(base + i * 1024), 16, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_global_load_lds((gbl_cvoid*)(b_base + boff[i] + kb - ((back >> i) & 1) * 64),
                                                 (lds_void*)(base + kMxStageA + i * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_cvoid*)(s_lane + (int64_t)s * s_kstride),
                                             (lds_void*)(st + kMxStageSA + wave * 256), 4, 0, 0);
        }
    };
    const int fr = lane & 31, half = lane >> 5;
    const int fsw = swz8(fr);  // a fragment's rows differ from fr by multiples of 32
    const int arow_b = (wm * 32 + fr) * kMxRow, brow_b = kMxStageA + (wn * 128 + fr) * kMxRow;
    // Fragments of K step ks (0, 1) of the stage in `slot`: per lane, bytes
    // 0..15 from the row's first 32-block of the K step, 16..31 from its second.
    // With ks = 0 also the rows' scale dwords, shifted right by 8 * half: then
    // byte 2 * ks of the register is the scale of (row, block half) of K step
    // ks, which the MFMA's scale byte select takes as an immediate.
    auto read_a = [&](int slot, int ks, int i, intx8& a, int& sa) {
        const uint8_t* st = smem + slot * kMxStageBytes;
        const int pc0 = ((4 * ks + half) ^ fsw) * 16, pc1 = ((4 * ks + 2 + half) ^ fsw) * 16;
        const intx4 lo4 = *(const intx4*)(st + arow_b + i * 128 * kMxRow + pc0);
        const intx4 hi4 = *(const intx4*)(st + arow_b + i * 128 * kMxRow + pc1);
        a = intx8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        if (ks == 0) sa = (int)(*(const uint32_t*)(st + kMxStageSA + (i * 128 + wm * 32 + fr) * 4) >> (8 * half));
    };
    auto read_b = [&](int slot, int ks, int j, intx8& b, int& sb) {
        const uint8_t* st = smem + slot * kMxStageBytes;
        const int pc0 = ((4 * ks + half) ^ fsw) * 16, pc1 = ((4 * ks + 2 + half) ^ fsw) * 16;
        const intx4 lo4 = *(const intx4*)(st + brow_b + j * 32 * kMxRow + pc0);
        const intx4 hi4 = *(const intx4*)(st + brow_b + j * 32 * kMxRow + pc1);
        b = intx8{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        if (ks == 0) sb = (int)(*(const uint32_t*)(st + kMxStageSB + (wn * 128 + j * 32 + fr) * 4) >> (8 * half));
    };
    floatx16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
    // B is the first operand (with its scales), so each accumulator holds the
    // transposed block: element 4q + s of fragment (i, j) of lane l sits in
    // tile row 128i + 32wm + l%32 and column wn*128 + 32j + 8q + 4(l/32) + s.
    // The MFMAs of K step ksc (std::integral_constant; its scales are byte
    // 2 * ks) on the fragments in registers, B fragment by B fragment.  The
    // fragments are single-buffered (the scaled operands are twice the bf16
    // ones and two waves share a SIMD's registers), so as soon as B fragment
    // j's last MFMA is issued its registers take fragment j of K step rks of
    // the stage in rslot, and the A fragments follow the last one: the next K
    // step's LDS reads overlap this one's MFMAs.
    auto mfmas_then = [&](auto ksc, int rslot, int rks, intx8 (&a)[2], intx8 (&b)[4], int (&sa)[2], int (&sb)[4]) {
        constexpr int sel = 2 * decltype(ksc)::value;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int i = 0; i < NV; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0, sel, sb[j],
                                                                             sel, sa[i]);
            read_b(rslot, rks, j, b[j], sb[j]);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) read_a(rslot, rks, i, a[i], sa[i]);
    };

    // Ring protocol (stage j in slot j % 2, 9 direct-to-LDS loads per lane and
    // stage): the prologue issues stages 0 and 1, waits for stage 0
    // (vmcnt(9)) and reads its first K step's fragments.  Full stage s runs
    // its first K step while reading its second's fragments, waits for stage
    // s+1 (vmcnt(0)) and its own LDS reads, barrier (no wave reads stage s any
    // more), refills its slot with stage s+2 and runs its second K step while
    // reading the first K step of stage s+1.  An odd number of K steps ends on
    // a half stage, whose one K step is read by then.
    // A chained tile's stages 0 and 1 went out with its predecessor's last
    // two: stage 0 was waited for before the predecessor's last barrier.
    static_assert(kMxStages == 2, "the vmcnt immediates below assume 2 stages of 9 loads");
    const int s0 = kChain ? en.slot0 : 0;
    if (!(kChain && en.pre)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        issue(0, s0);
        issue(1, s0 ^ 1);
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        __syncthreads();
    }
    intx8 fa[2], fb[4];
    int fsa[2], fsb[4];
#pragma unroll
    for (int i = 0; i < NV; ++i) read_a(s0, 0, i, fa[i], fsa[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) read_b(s0, 0, j, fb[j], fsb[j]);
    int slot = s0;
    for (int s = 0; s < KT / 2; ++s) {
        mfmas_then(std::integral_constant<int, 0>{}, slot, 1, fa, fb, fsa, fsb);
        Interleave<4 * NV, 0, 8 + 2 * NV>::run();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        issue(s + 2, slot);
        // after the last full stage this reads the half stage, or a stale but
        // in-bounds repeat of the last stage that nothing uses
        mfmas_then(std::integral_constant<int, 1>{}, slot ^ 1, 0, fa, fb, fsa, fsb);
        Interleave<4 * NV, 9, 8 + 2 * NV>::run();
        __builtin_amdgcn_sched_barrier(0);
        slot ^= 1;
    }
    if (KT & 1) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0, fsb[j], 0,
                                                                             fsa[i]);
    }

    if constexpr (kChain && EPI == kEpiStore) {
        if (!p.Cf) {
            // bf16 output through the block past the ring, 32 rows at a time:
            // tile rows 64 bl + 32 h .. are fragment bl/2 of the two waves
            // with wm == 2 (bl % 2) + h, row lane % 32.  Chunk c of staged row
            // r at c ^ r; asm LDS accesses and LDS-only barriers, so nothing
            // waits for the successor's loads in flight (as gemm_tile).
            if (!ln.next) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const uint32_t stg = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem + kMxSmem;
            int tid = threadIdx.x;  // opaque: the lane addresses are formed here, not kept live
            asm volatile("" : "+v"(tid));
            const int rs = tid & 31;
            const uint32_t wrow = stg + rs * kStgPitch + 8 * ((tid >> 5) & 1);
            const int wc0 = ((tid >> 6) & 1) * 16;
            const int r0 = tid >> 5, ch = tid & 31;  // copy-out: rows r0, r0 + 16 of a block, chunk ch
            const bool col_in = ch * 16 < (p.N - n0) * 2;
#pragma unroll
            for (int bl = 0; bl < 4; ++bl) {
                if (bl * kEpiRows >= trows) break;  // a half tile stores its kSegRows rows only
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (wm == 2 * (bl & 1) + h) {
                        const int i = bl >> 1;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const uint32_t la = wrow + (((wc0 + 4 * j + q) ^ rs) << 4);
                                const uint2 pv = pack_bf16x4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                             acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                                const u32x2 v2 = {pv.x, pv.y};
                                asm volatile("ds_write_b64 %0, %1" ::"v"(la), "v"(v2) : "memory");
                            }
                    }
                    lds_barrier();
                    const uint32_t ra0 = stg + r0 * kStgPitch + ((ch ^ r0) << 4);
                    const uint32_t ra1 = stg + (r0 + 16) * kStgPitch + ((ch ^ (r0 + 16)) << 4);
                    u32x4 d0, d1;
                    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                                 : "=&v"(d0), "=&v"(d1)
                                 : "v"(ra0), "v"(ra1)
                                 : "memory");
                    char* dst = (char*)(p.C + (int64_t)(prow0 + bl * 64 + h * 32 + r0) * p.ldc + n0) + ch * 16;
                    if (col_in) {
                        *(u32x4*)dst = d0;
                        *(u32x4*)(dst + (int64_t)p.ldc * 2 * 16) = d1;
                    }
                    lds_barrier();
                }
            }
            return;
        }
    }

    // The tile leaves through LDS, 64 rows at a time (whole-line stores).
    // Block b (tile rows 64b .. 64b+63) is fragment b/2 of the waves with
    // wm/2 == b%2, this lane's row in it (wm%2)*32 + lane%32.  N is a multiple
    // of 64, so a 4-column run, and a 16-byte chunk, lies wholly inside or
    // outside the matrix.
    epi_begin();
    const int rl = (wm & 1) * 32 + fr;
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
        for (int bl = 0; bl < 4; ++bl) {
            if (bl * kEpiRows >= trows) break;  // a half tile stores its kSegRows rows only
            if ((wm >> 1) == (bl & 1)) {
                const int i = bl >> 1;
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
                        *(uint32_t*)(qb + rl * kEpiPitch8 + hc) =
                            fp8x4(ldexpf(h[4 * q], -ex), ldexpf(h[4 * q + 1], -ex), ldexpf(h[4 * q + 2], -ex),
                                  ldexpf(h[4 * q + 3], -ex));
                        if (p.GU) {
                            *(floatx4*)(gb + rl * kEpiPitch32 + hc * 4) =
                                floatx4{g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]};
                            *(floatx4*)(ub + rl * kEpiPitch32 + hc * 4) =
                                floatx4{u[4 * q], u[4 * q + 1], u[4 * q + 2], u[4 * q + 3]};
                        }
                    }
                }
                // the row's two block scales of this 64-column pair, into the
                // operand scale layout; lanes 0..31 hold 32 consecutive rows
                const int64_t row = prow0 + bl * 64 + rl;
                if (live && half == 0) mx_store_scale_pair(p.Cs, p.cs_rows, row, (hc0 + wn * 64) >> 6, I / 64, sdw);
            }
            __syncthreads();
            const int64_t row0 = prow0 + bl * 64;
            const int lim = I - hc0;
            epi_copy_out<8, kTileThreads>(qb, kEpiPitch8, (char*)(p.Cq + row0 * I + hc0), (int64_t)I, lim);
            if (p.GU) {
                epi_copy_out<32, kTileThreads>(gb, kEpiPitch32, (char*)(p.GU + row0 * p.N + hc0), (int64_t)p.N * 4,
                                               lim * 4);
                epi_copy_out<32, kTileThreads>(ub, kEpiPitch32, (char*)(p.GU + row0 * p.N + I + hc0),
                                               (int64_t)p.N * 4, lim * 4);
            }
            __syncthreads();
        }
    } else if (p.Cf) {  // fp32 output
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) {
            if (bl * kEpiRows >= trows) break;  // a half tile stores its kSegRows rows only
            if ((wm >> 1) == (bl & 1)) {
                const int i = bl >> 1;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(floatx4*)(smem + rl * kEpiPitch64 + frag_col(j, q) * 4) =
                            floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            }
            __syncthreads();
            epi_copy_out<64, kTileThreads>(smem, kEpiPitch64, (char*)(p.Cf + (int64_t)(prow0 + bl * 64) * p.ldc + n0),
                                           (int64_t)p.ldc * 4, (p.N - n0) * 4);
            __syncthreads();
        }
    } else {  // bf16 output
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) {
            if (bl * kEpiRows >= trows) break;  // a half tile stores its kSegRows rows only
            if ((wm >> 1) == (bl & 1)) {
                const int i = bl >> 1;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(uint2*)(smem + rl * kEpiPitch32 + frag_col(j, q) * 2) = pack_bf16x4(
                            acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            }
            __syncthreads();
            epi_copy_out<32, kTileThreads>(smem, kEpiPitch32, (char*)(p.C + (int64_t)(prow0 + bl * 64) * p.ldc + n0),
                                           (int64_t)p.ldc * 2, (p.N - n0) * 2);
            __syncthreads();
        }
    }
}

// One 256 x 256 output tile (expert e, M tile ml, N tile ntile) of the MXFP8
// grouped GEMM; with p.rows_e the padding fragments of an expert's last tile
// get no MFMAs as kPad says (gemm_tile.hpp).
// kChain: as mx_tile_body; *en is set for the successor.
template <int EPI, int kPad = kPadPerWave, bool kChain = false>
__device__ __forceinline__ void mx_gemm_tile(const MxGemmArgs p, int e, int ml, int ntile, uint8_t* smem,
                                             TileEntry* en = nullptr, const MxLink* ln = nullptr) {
    const TileEntry te = kChain ? *en : TileEntry{};
    const MxLink tl = kChain ? *ln : MxLink{};
    if constexpr (kChain) {
        en->pre = tl.next;
        en->slot0 = te.slot0 ^ (((p.K / 64 + 1) / 2) & 1);  // the successor's stage 0 follows this tile's stages
    }
    if (kPad == kPadNone || !p.rows_e) {  // every fragment (a half tile's rows past kSegRows are not stored)
        mx_tile_body<EPI, 2, kChain>(p, e, ml, ntile, smem, te, tl);
        return;
    }
    // fragment i of this wave holds tile rows 128i + 32wm .. +31 (a half
    // tile has at most kSegRows valid rows, so NV <= 1)
    const int valid = (kChain ? ld_layout(p.rows_e + e) : p.rows_e[e]) - ml * BM;
    const int w32 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 7) * 32;
    switch (valid > 128 + w32 ? 2 : (valid > w32 ? 1 : 0)) {
        case 2: mx_tile_body<EPI, 2, kChain>(p, e, ml, ntile, smem, te, tl); break;
        case 1: mx_tile_body<EPI, 1, kChain>(p, e, ml, ntile, smem, te, tl); break;
        default: mx_tile_body<EPI, 0, kChain>(p, e, ml, ntile, smem, te, tl); break;
    }
}

// Whether a launch's kEpiStore MXFP8 tiles can chain: bf16 output, A rows
// read directly, whole N tiles, and an even number of K steps, at least four
// (two full stages).
__device__ __forceinline__ bool mx_tiles_chain(const MxGemmArgs& p) {
    return p.C && !p.Cf && !p.a_row_map && p.N % BN == 0 && p.K % 128 == 0 && p.K >= 256;
}

// The link from tile (p, e, ml, ntile) to its successor (pn, e2, ml2, nt2) of
// the same launch.  mx_tile_body's code rows of a lane are prow0 + (r &
// (trows - 1)), r = 32 wave + 8i + lane/8 (so r >= 128 for waves 4..7), B rows
// n0 + r; its scale dword comes from A row prow0 + (srow & (trows - 1)),
// srow = 64 (wave % 4) + lane (>= 128 for waves 2, 3), for waves 0..3 and from
// B row n0 + srow for waves 4..7.
__device__ __forceinline__ MxLink mx_tile_link(const MxGemmArgs& p, int e, int ml, int ntile, const MxGemmArgs& pn,
                                               int e2, int ml2, int nt2) {
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int seg0 = ld_layout(p.prow_start + e), prow0 = seg0 + ml * BM;
    const int trows = tile_rows_of(seg0, ld_layout(p.prow_start + e + 1), ml);
    const int seg2 = ld_layout(pn.prow_start + e2), prow2 = seg2 + ml2 * BM;
    const int trows2 = tile_rows_of(seg2, ld_layout(pn.prow_start + e2 + 1), ml2);
    // upper-half rows of a half tile fold back by kSegRows
    const int fold = (trows < BM ? kSegRows : 0) - (trows2 < BM ? kSegRows : 0);
    MxLink ln;
    ln.da = ((const char*)pn.A - (const char*)p.A) + ((int64_t)(prow2 - prow0) + (wave >= 4 ? fold : 0)) * p.lda;
    ln.db = ((const char*)(pn.B + (int64_t)e2 * pn.b_stride) - (const char*)(p.B + (int64_t)e * p.b_stride)) +
            (int64_t)(nt2 - ntile) * BN * p.K;
    if (wave >= 4)
        ln.ds = ((const char*)(pn.SB + (int64_t)e2 * pn.sb_stride) - (const char*)(p.SB + (int64_t)e * p.sb_stride)) +
                (int64_t)(nt2 - ntile) * BN * 4;
    else
        ln.ds = ((const char*)pn.SA - (const char*)p.SA) + ((int64_t)(prow2 - prow0) + (wave >= 2 ? fold : 0)) * 4;
    ln.next = true;
    return ln;
}

}  // namespace moe
