// Tile-level building blocks of the bf16 grouped GEMMs, shared by the
// one-launch-per-GEMM kernels and the persistent layer kernel.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Scheduling: interleave M MFMAs, V global loads and D LDS reads round robin.
template <int M, int V, int D>
struct Interleave {
    static __device__ __forceinline__ void run() {
        if constexpr (M > 0) __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(kSchedVMEM, 1, 0);
        if constexpr (D > 0) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
        if constexpr (M > 1 || V > 1 || D > 1)
            Interleave<(M > 0 ? M - 1 : 0), (V > 0 ? V - 1 : 0), (D > 0 ? D - 1 : 0)>::run();
    }
};

// The B fragment is the MFMA's first operand, so each accumulator holds the
// transposed 32 x 32 block: accumulator element 4q + s of fragment (i, j) of
// lane l sits in tile row 128i + 32wm + l%32 and tile column
// wn*128 + 32j + 8q + 4(l/32) + s -- one tile row, runs of four consecutive
// columns, which the epilogues stage 8 or 16 bytes at a time.  frag_col(j, q):
// the tile column of this lane's run q of fragment j.
__device__ __forceinline__ int frag_col(int j, int q) {
    const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
    return wn * 128 + j * 32 + q * 8 + 4 * (lane >> 5);
}

// Four fp32 values as four bf16 (round to nearest even, gfx950's packed
// conversion), packed for one 8-byte store.
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{a, b}), bf16x2)),
                      __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{c, d}), bf16x2)));
}

// silu(g) * u with the hardware reciprocal (about 1 ulp) for the logistic.
__device__ __forceinline__ float swiglu(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Tile coordinates of tile v of a grouped GEMM over experts [e_begin, e_end):
// expert-major, then N tile, then M tile (M fastest).
__device__ __forceinline__ void tile_coords(const int32_t* mt_start, int e_begin, int e_end, int NT, int v,
                                            int& e, int& ml, int& ntile) {
    const int mt_lo = ld_layout(mt_start + e_begin);
    int lo = e_begin, hi = e_end - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((ld_layout(mt_start + mid) - mt_lo) * NT <= v) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int mt0 = ld_layout(mt_start + e), mte = ld_layout(mt_start + e + 1) - mt0;
    const int loc = v - (mt0 - mt_lo) * NT;
    ntile = loc / mte;
    ml = loc - ntile * mte;
}

// Tiles of a grouped GEMM (M tiles of all processed experts times N tiles).
__device__ __forceinline__ int grouped_tiles(const int32_t* mt_start, int e_begin, int e_end, int N) {
    return (ld_layout(mt_start + e_end) - ld_layout(mt_start + e_begin)) * ceil_div(N, BN);
}

// A launch over p.nmb minibatches (GemmArgs / MxGemmArgs): its total tile
// count, and for tile v the minibatch holding it (v becomes the tile index
// within that minibatch).
template <class Args>
__device__ __forceinline__ int launch_tiles(const Args& p) {
    const int nmb = p.nmb > 1 ? p.nmb : 1;
    int total = 0;
    for (int b = 0; b < nmb; ++b) total += grouped_tiles(p.mt_start + (int64_t)b * p.mt_ld, p.e_begin, p.e_end, p.N);
    return total;
}
template <class Args>
__device__ __forceinline__ int minibatch_of_tile(const Args& p, int& v) {
    int b = 0;
    for (; b + 1 < p.nmb; ++b) {
        const int nt = grouped_tiles(p.mt_start + (int64_t)b * p.mt_ld, p.e_begin, p.e_end, p.N);
        if (v < nt) break;
        v -= nt;
    }
    return b;
}

// Epilogue staging.  A 64-row block of the tile is written to LDS with row
// pitches 16 bytes longer than the data (256, 512 or 1024 bytes), so the 32
// rows of one write instruction fall on different banks, then copied out in
// 16-byte chunks along rows.
constexpr int kEpiRows = 64;
constexpr int kEpiPitch16 = 16 * 16 + 16;  // 16 chunks of data per row
constexpr int kEpiPitch32 = 32 * 16 + 16;
constexpr int kEpiPitch64 = 64 * 16 + 16;
// Before the first staged block: the ring's trailing loads have landed and no
// wave reads the ring any more.
__device__ __forceinline__ void epi_begin() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// Rows 0..63 of an LDS block (kChunks 16-byte chunks per row, pitch `pitch`)
// to global rows dst + r * ld bytes; chunks at or beyond byte `limit` of a
// row are not stored.
template <int kChunks, int kThreads>
__device__ __forceinline__ void epi_copy_out(const uint8_t* lds, int pitch, char* dst, int64_t ld, int limit) {
    // an opaque copy of the thread index: its offsets are recomputed here
    // (a few adds) instead of being hoisted out of the tile loop and spilled
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
#pragma unroll
    for (int c = tid; c < kEpiRows * kChunks; c += kThreads) {
        const int r = c / kChunks, ch = c % kChunks;
        if (ch * 16 < limit) *(intx4*)(dst + r * ld + ch * 16) = *(const intx4*)(lds + r * pitch + ch * 16);
    }
}

// ---------------------------------------------------------------------------
// Eight-wave tile of the bf16 grouped GEMMs (forward, input gradients and the
// layer kernel): 256 x 256 output per workgroup of 512 threads, two waves per
// SIMD, each wave a 64 x 128 block of 2 x 4 fragments (128 accumulator
// registers, so two waves fit a SIMD's register file): when one wave waits
// on a load or a barrier, the other keeps the SIMD's matrix core busy.  K runs
// in 64-deep stages through a two-stage LDS ring (2 x 64 KB), every global
// load instruction moving whole 128-byte lines (8 lanes per row, 8 rows per
// instruction); measured against the four-wave tile on the same box: input-
// gradient GEMMs 8-13% faster.
// ---------------------------------------------------------------------------
constexpr int kTileThreads = 512;
constexpr int kBK8 = 64;
constexpr int kRow8 = kBK8 * 2;                   // bytes of one row per stage
constexpr int kStageA8 = BM * kRow8;              // 32 KB
constexpr int kStageBytes8 = (BM + BN) * kRow8;   // 64 KB
constexpr int kStages8 = 2;
constexpr int kTileSmem = kStages8 * kStageBytes8;
static_assert(kEpiRows * (kEpiPitch16 + 2 * kEpiPitch32) <= kTileSmem - 4, "staged SwiGLU block must fit");
static_assert(kEpiRows * kEpiPitch64 <= kTileSmem, "staged fp32 block must fit");

// Chunk c of row r of a 128-byte-row stage sits at position c ^ ((r >> 1) & 7):
// the 16 rows one 128-bit fragment read touches per pass fall on distinct banks.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Barrier over LDS only: this wave's LDS accesses have completed, then
// s_barrier.  __syncthreads' workgroup fence would also wait for every global
// memory operation in flight, direct-to-LDS loads and stores included.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Chained tiles.  A tile's first stage otherwise waits for its loads to come
// from memory after the previous tile's epilogue (about 5 us of a 60 us tile
// at K = 2048).  A chained tile loads its successor's stages 0 and 1 in place
// of the two loads past its own last stage, and stages its output through a
// separate LDS block (kStgBytes past the ring), so the successor starts on
// data already in LDS.  Measured on a dense probe (20480 rows, N = 7168):
// 8% faster at K = 2048, 3% at K = 4096, none at K = 7168, bitwise equal.
// Successor and tile read A rows directly (no row map) and whole N tiles,
// so the successor's per-lane load offsets are this tile's plus a per-wave
// constant, carried as base pointers.
// ---------------------------------------------------------------------------
constexpr int kStgPitch = 512;                    // 256 bf16 per staged row
constexpr int kStgBytes = kEpiRows * kStgPitch;   // 32 KB
struct TileLink {              // from a tile to its successor
    const char* na = nullptr;  // successor's A rows: na + aoff[q] + stage offset
    const char* nb = nullptr;  // successor's B rows: nb + boff[q] + stage offset
    bool next = false;         // the successor's stages 0 and 1 go out with this tile's last two
    bool next_load_a = true;   // the successor's waves load their A rows
};
struct TileEntry {      // how a tile starts
    bool pre = false;   // its stages 0 and 1 were loaded by its predecessor
    int slot0 = 0;      // ring slot of its stage 0
};

template <int NV>
__device__ __forceinline__ void mfma_block8(floatx16 (&acc)[2][4], const bf16x8 (&a)[2], const bf16x8 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
}

// acc = A_tile * B_tile^T over KT2 stages of 64.  Wave w (wm = w/2, wn = w%2)
// owns fragments i = 0, 1 at tile rows 128i + 32wm .. +31 and j = 0..3 at tile
// columns 128wn + 32j .. +31; NV = fragments holding a valid row.  aoff/boff:
// byte offsets of the 4 A and 4 B rows this lane loads per stage (tile rows
// 32w + 8i + lane/8, swizzled chunk); kit.next() yields each stage's K offset.
// load_a (wave-uniform): false for waves 4..7 of a half tile, whose A rows lie
// outside the tile; they load only their B rows (no wave reads those A rows).
// kChain: the tile starts as `en` says, and with ln.next the two loads past
// its last stage fetch the successor's stages 0 and 1 (dense K: stage j at
// j * kRow8 bytes into the rows).
template <int NV, class KIt, bool kChain = false>
__device__ __forceinline__ void tile_mainloop8(floatx16 (&acc)[2][4], uint8_t* smem, const char* a_base,
                                               const uint32_t (&aoff)[4], const char* b_base,
                                               const uint32_t (&boff)[4], int KT2, KIt kit, bool load_a = true,
                                               TileEntry en = {}, TileLink ln = {}) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
    if (KT2 <= 0) return;
    // Past the last stage the loads repeat it into the slot no wave reads any
    // more (no branch, constant vmcnt waits), or load the successor's first
    // stages.
    int64_t ka = 0, kb = 0;
    const char* ab = a_base;
    const char* bb = b_base;
    bool la = load_a;
    int issued = 0;
    auto advance = [&]() {
        if (issued < KT2) {
            kit.next(ka, kb);
        } else if (kChain && ln.next) {
            ab = ln.na;
            bb = ln.nb;
            la = ln.next_load_a;
            ka = kb = (int64_t)(issued - KT2) * kRow8;
        }
        ++issued;
    };
    // load q of this lane for the stage going into `slot`: q = 0..3 its A rows,
    // 4..7 its B rows
    auto load1 = [&](int slot, int q) {
        uint8_t* base = smem + slot * kStageBytes8 + (wave * 32) * kRow8;
        if (q < 4) {
            if (la)
                __builtin_amdgcn_global_load_lds((gbl_cvoid*)(ab + ka + aoff[q]), (lds_void*)(base + q * 1024), 16,
                                                 0, 0);
        } else {
            __builtin_amdgcn_global_load_lds((gbl_cvoid*)(bb + kb + boff[q - 4]),
                                             (lds_void*)(base + kStageA8 + (q - 4) * 1024), 16, 0, 0);
        }
    };
    const int fr = lane & 31;
    const int arow_b = (wm * 32 + fr) * kRow8, brow_b = kStageA8 + (wn * 128 + fr) * kRow8;
    const int fsw = swz8(fr);  // a fragment's rows differ from fr by multiples of 32
    // fragment f of k-step kk of the stage in `slot`: f = 0, 1 A rows, 2..5 B rows
    auto frag1 = [&](int slot, int kk, int f, bf16x8 (&a)[2], bf16x8 (&b)[4]) {
        const uint8_t* st = smem + slot * kStageBytes8;
        const int pc = ((kk * 2 + (lane >> 5)) ^ fsw) * 16;
        if (f < 2) {
            if (f < NV) a[f] = *(const bf16x8*)(st + arow_b + f * 128 * kRow8 + pc);
        } else {
            b[f - 2] = *(const bf16x8*)(st + brow_b + (f - 2) * 32 * kRow8 + pc);
        }
    };
    auto frags = [&](int slot, int kk, bf16x8 (&a)[2], bf16x8 (&b)[4]) {
#pragma unroll
        for (int f = 0; f < 6; ++f) frag1(slot, kk, f, a, b);
    };
    // Ring protocol (stage j in slot j % 2, 8 direct-to-LDS loads per lane
    // and stage, 4 for a wave without A rows, counted by vmcnt): the prologue
    // issues stages 0 and 1 and waits for stage 0; stage s runs four k-steps of
    // 8 MFMAs, each reading the next k-step's fragments; before the last one
    // it waits for stage s+1 (vmcnt(0)) and its own LDS reads (lgkmcnt(0)),
    // then a barrier: no wave reads stage s any more, so its slot takes stage
    // s+2.  Those loads, and the next stage's first fragment reads, go out one
    // per MFMA of the last k-step, pinned in that order: issued as a burst
    // after the barrier, the eight waves' loads stalled their own MFMAs behind
    // the busy load path (probe on the dense 20480 x 4096 x 7168 and
    // 20480 x 7168 x 2048 GEMMs: +7% and +9%, same bits).  First the previous
    // tile's stores leave the count and every wave is done with the previous
    // tile's LDS.  A chained tile's stages 0 and 1 went out with its
    // predecessor's last two; stage 0 was waited for before the predecessor's
    // last barrier, and stage 1 is waited for, with the predecessor's stores,
    // at the first stage's end.
    const int s0 = kChain ? en.slot0 : 0;
    if (kChain && en.pre) {
        advance();
        advance();
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        advance();
#pragma unroll
        for (int q = 0; q < 8; ++q) load1(s0, q);
        advance();
#pragma unroll
        for (int q = 0; q < 8; ++q) load1(s0 ^ 1, q);
        if (load_a)
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        __syncthreads();
    }
    bf16x8 a0[2], b0[4], a1[2], b1[4];
    frags(s0, 0, a0, b0);
    int slot = s0;
    for (int s = 0; s < KT2; ++s) {
        frags(slot, 1, a1, b1);
        mfma_block8<NV>(acc, a0, b0);
        Interleave<4 * NV, 0, NV + 4>::run();
        __builtin_amdgcn_sched_barrier(0);
        frags(slot, 2, a0, b0);
        mfma_block8<NV>(acc, a1, b1);
        Interleave<4 * NV, 0, NV + 4>::run();
        __builtin_amdgcn_sched_barrier(0);
        frags(slot, 3, a1, b1);
        mfma_block8<NV>(acc, a0, b0);
        Interleave<4 * NV, 0, NV + 4>::run();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        advance();  // offsets of stage s + 2
        // MFMA m of the last k-step, then load m of stage s + 2, then
        // fragment read m of the next stage's first k-step (a stale but
        // in-bounds read after the last stage)
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int i = m >> 2, j = m & 3;
            if (i < NV) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[j], a1[i], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            load1(slot, m);
            __builtin_amdgcn_sched_barrier(0);
            if (m < 6) frag1(slot ^ 1, 0, m, a0, b0);
            __builtin_amdgcn_sched_barrier(0);
        }
        slot ^= 1;
    }
}

// K sequence of a dense GEMM in 64-deep stages: stage s sits s * 128 bytes
// into every row.
struct DenseK8 {
    int kt = 0;
    __device__ __forceinline__ void next(int64_t& a_off, int64_t& b_off) {
        a_off = b_off = (int64_t)kt * kRow8;
        ++kt;
    }
};

// ---------------------------------------------------------------------------
// Token-major operands (the weight-gradient GEMMs, which contract over token
// rows): a stage holds 64 K rows of 256 columns (512 bytes) of each operand,
// in the same 2 x 64 KB ring and with the same direct-to-LDS loads as the
// eight-wave tile (load q of wave w fills K rows 2(4w + q) and 2(4w + q) + 1,
// lane l row 2(4w + q) + l/32 and LDS chunk l % 32).  The MFMA fragments need
// eight K-consecutive values per lane; gfx950's transposing LDS read
// ds_read_b64_tr_b16 gathers them: within each group of 16 lanes every lane
// points at four consecutive 16-bit elements of a row, and lane j receives
// element j % 4 of the rows that lanes j/4 + 4q point at (q = 0..3).  So lane
// j = 4c + s of a group points at K row k0 + j/4, columns c0 + 4(j % 4) ..,
// and receives column c0 + j at K rows k0 .. k0 + 3; two reads make a
// fragment.  A K row's 16-byte chunk c sits at position c ^ 4(kr % 4), so the
// four K rows of a read fall on distinct banks.
// ---------------------------------------------------------------------------
constexpr int kRowT = BM * 2;  // bytes of one K row of a stage
static_assert(kRowT * kBK8 == kStageA8, "a token-major stage fills the same ring slot");

// Logical 16-byte chunk that lane `lane`'s load q brings into its fixed LDS
// position (K row 2(4w + q) + lane/32, chunk lane % 32); depends on q % 2 only.
__device__ __forceinline__ int kmajor_chunk(int lane, int q) {
    return (lane & 31) ^ (4 * (2 * (q & 1) + (lane >> 5)));
}

// acc = A^T B over KT2 stages of 64 token rows, A and B token-major (tile
// columns m0.. of A, n0.. of B).  kit.next(pa, pb) yields each stage's eight
// per-lane load addresses (pa[q], pb[q]: load q of this lane).  A k-step's
// twelve fragment reads go out in one asm block together with four MFMAs of
// the previous k-step and end with the block's own lgkmcnt wait, so the
// reads' latency lies under those MFMAs.  (Written as builtins, the compiler,
// unable to tell the transposing reads from the ring's direct-to-LDS writes,
// waits for every load in flight before each of them.)  Same accumulator
// layout and ring protocol as tile_mainloop8.
template <class KIt>
__device__ __forceinline__ void tile_mainloop8t(floatx16 (&acc)[2][4], uint8_t* smem, int KT2, KIt& kit) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
    if (KT2 <= 0) return;
    const char* pa[4];
    const char* pb[4];
    int issued = 0;
    auto advance = [&]() {
        if (issued < KT2) kit.next(pa, pb);
        ++issued;
    };
    auto load1 = [&](int slot, int q) {
        uint8_t* base = smem + slot * kStageBytes8 + wave * 4096;
        if (q < 4)
            __builtin_amdgcn_global_load_lds((gbl_cvoid*)pa[q], (lds_void*)(base + q * 1024), 16, 0, 0);
        else
            __builtin_amdgcn_global_load_lds((gbl_cvoid*)pb[q - 4], (lds_void*)(base + kStageA8 + (q - 4) * 1024),
                                             16, 0, 0);
    };
    // this lane's read: group g = lane/16, j = lane % 16; K row 8(g/2) + j/4
    // (+4 for the second read of a fragment), columns 16(g % 2) + 4(j % 4) of
    // the fragment's 32; the swizzle term 4(j/4) lands in the chunk bits that
    // hold the fragment's 32-column block
    const int tg = lane >> 4, tj = lane & 15;
    const int tsub = (8 * (tg >> 1) + (tj >> 2)) * kRowT + (2 * (tg & 1) + ((tj >> 1) & 1)) * 16 + 8 * (tj & 1);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    const uint32_t ta = lds0 + tsub + 64 * (wm ^ (tj >> 2));
    uint32_t tb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tb[j] = lds0 + kStageA8 + tsub + 256 * wn + 64 * (j ^ (tj >> 2));
    typedef int intx2 __attribute__((ext_vector_type(2)));
    // Reads of k-step kk of the stage in `slot` into (an, bn); with them the
    // four MFMAs of fragment row I of the previous k-step, on (a, b), then the
    // wait.  Every accumulator the asm MFMAs write is next read by an MFMA or
    // a store at least four MFMAs later.
    auto rd_mfma = [&](int slot, auto kkc, auto ic, const bf16x8 (&a)[2], const bf16x8 (&b)[4], bf16x8 (&an)[2],
                       bf16x8 (&bn)[4]) {
        constexpr int K0 = decltype(kkc)::value * 16 * kRowT;
        constexpr int I = decltype(ic)::value;
        const uint32_t so = slot * kStageBytes8;
        intx2 r[12];
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16 offset:%26\n"
            "ds_read_b64_tr_b16 %1, %16 offset:%27\n"
            "ds_read_b64_tr_b16 %2, %16 offset:%28\n"
            "ds_read_b64_tr_b16 %3, %16 offset:%29\n"
            "ds_read_b64_tr_b16 %4, %17 offset:%26\n"
            "ds_read_b64_tr_b16 %5, %17 offset:%27\n"
            "ds_read_b64_tr_b16 %6, %18 offset:%26\n"
            "ds_read_b64_tr_b16 %7, %18 offset:%27\n"
            "ds_read_b64_tr_b16 %8, %19 offset:%26\n"
            "ds_read_b64_tr_b16 %9, %19 offset:%27\n"
            "ds_read_b64_tr_b16 %10, %20 offset:%26\n"
            "ds_read_b64_tr_b16 %11, %20 offset:%27\n"
            "v_mfma_f32_32x32x16_bf16 %12, %22, %21, %12\n"
            "v_mfma_f32_32x32x16_bf16 %13, %23, %21, %13\n"
            "v_mfma_f32_32x32x16_bf16 %14, %24, %21, %14\n"
            "v_mfma_f32_32x32x16_bf16 %15, %25, %21, %15\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
              "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
              "+v"(acc[I][0]), "+v"(acc[I][1]), "+v"(acc[I][2]), "+v"(acc[I][3])
            : "v"(ta + so), "v"(tb[0] + so), "v"(tb[1] + so), "v"(tb[2] + so), "v"(tb[3] + so), "v"(a[I]),
              "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "i"(K0), "i"(K0 + 4 * kRowT), "i"(K0 + 256),
              "i"(K0 + 4 * kRowT + 256)
            : "memory");
        an[0] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3));
        an[1] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[2], r[3], 0, 1, 2, 3));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bn[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[4 + 2 * j], r[5 + 2 * j], 0, 1, 2, 3));
    };
    auto mfma_row = [&](int i, const bf16x8 (&a)[2], const bf16x8 (&b)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    };
    using KS0 = std::integral_constant<int, 0>;
    using KS1 = std::integral_constant<int, 1>;
    using KS2 = std::integral_constant<int, 2>;
    using KS3 = std::integral_constant<int, 3>;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    advance();
#pragma unroll
    for (int q = 0; q < 8; ++q) load1(0, q);
    advance();
#pragma unroll
    for (int q = 0; q < 8; ++q) load1(1, q);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    __syncthreads();
    bf16x8 a0[2], b0[4], a1[2], b1[4];
    {
        // k-step 0 of stage 0: its reads cover no MFMA yet (acc is zero, so
        // the block's four MFMAs on the zero fragments below add nothing)
#pragma unroll
        for (int i = 0; i < 2; ++i) a1[i] = bf16x8{};
#pragma unroll
        for (int j = 0; j < 4; ++j) b1[j] = bf16x8{};
        rd_mfma(0, KS0{}, I0{}, a1, b1, a0, b0);
    }
    int slot = 0;
    for (int s = 0; s < KT2; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        rd_mfma(slot, KS1{}, I0{}, a0, b0, a1, b1);
        mfma_row(1, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        rd_mfma(slot, KS2{}, I0{}, a1, b1, a0, b0);
        mfma_row(1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        rd_mfma(slot, KS3{}, I0{}, a0, b0, a1, b1);
        mfma_row(1, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        advance();  // addresses of stage s + 2
        // the last k-step: fragment row 0's MFMAs with the A loads of stage
        // s + 2 between them, then the next stage's first reads (a stale but
        // in-bounds read after the last stage) under fragment row 1's MFMAs,
        // then the B loads
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            acc[0][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[m], a1[0], acc[0][m], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            load1(slot, m);
            __builtin_amdgcn_sched_barrier(0);
        }
        rd_mfma(slot ^ 1, KS0{}, I1{}, a1, b1, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 4; q < 8; ++q) load1(slot, q);
        __builtin_amdgcn_sched_barrier(0);
        slot ^= 1;
    }
    // the last asm MFMAs' results reach VALU reads in the caller's epilogue:
    // wait states the compiler cannot count through the asm
    asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
}

// How a tile treats the padding rows of an expert's last tile (with
// p.rows_e): kPadNone runs every fragment, a half tile's too; kPadPerWave
// drops each wave's fragments that hold only padding rows (a mainloop variant
// per count of valid fragments) and a half tile's A loads past its rows.
constexpr int kPadNone = 0, kPadPerWave = 1;

// One 256 x 256 output tile (expert e, M tile ml of the expert, N tile ntile)
// of the bf16 grouped GEMM with its epilogue, by 512 threads; smem is the
// kTileSmem LDS ring.  Padding rows are skipped as kPad says (their outputs
// are then zero; no caller reads them).  kChain (plain bf16 stores, no row
// scale, smem holding kTileSmem + kStgBytes): the tile starts as *en says,
// loads its successor's first stages as *ln says, and sets *en for the
// successor.
template <int EPI, int kPad = kPadPerWave, bool kChain = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs p, int e, int ml, int ntile, uint8_t* smem,
                                          TileEntry* en = nullptr, const TileLink* ln = nullptr) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1;
    const int KT2 = p.K / kBK8;
    // (chained: scalar loads, which do not wait for the loads and stores in
    // flight from the previous tile)
    auto lay = [&](const int32_t* q) -> int { return kChain ? ld_layout(q) : *q; };
    const int seg0 = lay(p.prow_start + e);
    const int prow0 = seg0 + ml * BM;
    // BM rows, or kSegRows for an expert's last tile when it is a half tile:
    // then the second row of fragments lies outside the tile and is skipped
    const int trows = tile_rows_of(seg0, lay(p.prow_start + e + 1), ml);
    const int n0 = ntile * BN;

    // Byte offsets of the 4 A rows and 4 B rows this lane loads per stage:
    // instruction i fills tile rows 32*wave + 8i .. +7 (lane/8 picks the row,
    // lane%8 the fixed LDS chunk; the lane loads the logical chunk stored there).
    // A half tile's rows past kSegRows load its own rows again (cache hits):
    // no read leaves the tile.
    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wave * 32 + i * 8 + (lane >> 3);
        const int lchunk = (lane & 7) ^ swz8(r);
        const int prow = prow0 + (r & (trows - 1));
        const int arow = p.a_row_map ? p.a_row_map[prow] : prow;
        aoff[i] = (uint32_t)(((int64_t)arow * p.lda + lchunk * 8) * 2);
        const int n = min(n0 + r, p.N - 1);
        boff[i] = (uint32_t)(((int64_t)n * p.K + lchunk * 8) * 2);
    }
    floatx16 acc[2][4];
    const char* bbase = (const char*)(p.B + (int64_t)e * p.b_stride);
    // kPadNone runs a half tile at full work (both fragment rows, every A load;
    // its rows past kSegRows repeat its own rows and are not stored)
    int nv = (kPad == kPadNone || trows == BM) ? 2 : 1;
    if (kPad != kPadNone && p.rows_e) {
        // fragment i of this wave holds tile rows 128i + 32wm .. +31
        const int valid = lay(p.rows_e + e) - ml * BM, w32 = __builtin_amdgcn_readfirstlane(wm) * 32;
        nv = valid > 128 + w32 ? 2 : (valid > w32 ? 1 : 0);
    }
    // waves 4..7 hold tile rows 128..255: none of them in a half tile
    const bool load_a = kPad == kPadNone || trows == BM || __builtin_amdgcn_readfirstlane(wave) < 4;
    const TileEntry te = kChain ? *en : TileEntry{};
    const TileLink tl = kChain ? *ln : TileLink{};
    switch (nv) {
        case 2:
            tile_mainloop8<2, DenseK8, kChain>(acc, smem, (const char*)p.A, aoff, bbase, boff, KT2, DenseK8{}, load_a,
                                               te, tl);
            break;
        case 1:
            tile_mainloop8<1, DenseK8, kChain>(acc, smem, (const char*)p.A, aoff, bbase, boff, KT2, DenseK8{}, load_a,
                                               te, tl);
            break;
        default:
            tile_mainloop8<0, DenseK8, kChain>(acc, smem, (const char*)p.A, aoff, bbase, boff, KT2, DenseK8{}, load_a,
                                               te, tl);
            break;
    }
    if constexpr (kChain) {
        en->pre = tl.next;
        en->slot0 = te.slot0 ^ (KT2 & 1);
    }

    if constexpr (kChain && EPI == kEpiStore) {
        if (!p.Cf && !p.row_scale) {
            // Staged through the block past the ring: 64 rows of 512 bytes,
            // the 16-byte chunk c of row r at c ^ (r % 32), so the 32 rows of
            // a staging write and the two rows of a copy-out read fall on
            // distinct banks.  Its LDS accesses are asm and its barriers
            // LDS-only: nothing here waits for the successor's loads in flight
            // (the compiler would make LDS accesses, and __syncthreads, wait
            // for every direct-to-LDS load).  Without a successor the loads
            // past the last stage land first, as in the plain epilogue.
            if (!tl.next) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const uint32_t stg = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem + kTileSmem;
            // lane-only addresses from an opaque copy of the thread index, so
            // they are formed here rather than hoisted out of the tile loop
            // (kept live across it they spill)
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int rl = ((tid >> 7) & 1) * 32 + (tid & 31);  // row in the block: (wm % 2) * 32 + lane % 32
            const uint32_t wrow = stg + rl * kStgPitch + 8 * ((tid >> 5) & 1);
            const int wc0 = ((tid >> 6) & 1) * 16;  // chunk of fragment column 0: 128 wn columns
            const int r0 = tid >> 5, ch = tid & 31;
            const bool col_in = ch * 16 < (p.N - n0) * 2;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if (b * kEpiRows >= trows) break;  // a half tile stores its kSegRows rows only
                if ((wm >> 1) == (b & 1)) {
                    const int i = b >> 1;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            // frag_col(j, q) * 2 bytes: chunk wc0 + 4j + q, byte 8 * (lane / 32) in it
                            const uint32_t la = wrow + (((wc0 + 4 * j + q) ^ (rl & 31)) << 4);
                            const uint2 pv = pack_bf16x4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                                         acc[i][j][4 * q + 3]);
                            const u32x2 v2 = {pv.x, pv.y};
                            asm volatile("ds_write_b64 %0, %1" ::"v"(la), "v"(v2) : "memory");
                        }
                }
                lds_barrier();
                // thread t: rows t/32 + 16k (k = 0..3) of the block, chunk t % 32
                uint32_t ra[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) ra[k] = stg + (r0 + 16 * k) * kStgPitch + ((ch ^ ((r0 + 16 * k) & 31)) << 4);
                u32x4 d0, d1, d2, d3;
                asm volatile(
                    "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
                    : "v"(ra[0]), "v"(ra[1]), "v"(ra[2]), "v"(ra[3])
                    : "memory");
                char* dst = (char*)(p.C + (int64_t)(prow0 + b * 64 + r0) * p.ldc + n0) + ch * 16;
                const int64_t ld16 = (int64_t)p.ldc * 2 * 16;
                if (col_in) {
                    *(u32x4*)dst = d0;
                    *(u32x4*)(dst + ld16) = d1;
                    *(u32x4*)(dst + 2 * ld16) = d2;
                    *(u32x4*)(dst + 3 * ld16) = d3;
                }
                lds_barrier();
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
    const int rl = (wm & 1) * 32 + (lane & 31);
    if (EPI == kEpiSwiGLU) {
        // columns come in 64-wide groups of 32 gate then 32 up columns
        const int I = p.N / 2, hc0 = n0 / 2;
        const bool f32gu = p.GUf != nullptr, anygu = f32gu || p.GU != nullptr;
        uint8_t* hb = smem;                                  // [64][128] bf16
        uint8_t* gb = smem + kEpiRows * kEpiPitch16;         // [64][128] fp32 or bf16
        uint8_t* ub = gb + kEpiRows * kEpiPitch32;
        const int gpitch = f32gu ? kEpiPitch32 : kEpiPitch16;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b * kEpiRows >= trows) break;  // a half tile stores its kSegRows rows only
            if ((wm >> 1) == (b & 1)) {
                const int i = b >> 1;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int hc = (wave & 1) * 64 + jj * 32 + q * 8 + 4 * (lane >> 5);
                        float g[4], u[4], h[4];
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            g[s] = acc[i][2 * jj][4 * q + s];
                            u[s] = acc[i][2 * jj + 1][4 * q + s];
                            h[s] = swiglu(g[s], u[s]);
                        }
                        *(uint2*)(hb + rl * kEpiPitch16 + hc * 2) = pack_bf16x4(h[0], h[1], h[2], h[3]);
                        if (f32gu) {
                            *(floatx4*)(gb + rl * kEpiPitch32 + hc * 4) = floatx4{g[0], g[1], g[2], g[3]};
                            *(floatx4*)(ub + rl * kEpiPitch32 + hc * 4) = floatx4{u[0], u[1], u[2], u[3]};
                        } else if (anygu) {
                            *(uint2*)(gb + rl * kEpiPitch16 + hc * 2) = pack_bf16x4(g[0], g[1], g[2], g[3]);
                            *(uint2*)(ub + rl * kEpiPitch16 + hc * 2) = pack_bf16x4(u[0], u[1], u[2], u[3]);
                        }
                    }
            }
            __syncthreads();
            const int64_t row0 = prow0 + b * 64;
            const int lim = I - hc0;
            epi_copy_out<16, kTileThreads>(hb, kEpiPitch16, (char*)(p.C + row0 * p.ldc + hc0), (int64_t)p.ldc * 2,
                                           lim * 2);
            if (f32gu) {
                epi_copy_out<32, kTileThreads>(gb, gpitch, (char*)(p.GUf + row0 * 2 * I + hc0), (int64_t)I * 8,
                                               lim * 4);
                epi_copy_out<32, kTileThreads>(ub, gpitch, (char*)(p.GUf + row0 * 2 * I + I + hc0),
                                               (int64_t)I * 8, lim * 4);
            } else if (anygu) {
                epi_copy_out<16, kTileThreads>(gb, gpitch, (char*)(p.GU + row0 * 2 * I + hc0), (int64_t)I * 4,
                                               lim * 2);
                epi_copy_out<16, kTileThreads>(ub, gpitch, (char*)(p.GU + row0 * 2 * I + I + hc0),
                                               (int64_t)I * 4, lim * 2);
            }
            __syncthreads();
        }
    } else if (p.Cf) {  // kEpiStore, fp32 output
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b * kEpiRows >= trows) break;  // a half tile stores its kSegRows rows only
            if ((wm >> 1) == (b & 1)) {
                const int i = b >> 1;
                const float sc = p.row_scale ? p.row_scale[prow0 + b * 64 + rl] : 1.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(floatx4*)(smem + rl * kEpiPitch64 + frag_col(j, q) * 4) =
                            floatx4{acc[i][j][4 * q] * sc, acc[i][j][4 * q + 1] * sc, acc[i][j][4 * q + 2] * sc,
                                    acc[i][j][4 * q + 3] * sc};
            }
            __syncthreads();
            epi_copy_out<64, kTileThreads>(smem, kEpiPitch64, (char*)(p.Cf + (int64_t)(prow0 + b * 64) * p.ldc + n0),
                                           (int64_t)p.ldc * 4, (p.N - n0) * 4);
            __syncthreads();
        }
    } else {  // kEpiStore, bf16 output
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b * kEpiRows >= trows) break;  // a half tile stores its kSegRows rows only
            if ((wm >> 1) == (b & 1)) {
                const int i = b >> 1;
                const float sc = p.row_scale ? p.row_scale[prow0 + b * 64 + rl] : 1.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(uint2*)(smem + rl * kEpiPitch32 + frag_col(j, q) * 2) =
                            pack_bf16x4(acc[i][j][4 * q] * sc, acc[i][j][4 * q + 1] * sc, acc[i][j][4 * q + 2] * sc,
                                        acc[i][j][4 * q + 3] * sc);
            }
            __syncthreads();
            epi_copy_out<32, kTileThreads>(smem, kEpiPitch32, (char*)(p.C + (int64_t)(prow0 + b * 64) * p.ldc + n0),
                                           (int64_t)p.ldc * 2, (p.N - n0) * 2);
            __syncthreads();
        }
    }
}

// Whether a launch's kEpiStore tiles can chain: bf16 output without row
// scales, A rows read directly, whole N tiles, and at least two stages.
__device__ __forceinline__ bool tiles_chain(const GemmArgs& p) {
    return p.C && !p.Cf && !p.row_scale && !p.a_row_map && p.N % BN == 0 && p.K >= 2 * kBK8;
}

// The link from tile (p, e, ml, ntile) to its successor (pn, e2, ml2, nt2) of
// the same GEMM (equal lda, K and N; A rows direct; kPadPerWave): gemm_tile's
// load offsets of a lane are ((prow0 + r') lda + chunk) * 2 bytes into p.A
// and ((n0 + r) K + chunk) * 2 into expert e's B, with r' = r except for the
// waves 4..7 of a half tile (r - 128, which that tile does not load).
__device__ __forceinline__ TileLink tile_link(const GemmArgs& p, int e, int ml, int ntile, const GemmArgs& pn, int e2,
                                              int ml2, int nt2) {
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int seg0 = ld_layout(p.prow_start + e), prow0 = seg0 + ml * BM;
    const int trows = tile_rows_of(seg0, ld_layout(p.prow_start + e + 1), ml);
    const int seg2 = ld_layout(pn.prow_start + e2), prow2 = seg2 + ml2 * BM;
    const int trows2 = tile_rows_of(seg2, ld_layout(pn.prow_start + e2 + 1), ml2);
    const int64_t dr = (int64_t)(prow2 - prow0) + ((wave >= 4 && trows < BM) ? BM - kSegRows : 0);
    TileLink ln;
    ln.na = (const char*)pn.A + dr * p.lda * 2;
    ln.nb = (const char*)(pn.B + (int64_t)e2 * pn.b_stride) + (int64_t)(nt2 - ntile) * BN * p.K * 2;
    ln.next_load_a = trows2 == BM || wave < 4;
    ln.next = true;
    return ln;
}

// ---------------------------------------------------------------------------
// Weight-gradient tiles, shared by the bf16 and MXFP8 kernels.  Every expert's
// MT x NT grid of 256 x 256 output tiles is cut into mq x nq = 8 blocks, block
// (xcd % mq, xcd / mq) going to XCD xcd (workgroups are dealt to the 8 XCDs
// round-robin), so each A panel is fetched into nq XCDs' L2s and each B panel
// into mq.  An XCD's workgroups walk its blocks expert by expert, M tile
// fastest.
// ---------------------------------------------------------------------------
struct WgradTiles {
    int mlo, nlo, bmt, bnt, cnt, per, local, G;
    __device__ WgradTiles(int M, int N, int mq, int nq) {
        const int MT = ceil_div(M, BM), NT = ceil_div(N, BN);
        const int xcd = blockIdx.x & 7, bm = xcd % mq, bn = xcd / mq;
        per = gridDim.x >> 3;
        local = blockIdx.x >> 3;
        mlo = bm * MT / mq;
        nlo = bn * NT / nq;
        bmt = (bm + 1) * MT / mq - mlo;
        bnt = (bn + 1) * NT / nq - nlo;
        cnt = bmt * bnt;
        // a block's M tiles in groups of G, a group's tiles together (M
        // fastest): the XCD's `per` workgroups then run a G x bnt patch at a
        // time, each A panel read by bnt of them at once and each B panel by G
        G = per / bnt > 1 ? per / bnt : 1;
    }
    // this workgroup's tile number `it` over experts [0, Et): false past the last
    __device__ bool get(int it, int Et, int& e, int& m0, int& n0) const {
        const int li = it * per + local;
        if (cnt == 0 || li >= Et * cnt) return false;
        e = li / cnt;
        const int t = li - e * cnt;
        const int g = t / (G * bnt), tt = t - g * G * bnt;
        const int gs = bmt - g * G < G ? bmt - g * G : G;  // M tiles of group g
        m0 = (mlo + g * G + tt % gs) * BM;
        n0 = (nlo + tt / gs) * BN;
        return true;
    }
};

// The XCD cut with the least L2 fill traffic: A panels (M rows) land in nq
// XCDs, B panels (N rows) in mq.
inline void wgrad_cut(int M, int N, int& mq, int& nq) {
    const int64_t cost[4] = {(int64_t)M + 8ll * N, 2ll * M + 4ll * N, 4ll * M + 2ll * N, 8ll * M + N};
    int best = 0;
    for (int i = 1; i < 4; ++i)
        if (cost[i] < cost[best]) best = i;
    mq = 8 >> best;
    nq = 1 << best;
}

// Stores a 256 x 256 fp32 weight-gradient tile (accumulators in the tiles'
// fragment layout) at rows m0.., columns n0..: columns < n_split to c0
// [M][n_split], the rest to c1 [M][N - n_split] at column - n_split.  Straight
// from the registers: each store writes 16 bytes (a run of four columns) of 32
// rows per half-wave, and the four runs of a fragment fill 128 contiguous
// bytes of each row.  Staged through LDS as whole rows instead (four 64-row
// blocks, two barriers each) the MXFP8 weight gradients of 16384 tokens at
// H=7168, I=2048, E=32, k=8 took 7.72 ms per step against 7.22 ms; with
// non-temporal stores 9.23 ms.  M, N and n_split are multiples of 64: a run
// lies on one side of the split and inside or outside the matrix as a whole.
__device__ __forceinline__ void wgrad_store(const floatx16 (&acc)[2][4], int m0, int n0, int M, int N, int n_split,
                                            float* c0, float* c1) {
    const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) >> 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + 128 * i + 32 * wm + (lane & 31);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + frag_col(j, q);
                if (m >= M || col >= N) continue;
                float* dst = col < n_split ? c0 + (int64_t)m * n_split + col
                                           : c1 + (int64_t)m * (N - n_split) + (col - n_split);
                *(floatx4*)dst = floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                         acc[i][j][4 * q + 3]};
            }
    }
}

__device__ __forceinline__ void bf16x8_to_f32(const intx4 raw, float* f) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t v = (uint32_t)raw[q];
        f[2 * q] = __builtin_bit_cast(float, v << 16);
        f[2 * q + 1] = __builtin_bit_cast(float, v & 0xffff0000u);
    }
}

// Combine of one token by nthreads threads (thread index tid):
//   out[h] = bf16( sum_j fmaf(w[j], Y[rows[j]][h]) (+ Y[rows[k]][h]) ), j ascending,
// the routed slots first in slot order, then the shared expert's row.
__device__ __forceinline__ void combine_token(const uint16_t* __restrict__ Y, int64_t ldy, const int* rows,
                                              const float* w, int k, int with_shared, int H,
                                              uint16_t* __restrict__ out, int tid, int nthreads) {
    for (int c = tid; c < H / 8; c += nthreads) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        for (int j = 0; j < k; ++j) {
            float y[8];
            bf16x8_to_f32(*(const intx4*)(Y + (int64_t)rows[j] * ldy + c * 8), y);
            const float wj = w[j];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(wj, y[q], acc[q]);
        }
        if (with_shared) {
            float y[8];
            bf16x8_to_f32(*(const intx4*)(Y + (int64_t)rows[k] * ldy + c * 8), y);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = acc[q] + y[q];
        }
        intx4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = (int)((uint32_t)f32_to_bf16_rne(acc[2 * q]) | ((uint32_t)f32_to_bf16_rne(acc[2 * q + 1]) << 16));
        *(intx4*)(out + c * 8) = o;
    }
}

// Combine of up to kTok tokens by one workgroup, every load of a chunk issued
// before its arithmetic (memory-level parallelism for the few workgroups of
// the layer kernel's combine role).  rows[t][kMaxTopK + 1], w[t][kMaxTopK];
// tokens t < ntok are written to out_rows[t].  Same arithmetic per element as
// combine_token.
template <int kTok>
__device__ __forceinline__ void combine_tokens_mlp(const uint16_t* __restrict__ Y, int64_t ldy, const int (*rows)[kMaxTopK + 1],
                                                   const float (*w)[kMaxTopK], int ntok, int k, int with_shared, int H,
                                                   uint16_t* const* out_rows, int tid, int nthreads) {
    for (int c = tid; c < H / 8; c += nthreads) {
        float acc[kTok][8];
#pragma unroll
        for (int t = 0; t < kTok; ++t)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[t][q] = 0.0f;
        int j = 0;
        for (; j + 4 <= k; j += 4) {  // 4 slots x kTok tokens of loads in flight
            intx4 raw[kTok][4];
#pragma unroll
            for (int t = 0; t < kTok; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    raw[t][u] = t < ntok ? *(const intx4*)(Y + (int64_t)rows[t][j + u] * ldy + c * 8) : intx4{};
#pragma unroll
            for (int t = 0; t < kTok; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float y[8];
                    bf16x8_to_f32(raw[t][u], y);
                    const float wj = w[t][j + u];
#pragma unroll
                    for (int q = 0; q < 8; ++q) acc[t][q] = __builtin_fmaf(wj, y[q], acc[t][q]);
                }
        }
        for (; j < k; ++j) {
#pragma unroll
            for (int t = 0; t < kTok; ++t) {
                if (t >= ntok) continue;
                float y[8];
                bf16x8_to_f32(*(const intx4*)(Y + (int64_t)rows[t][j] * ldy + c * 8), y);
                const float wj = w[t][j];
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[t][q] = __builtin_fmaf(wj, y[q], acc[t][q]);
            }
        }
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
            if (t >= ntok) continue;
            if (with_shared) {
                float y[8];
                bf16x8_to_f32(*(const intx4*)(Y + (int64_t)rows[t][k] * ldy + c * 8), y);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[t][q] = acc[t][q] + y[q];
            }
            intx4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = (int)((uint32_t)f32_to_bf16_rne(acc[t][2 * q]) | ((uint32_t)f32_to_bf16_rne(acc[t][2 * q + 1]) << 16));
            *(intx4*)(out_rows[t] + c * 8) = o;
        }
    }
}

}  // namespace moe
