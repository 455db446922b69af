// Persistent layer kernel: the expert FFN of every minibatch and its combine
// in one cooperative launch.
//
// MoK runs the MoE layer as one persistent megakernel: a few SMs move tokens
// (dispatch / combine) while the rest run the grouped GEMMs, the two sides
// signal each other through counters in device memory with no host round
// trip, a fixed ring of token slots is reused as soon as combine has drained
// one, and a minibatch is sized so the GEMM side keeps at least two full waves
// of tiles (KuCoin flash "Cursor's MoK achieves 2.37x performance boost on
// NVIDIA GB300 NVL72", sections 01-03; RuntimeWire "Cursor open-sources MoK",
// "Rebuilding the MoE layer around communication").
//
// On one MI355X the layout of every minibatch is computed before this launch
// (one workgroup per minibatch) and the dispatch gather is the GEMM's own
// row-mapped direct-to-LDS load, so the token-moving work is combine.  The
// GEMM workgroups walk one static sequence of tiles, dealt XCD-aware as in the
// one-GEMM-per-launch kernels: step s holds gate|up(s), then down(s-1), then
// combine(s-2) when combine runs as tiles:
//   gate|up(0), gate|up(1), down(0), gate|up(2), down(1), [combine(0),] ...
// The skew puts at least one phase between a phase and the one that reads its
// output, so inputs are rarely unfinished when a workgroup reaches them, and a
// workgroup waits at most once per phase.  Combine runs either
//   * on comm dedicated workgroups (blockIdx < comm), minibatch by minibatch,
//     as MoK splits its SMs between communication and GEMM work, or
//   * (comm = 0) as tiles of 16 tokens in the same sequence, so that every CU
//     runs GEMM tiles: on one GPU combine is a few per cent of the layer.
// Groups and ring: the phases run over groups of `group` consecutive
// minibatches (the GEMM tiles of a group share each expert's weight panels);
// minibatch b writes h (and, without saved outputs, Y) into slot b % S, S a
// multiple of group, so group j holds Sg = S / group slot groups.  Gate|up(j)
// waits until down(j-Sg) -- and combine(j-Sg) when Y is in the ring -- are
// done.  Every wait depends only on phases earlier in the sequence (Sg >= 2,
// and Sg >= 3 for combine tiles with Y in the ring) or on the dedicated
// combine workgroups, which only wait on earlier down phases; every workgroup
// takes its tiles in sequence order, so the launch always drains (all
// workgroups are co-resident: it is a cooperative launch).  Outputs do not
// depend on the grouping: every output row is computed by the same tile code.
//
// Cross-XCD visibility: each XCD has its own L2, so producers end a tile with
// every wave's stores complete, a barrier, and one agent-scope release
// (L2 write-back) on the counter; consumers poll the counter with relaxed
// agent-scope loads and take one agent-scope acquire (L2 invalidate) when it
// reaches the target, before reading.  Every wait is bounded in
// wall-clock time: on expiry the workgroup records MOE_DEV_WAIT_TIMEOUT in the
// device status word and every workgroup leaves.
#include "common.hpp"
#include "gemm_tile.hpp"
#include "kernels.hpp"
#include "moe.h"
#include "mx_tile.hpp"

namespace moe {

namespace {

enum PhaseKind { kGateUp = 0, kCombine = 1, kDown = 2 };
constexpr int kCombTilesTok = 16;  // tokens per combine tile

// Cursor over the phases of the tile sequence, in units of minibatch groups
// (a group is `group` consecutive minibatches whose GEMM tiles run as one
// phase, so an expert's weight panels serve the row tiles of all of them).
// Step s holds gate|up(s), then down(s-1), then (with combine tiles)
// combine(s-2), each only if its group exists: gate|up(0), gate|up(1),
// down(0), gate|up(2), down(1), combine(0), down(2), combine(1), combine(2).
// Every phase depends only on phases at least one phase earlier, so a
// workgroup's wait finds the phase it needs drained by the others while it
// ran the phase in between; only the last combine follows its down phase
// closely.  With combine(s-2) before down(s-1) (comb_first), combine(j) came
// right after down(j) for the last two groups (each a wait for the slowest
// workgroup's down tiles); that order stays for the layer whose Y rows live
// in a ring of three groups, where gate|up(s) waits for combine(s-3) to free
// the slot and would otherwise come right after it.
struct PhaseCursor {
    int s = 0, slot = -1, kind = 0, j = 0;
    __device__ bool next(int ng, bool with_combine, bool comb_first) {
        for (;;) {
            if (++slot > 2) { slot = 0; ++s; }
            if (s > ng + 1) return false;
            if (slot == 0) {
                kind = kGateUp; j = s;
            } else if ((slot == 1) == comb_first) {
                if (!with_combine) continue;
                kind = kCombine; j = s - 2;
            } else {
                kind = kDown; j = s - 1;
            }
            if (j >= 0 && j < ng) return true;
        }
    }
};

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Thread 0 waits until *ctr >= target (agent-scope acquire), then the whole
// workgroup continues.  Returns false if this launch is being abandoned (this
// wait expired, or another workgroup's did: the launch's abort word, zeroed
// with the counters, is set).  An expiry is also recorded in the device status
// word (first expiry wins; it stays until moe_read_device_status reads it).
// acquire = false serves waits that only order this workgroup's later stores
// after other workgroups' completed reads (a ring slot becoming free): no data
// is read, so the L2 is left as it is.
__device__ bool wait_counter(const MegaArgs& a, int* ctr, int target, int site, int* s_flag, bool acquire) {
    if (threadIdx.x == 0) {
        int ok = 1;
        int* abort_word = a.counters + 3 * a.nmb;
        const uint64_t t0 = now_ticks();
        // Poll with relaxed loads (they read the coherent value past this XCD's
        // L2) and acquire once at the end: an acquire per poll would invalidate
        // the XCD's L2 on every iteration, under every GEMM tile running there.
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (__hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) { ok = 0; break; }
            if (now_ticks() - t0 > a.spin_ticks) {
                __hip_atomic_store(abort_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                int expected = 0;
                if (__hip_atomic_compare_exchange_strong(a.status, &expected, (int)MOE_DEV_WAIT_TIMEOUT,
                                                         __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                    __hip_atomic_store(a.status + 1, site, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (acquire) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *s_flag = ok;
    }
    __syncthreads();
    const bool ok = *s_flag != 0;
    __syncthreads();
    return ok;
}

// End of a unit of work: every wave's stores complete, then one release.
__device__ __forceinline__ void signal_counter(int* ctr) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}


__device__ __forceinline__ const int32_t* mt_of(const MegaArgs& a, int b) { return a.mt_all + (int64_t)b * a.mt_ld; }

__device__ __forceinline__ int tokens_of(const MegaArgs& a, int b) { return min(a.Mb, a.T - b * a.Mb); }

// Tile-table entry; kS: a scalar load (the bf16 kernel, whose chained tiles
// must not wait for loads in flight; in the MXFP8 kernels the extra scalar
// registers cost vector-register spills).
template <bool kS>
__device__ __forceinline__ int mt_entry(const int32_t* p) { return kS ? ld_layout(p) : *p; }

// M tiles of experts [0, e) summed over the minibatches [b0, b1)
template <bool kS>
__device__ __forceinline__ int group_mtiles_before(const MegaArgs& a, int b0, int b1, int e) {
    int n = 0;
    for (int b = b0; b < b1; ++b) n += mt_entry<kS>(mt_of(a, b) + e) - mt_entry<kS>(mt_of(a, b));
    return n;
}

// Tile lv of a GEMM phase over minibatches [b0, b1): expert-major, then N
// tile, then M tile, the M tiles of expert e running over minibatch b0's, then
// b0+1's, ...: returns the minibatch b and the tile (e, ml, ntile) in it.
template <bool kS>
__device__ __forceinline__ void group_tile(const MegaArgs& a, int b0, int b1, int NT, int lv, int& b, int& e,
                                           int& ml, int& ntile) {
    int lo = 0, hi = a.e_end - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (group_mtiles_before<kS>(a, b0, b1, mid) * NT <= lv) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int loc = lv - group_mtiles_before<kS>(a, b0, b1, e) * NT;
    const int mte = group_mtiles_before<kS>(a, b0, b1, e + 1) - group_mtiles_before<kS>(a, b0, b1, e);
    ntile = loc / mte;
    int m = loc - ntile * mte;
    for (b = b0; b < b1 - 1; ++b) {
        const int mb = mt_entry<kS>(mt_of(a, b) + e + 1) - mt_entry<kS>(mt_of(a, b) + e);
        if (m < mb) break;
        m -= mb;
    }
    ml = m;
}

}  // namespace

// Combine of tokens [c0, c1) of minibatch b (relative to the minibatch) by the
// whole workgroup of nthreads threads, two tokens at a time; LDS: the first
// 1.5 KB of smem.
__device__ void combine_range(const MegaArgs& a, int b, int c0, int c1, uint8_t* smem, int nthreads) {
    constexpr int kTok = 2;
    int (*s_row)[kMaxTopK + 1] = (int (*)[kMaxTopK + 1])smem;
    float (*s_w)[kMaxTopK] = (float (*)[kMaxTopK])(smem + 512);
    uint16_t** s_out = (uint16_t**)(smem + 1024);
    const int t0 = b * a.Mb;
    const uint8_t* lay = a.lay0 + (int64_t)b * a.lay_bytes;
    const int32_t* tok_prow = (const int32_t*)(lay + a.ly_tok_prow);
    const uint16_t* Y = a.saved_mb0 ? (const uint16_t*)(a.saved_mb0 + (int64_t)b * a.sv_mb + a.sv_y)
                                    : (const uint16_t*)(a.slot0 + (int64_t)(b % a.S) * a.slot_bytes + a.sl_y);
    for (int t = c0; t < c1; t += kTok) {
        const int ntok = min(kTok, c1 - t);
        const int tt = threadIdx.x >> 5, j = threadIdx.x & 31;
        if (tt < ntok) {
            if (j < a.k + a.with_shared) s_row[tt][j] = tok_prow[(int64_t)(t + tt) * a.ld_tok_prow + j];
            if (j < a.k) s_w[tt][j] = a.gw[(int64_t)(t0 + t + tt) * a.k + j];
            if (j == 0) s_out[tt] = a.out + (int64_t)(t0 + t + tt) * a.H;
        }
        __syncthreads();
        combine_tokens_mlp<kTok>(Y, a.H, s_row, s_w, ntok, a.k, a.with_shared, a.H, s_out, threadIdx.x,
                                 nthreads);
        __syncthreads();
    }
}


// 512 threads: the bf16 and MXFP8 tiles both run eight waves (two per SIMD).
// kMx: the routed experts run scaled-MFMA tiles; kBf16 (always with !kMx):
// bf16 tiles are compiled in, for a bf16 layer or the shared expert of an
// MXFP8 one.  Without them the MXFP8 kernel holds its state in 253 VGPRs with
// no spill, against 256 with 38 spilled (and 199 against 411 SGPRs spilled).
template <bool kMx, bool kBf16>
__global__ __attribute__((amdgpu_flat_work_group_size(kTileThreads, kTileThreads), amdgpu_waves_per_eu(2, 2)))
void mega_kernel(MegaArgs a) {
    static_assert(kMx || kBf16, "a bf16 layer runs bf16 tiles");
    // The bf16 kernel's down tiles chain: the ring plus the staging block past
    // it.  (Chained MXFP8 down tiles, with a 32-row staging block beside the
    // 132 KB ring, measured 1.7% slower in this kernel: not used.)
    constexpr int kSmem = kMx ? (kMxSmem > kTileSmem ? kMxSmem : kTileSmem) : kTileSmem + kStgBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmem];
    // wait result broadcast: the last dword, free between tiles (a phase's last
    // tile has drained its loads, and every wave passed a barrier)
    int& s_flag = *(int*)(smem + kSmem - 4);
    int* gu_done = a.counters;
    int* d_done = a.counters + a.nmb;
    int* comb_done = a.counters + 2 * a.nmb;
    const int NT1 = ceil_div(2 * a.I, BN), NT2 = ceil_div(a.H, BN);
    const bool y_in_ring = a.saved_mb0 == nullptr;
    const int G = gridDim.x - a.comm, g = blockIdx.x - a.comm;  // GEMM workgroups
    const bool comb_tiles = a.comm == 0;                      // combine as tiles of the GEMM workgroups
    const int comb_target = comb_tiles ? G : a.comm;
    const int ng = ceil_div(a.nmb, a.group), Sg = a.S / a.group;  // groups; ring slots in groups

    if ((int)blockIdx.x < a.comm) {
        // ---- combine workers: group by group, each minibatch's tokens split in
        // contiguous chunks
        for (int j = 0; j < ng; ++j) {
            if (!wait_counter(a, d_done + j, G, 2, &s_flag, true)) return;
            for (int b = j * a.group; b < min(a.nmb, (j + 1) * a.group); ++b) {
                const int Tm = tokens_of(a, b);
                const int chunk = ceil_div(Tm, a.comm);
                const int c0 = min(Tm, (int)blockIdx.x * chunk), c1 = min(Tm, c0 + chunk);
                combine_range(a, b, c0, c1, smem, kTileThreads);
            }
            signal_counter(comb_done + j);
        }
        return;
    }

    // ---- GEMM workers.  Each phase counter counts the GEMM workgroups that have
    // finished all of their tiles of that phase (each releases once per phase,
    // owning tiles in it or not), so a phase is complete at G.
    const int per = G >> 3, xcd = g & 7, local = g >> 3;
    auto phase_tiles = [&](int kind, int j) -> int {
        const int b0 = j * a.group, b1 = min(a.nmb, b0 + a.group);
        if (kind == kCombine) {
            int n = 0;
            for (int b = b0; b < b1; ++b) n += ceil_div(tokens_of(a, b), kCombTilesTok);
            return n;
        }
        return group_mtiles_before<!kMx>(a, b0, b1, a.e_end) * (kind == kGateUp ? NT1 : NT2);
    };
    auto counter_of = [&](int kind, int j) -> int* {
        return kind == kGateUp ? gu_done + j : (kind == kDown ? d_done + j : comb_done + j);
    };
    PhaseCursor cur;
    const bool comb_first = y_in_ring && Sg == 3;
    bool more = cur.next(ng, comb_tiles, comb_first);
    int64_t qstart = 0;
    int qtiles = phase_tiles(cur.kind, cur.j);
    bool ready = false;  // inputs of the current phase waited for
    TileEntry en;        // how the next chained down tile starts
    for (int it = 0;; ++it) {
        const int64_t v = (int64_t)it * G + xcd * per + local;
        while (more && v >= qstart + qtiles) {  // done with this phase: publish
            const bool dropped = a.debug_drop && g == 0 && cur.kind == kGateUp && cur.j == 0;
            if (!dropped) signal_counter(counter_of(cur.kind, cur.j));
            qstart += qtiles;
            more = cur.next(ng, comb_tiles, comb_first);
            if (more) qtiles = phase_tiles(cur.kind, cur.j);
            ready = false;
        }
        if (!more) break;
        const int kind = cur.kind, j = cur.j;
        const int b0 = j * a.group, b1 = min(a.nmb, b0 + a.group);
        if (!ready) {
            if (kind == kGateUp && j >= Sg) {  // the group's ring slots free again
                if (!wait_counter(a, d_done + (j - Sg), G, 0, &s_flag, false)) return;
                if (y_in_ring && !wait_counter(a, comb_done + (j - Sg), comb_target, 1, &s_flag, false)) return;
            }
            if (kind == kDown && !wait_counter(a, gu_done + j, G, 3, &s_flag, true)) return;
            if (kind == kCombine && !wait_counter(a, d_done + j, G, 2, &s_flag, true)) return;
            ready = true;
        }
        int lv = (int)(v - qstart);
        if (kind == kCombine) {
            int b = b0;
            for (; b < b1 - 1; ++b) {
                const int nt = ceil_div(tokens_of(a, b), kCombTilesTok);
                if (lv < nt) break;
                lv -= nt;
            }
            combine_range(a, b, lv * kCombTilesTok, min(tokens_of(a, b), (lv + 1) * kCombTilesTok), smem,
                          kTileThreads);
            continue;
        }
        int b, e, ml, ntile;
        group_tile<!kMx>(a, b0, b1, kind == kGateUp ? NT1 : NT2, lv, b, e, ml, ntile);
        const uint8_t* lay = a.lay0 + (int64_t)b * a.lay_bytes;
        const int32_t* mt = a.mt_all + (int64_t)b * a.mt_ld;
        const int32_t* prs = a.prs_all + (int64_t)b * a.mt_ld;
        const int32_t* rows = a.rows_all + (int64_t)b * a.mt_ld;
        const LayoutHeader* hdr = (const LayoutHeader*)lay;
        uint8_t* slot = a.slot0 + (int64_t)(b % a.S) * a.slot_bytes;
        uint8_t* svb = a.saved_mb0 ? a.saved_mb0 + (int64_t)b * a.sv_mb : nullptr;
        uint16_t* Y = svb ? (uint16_t*)(svb + a.sv_y) : (uint16_t*)(slot + a.sl_y);
        // MXFP8 routed experts run scaled-MFMA tiles; bf16 experts (every
        // expert of a bf16 layer, the shared expert of an MXFP8 one) bf16 tiles.
        // Under MXFP8 the saved g|u is fp32 for both.  The down tiles skip the
        // fragments that hold only padding rows of an expert's last tile
        // (kPadPerWave; layer kernel 13.0 -> 12.7 ms bf16, 8.1 -> 8.0 ms
        // MXFP8); the gate|up tiles run every fragment: the same skip there
        // measured 4% slower.
        const bool mx_tile = kMx && (!kBf16 || e < a.e_mx);
        if (kind == kGateUp) {
            if (mx_tile) {
                MxGemmArgs m = a.m1;
                m.a_row_map = (const int32_t*)(lay + a.ly_prow_token);
                m.mt_start = mt; m.prow_start = prs; m.hdr = hdr;
                m.Cq = slot + a.sl_hq; m.Cs = slot + a.sl_sh;
                m.GU = svb ? (float*)svb : nullptr;
                mx_gemm_tile<kEpiSwiGLU, kPadNone>(m, e, ml, ntile, smem);
            } else {
                GemmArgs gg = a.g1;
                gg.a_row_map = (const int32_t*)(lay + a.ly_prow_token);
                gg.mt_start = mt; gg.prow_start = prs; gg.hdr = hdr; gg.rows_e = rows;
                gg.C = (uint16_t*)(slot + a.sl_h);
                gg.GU = (!kMx && svb) ? (uint16_t*)svb : nullptr;
                gg.GUf = (kMx && svb) ? (float*)svb : nullptr;
                gemm_tile<kEpiSwiGLU, kPadNone>(gg, e, ml, ntile, smem);
            }
        } else {
            if (mx_tile) {
                MxGemmArgs m = a.m2;
                m.A = slot + a.sl_hq; m.SA = slot + a.sl_sh;
                m.mt_start = mt; m.prow_start = prs; m.hdr = hdr; m.rows_e = rows;
                m.C = Y;
                mx_gemm_tile<kEpiStore, kPadPerWave>(m, e, ml, ntile, smem);
            } else {
                GemmArgs gg = a.g2;
                gg.A = (const uint16_t*)(slot + a.sl_h);
                gg.mt_start = mt; gg.prow_start = prs; gg.hdr = hdr; gg.rows_e = rows;
                gg.C = Y;
                if constexpr (!kMx) {
                    // the workgroup's next down tile of this phase starts on
                    // stages loaded with this tile's last two
                    TileLink ln;
                    const int64_t vn = v + G;
                    if (vn < qstart + qtiles && tiles_chain(gg)) {
                        int b2, e2, ml2, nt2;
                        group_tile<true>(a, b0, b1, NT2, (int)(vn - qstart), b2, e2, ml2, nt2);
                        GemmArgs gn = a.g2;
                        gn.A = (const uint16_t*)(a.slot0 + (int64_t)(b2 % a.S) * a.slot_bytes + a.sl_h);
                        gn.prow_start = a.prs_all + (int64_t)b2 * a.mt_ld;
                        ln = tile_link(gg, e, ml, ntile, gn, e2, ml2, nt2);
                    }
                    gemm_tile<kEpiStore, kPadPerWave, true>(gg, e, ml, ntile, smem, &en, &ln);
                } else {
                    gemm_tile<kEpiStore, kPadPerWave>(gg, e, ml, ntile, smem);
                }
            }
        }
    }
}

__global__ void zero_i32_kernel(int* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

hipError_t launch_mega(const MegaArgs& a, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(ceil_div(3 * a.nmb + 1, 256)), dim3(256), 0, stream, a.counters,
                       3 * a.nmb + 1);
    MegaArgs args = a;
    void* kargs[] = {&args};
    const void* fn = !a.mx ? (const void*)mega_kernel<false, true>
                           : (a.e_mx < a.e_end ? (const void*)mega_kernel<true, true>   // with the shared expert
                                               : (const void*)mega_kernel<true, false>);
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kTileThreads), kargs, 0, stream);
}

}  // namespace moe
