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
    // plain-store tiles chain (the ring plus the staging block past it)
    constexpr bool kChain = EPI == kEpiStore;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kChain ? kTileSmem + kStgBytes : kTileSmem];
    const int NT = ceil_div(p.N, BN);
    const int total = launch_tiles(p);
    const int G = gridDim.x, per = G >> 3;
    // Workgroups are dealt to the 8 XCDs round-robin; the 'per' workgroups of
    // one XCD take consecutive tiles so that they share weight and row tiles
    // in that XCD's L2.
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    // tile v: its minibatch's arguments and its coordinates
    auto tile_of = [&](int v, GemmArgs& q, int& e, int& ml, int& ntile) {
        q = p;
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
            if (q.GU) q.GU += b * p.gu_mb;
            if (q.GUf) q.GUf += b * p.gu_mb;
        }
        tile_coords(q.mt_start, q.e_begin, q.e_end, NT, v, e, ml, ntile);
    };
    const bool chain = kChain && tiles_chain(p);
    TileEntry en;
    for (int it = 0;; ++it) {
        const int v = it * G + xcd * per + local;
        if (v >= total) break;
        GemmArgs q;
        int e, ml, ntile;
        tile_of(v, q, e, ml, ntile);
        if constexpr (kChain) {
            TileLink ln;
            if (chain && v + G < total) {
                GemmArgs qn;
                int e2, ml2, nt2;
                tile_of(v + G, qn, e2, ml2, nt2);
                ln = tile_link(q, e, ml, ntile, qn, e2, ml2, nt2);
            }
            gemm_tile<EPI, kPadPerWave, true>(q, e, ml, ntile, smem, &en, &ln);
        } else {
            gemm_tile<EPI>(q, e, ml, ntile, smem);
        }
    }
}

// ---------------------------------------------------------------------------
// weight gradients: C[e] = A_e^T B_e over every routed row of expert e,
// minibatch by minibatch in order (a fixed summation order), from token-major
// operands: one read directly from its row-major buffer, the other (x or
// dout) gathered from the token matrix by the layout's row -> token map.
// ---------------------------------------------------------------------------

// K sequence of expert e's rows: for each minibatch b its padded rows from
// prs_b[e] on, in 64-row stages up to the last one holding a routed row (the
// padding rows a stage takes in add nothing: the directly read operand is
// zero on them, and the gathered one holds a real token's finite row).
// Operand X of A, B is read directly (row prow of minibatch b at X + b * x_mb
// + prow * ldx bytes) or, for X = kGather, gathered (row prow of minibatch b
// is token map[b * map_mb + prow] of a [T][ldx-byte] matrix).  Wave w loads K
// rows 8w .. 8w + 7 of a stage; their tokens come with one scalar load issued
// a stage before they are used.
template <int kGather>
struct TokenK {
    const int32_t* prs;
    const int32_t* rows;
    int mt_ld, e, nmb;
    const char* A;
    const char* B;
    const int32_t* map;
    int64_t a_mb, b_mb, map_mb;  // bytes, bytes, elements
    uint32_t lda, ldb;           // bytes
    uint32_t acol[2], bcol[2];   // this lane's column bytes (load q takes [q % 2])
    int wave, hi;                // hi = lane / 32: the lane's K row of a load pair
    int b = -1, step = 0, nsteps = 0, row0 = 0;
    const char* da;              // minibatch b's copy of a directly read operand
    const char* db;
    const int32_t* mapb;         // minibatch b's row -> token map
    intx8 tok;                   // tokens of rows 8 wave .. +7 of the stage next() returns
    __device__ __forceinline__ void seek() {
        // the tile map and row map are read-only here: read them through the
        // constant address space (scalar loads, counted by lgkmcnt) so that
        // the ring's vmcnt accounting sees only the ring's own loads
        typedef const __attribute__((address_space(4))) int32_t cint;
        while (step >= nsteps && b + 1 < nmb) {
            ++b;
            row0 = ((cint*)prs)[(int64_t)b * mt_ld + e];
            nsteps = ceil_div(((cint*)rows)[(int64_t)b * mt_ld + e], kBK8);
            step = 0;
            da = A + b * a_mb;
            db = B + b * b_mb;
            mapb = map + b * map_mb;
        }
        if (kGather && step < nsteps)
            tok = *(const __attribute__((address_space(4))) intx8*)(mapb + row0 + step * kBK8 + 8 * wave);
    }
    // offsets stay below 4 GiB: a token matrix and one minibatch's copy of an
    // operand are checked to on the host
    __device__ __forceinline__ void next(const char* (&pa)[4], const char* (&pb)[4]) {
        const uint32_t r = (uint32_t)(row0 + step * kBK8 + 8 * wave + hi);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // the pair's two tokens as scalars, then one select per lane
            const int t0 = __builtin_amdgcn_readfirstlane(tok[2 * q]);
            const int t1 = __builtin_amdgcn_readfirstlane(tok[2 * q + 1]);
            const uint32_t t = (uint32_t)(hi ? t1 : t0);
            pa[q] = kGather == 1 ? A + (t * lda + acol[q & 1]) : da + ((r + 2 * q) * lda + acol[q & 1]);
            pb[q] = kGather == 2 ? B + (t * ldb + bcol[q & 1]) : db + ((r + 2 * q) * ldb + bcol[q & 1]);
        }
        ++step;
        seek();
    }
};

template <int kGather>
__global__ __attribute__((amdgpu_flat_work_group_size(kTileThreads, kTileThreads), amdgpu_waves_per_eu(2, 2)))
void wgrad_kernel(WgradArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kTileSmem];
    const int lane = threadIdx.x & 63;
    const WgradTiles tiles(p.M, p.N, p.mq, p.nq);
    int e, m0, n0;
    for (int it = 0; tiles.get(it, p.Et - p.e_begin, e, m0, n0); ++it) {
        e += p.e_begin;
        int KT = 0;
        for (int b = 0; b < p.nmb; ++b) KT += ceil_div(p.rows[(int64_t)b * p.mt_ld + e], kBK8);
        TokenK<kGather> kit;
        kit.prs = p.prs; kit.rows = p.rows; kit.mt_ld = p.mt_ld; kit.e = e; kit.nmb = p.nmb;
        kit.A = (const char*)p.A; kit.B = (const char*)p.B;
        kit.lda = (uint32_t)p.lda * 2; kit.ldb = (uint32_t)p.ldb * 2; kit.a_mb = p.a_mb * 2; kit.b_mb = p.b_mb * 2;
        kit.map = p.map; kit.map_mb = p.map_mb;
        kit.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        kit.hi = lane >> 5;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // M and N are multiples of 64: columns past them (a last tile's)
            // read the matrix's last columns again and are not stored
            const int c = kmajor_chunk(lane, h);
            kit.acol[h] = (uint32_t)min(m0 + 8 * c, p.M - 8) * 2;
            kit.bcol[h] = (uint32_t)min(n0 + 8 * c, p.N - 8) * 2;
        }
        kit.seek();
        floatx16 acc[2][4];
        tile_mainloop8t(acc, smem, KT, kit);
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
    if (a.gather == 1)
        hipLaunchKernelGGL(wgrad_kernel<1>, dim3(grid), dim3(kTileThreads), 0, stream, w);
    else if (a.gather == 2)
        hipLaunchKernelGGL(wgrad_kernel<2>, dim3(grid), dim3(kTileThreads), 0, stream, w);
    else
        hipLaunchKernelGGL(wgrad_kernel<0>, dim3(grid), dim3(kTileThreads), 0, stream, w);
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
