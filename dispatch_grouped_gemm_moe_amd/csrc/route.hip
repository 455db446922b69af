// Router and dispatch-layout kernels (gfx950).
//
// Router: the router scores every expert for every token and picks several,
// re-deciding at each step (KuCoin flash "Cursor's MoK achieves 2.37x
// performance boost on NVIDIA GB300 NVL72", section 01).  The logits decide
// integers (the expert choice), so their fp32 rounding order is fixed: lane l
// of a wave accumulates h = l, l+64, ... with fused multiply-add, and a
// halving tree over the 64 lanes finishes the sum.  This runs on the vector
// ALUs, never on MFMA, whose internal accumulation order is not this one.
//
// Layout: count the rows of every expert, place each expert's rows next to
// each other, ascending in token, and build the padded tile map the grouped
// GEMM walks (same page, section 01: count, place, keep an expert's tokens
// adjacent; section 02: the receiving side decides the placement itself).
// The count uses integer atomics only (order-free); ranks come from wave
// ballots in token order, so the layout is deterministic.
#include "common.hpp"
#include "kernels.hpp"
#include "mxfp8.hpp"

namespace moe {

#pragma clang fp contract(off)

constexpr int kRouteWaveTokens = 2;                       // tokens per wave
constexpr int kRouteThreads = 512;                        // eight waves
constexpr int kRouteTokens = kRouteWaveTokens * kRouteThreads / kWave;  // per workgroup
constexpr int kRouteEC = 32;                              // experts per accumulation pass
constexpr int kRouteWRow = kRouteEC + 4;                  // padded LDS row (conflict-free 128-bit reads)

// Lane l holds p[l]; returns in lane 0 the fixed halving tree
// p[l] = p[l] + p[l+s] for s = 32, 16, 8, 4, 2, 1.  At each step only lanes
// l < s must be right, and each of them receives p[l+s]: lanes 16 and 32 apart
// through ds_bpermute, the rest through DPP row shifts / quad permutes.
__device__ __forceinline__ float lane_tree64(float v) {
    v = v + __shfl_xor(v, 32, kWave);
    v = v + __shfl_xor(v, 16, kWave);
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x108, 0xF, 0xF, false));  // row_shl:8
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x104, 0xF, 0xF, false));  // row_shl:4
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    v = v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    return v;
}

// A wave scores 2 tokens against up to 32 experts per pass: lane l runs the
// partial sums p[l] of all 64 (token, expert) pairs over h = l, l+64, ...
// The router weight rows of each 64-wide h chunk (32 experts) are staged once
// per workgroup in LDS, double-buffered, and read by its 8 waves (16 tokens),
// so a Wr element is fetched once per 16 tokens instead of once per 2.  Two
// tokens per wave keep the kernel at 128 VGPRs, two workgroups per CU; four
// tokens need 190 VGPRs, one workgroup per CU (0.24 against 0.35 ms at 16384
// tokens, H 7168, 32 experts), and at one token the LDS reads of the staged
// weights cost as much as the FMAs they feed.
template <bool kVec4>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ bias,
    int T, int H, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_out, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
    __shared__ float s_logit[kRouteTokens][kMaxExperts];
    __shared__ __attribute__((aligned(16))) float s_w[2][kWave][kRouteWRow];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kRouteTokens;
    const int nt = min(kRouteTokens, T - t0);
    const int tw0 = t0 + wave * kRouteWaveTokens;  // this wave's first token
    const int ntw = max(0, min(kRouteWaveTokens, T - tw0));
    const int nchunk = H / kWave;
    // staging: thread tid moves 4 consecutive experts of one h row of a chunk
    const int sr = tid >> 3, sq = (tid & 7) * 4;

    for (int e0 = 0; e0 < E; e0 += kRouteEC) {
        // the router weight of chunk c: this thread's 4 experts of one h row
        auto load_w = [&](int c) {
            const int h = c * kWave + sr;
            const float* wrow = Wr + (size_t)h * E + e0 + sq;
            floatx4 w4;
            if (kVec4) {
                w4 = (e0 + sq < E) ? *(const floatx4*)wrow : floatx4{0, 0, 0, 0};
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) w4[q] = (e0 + sq + q < E) ? wrow[q] : 0.0f;
            }
            return w4;
        };
        float acc[kRouteWaveTokens][kRouteEC];
#pragma unroll
        for (int tt = 0; tt < kRouteWaveTokens; ++tt)
#pragma unroll
            for (int ee = 0; ee < kRouteEC; ++ee) acc[tt][ee] = 0.0f;
        // this lane's token values of chunk c (one h per lane), loaded a chunk ahead
        auto load_x = [&](int c, uint16_t (&xr)[kRouteWaveTokens]) {
#pragma unroll
            for (int tt = 0; tt < kRouteWaveTokens; ++tt)
                xr[tt] = (tt < ntw) ? x[(size_t)(tw0 + tt) * H + c * kWave + lane] : (uint16_t)0;
        };
        uint16_t xnext[kRouteWaveTokens];
        __syncthreads();  // previous pass done with s_w
        *(floatx4*)&s_w[0][sr][sq] = load_w(0);
        // chunk c + 1's weights are loaded during chunk c - 1 and written to
        // LDS after chunk c's barrier, so no chunk waits on a global load
        floatx4 wnext = nchunk > 1 ? load_w(1) : floatx4{0, 0, 0, 0};
        load_x(0, xnext);
        for (int c = 0; c < nchunk; ++c) {
            __syncthreads();  // chunk c staged; chunk c-1's buffer free
            if (c + 1 < nchunk) *(floatx4*)&s_w[(c + 1) & 1][sr][sq] = wnext;
            if (c + 2 < nchunk) wnext = load_w(c + 2);
            float xv[kRouteWaveTokens];
#pragma unroll
            for (int tt = 0; tt < kRouteWaveTokens; ++tt) xv[tt] = bf16_to_f32(xnext[tt]);
            if (c + 1 < nchunk) load_x(c + 1, xnext);
            float wv[kRouteEC];
#pragma unroll
            for (int q = 0; q < kRouteEC / 4; ++q) {
                const floatx4 w4 = *(const floatx4*)&s_w[c & 1][lane][4 * q];
                wv[4 * q] = w4[0]; wv[4 * q + 1] = w4[1]; wv[4 * q + 2] = w4[2]; wv[4 * q + 3] = w4[3];
            }
#pragma unroll
            for (int tt = 0; tt < kRouteWaveTokens; ++tt)
#pragma unroll
                for (int ee = 0; ee < kRouteEC; ++ee) acc[tt][ee] = __builtin_fmaf(xv[tt], wv[ee], acc[tt][ee]);
        }
#pragma unroll
        for (int tt = 0; tt < kRouteWaveTokens; ++tt)
#pragma unroll
            for (int ee = 0; ee < kRouteEC; ++ee) {
                float v = lane_tree64(acc[tt][ee]);
                if (lane == 0 && e0 + ee < E && tt < ntw) {
                    if (bias) v = v + bias[e0 + ee];
                    s_logit[wave * kRouteWaveTokens + tt][e0 + ee] = v;
                }
            }
    }
    __syncthreads();

    // MXFP8 dispatch-side quantisation of this workgroup's token rows (the
    // rows the router has just read, so mostly cache hits): one thread per
    // 32-element block, codes along H and the operand-layout scales.
    if (xq) {
        const int nb = H / 32;
        for (int i = tid; i < nt * nb; i += kRouteThreads) {
            const int tt = i / nb, b = i - tt * nb;
            const int64_t t = t0 + tt;
            const uint8_t sc = mx_quant_block32(x + t * H + b * 32, xq + t * H + b * 32);
            mx_store_scale_byte(xs, T, t, b, nb, sc);
        }
    }

    // Top-k per token: one wave per token; lane l holds experts l, l+64, ...
    for (int tt = wave; tt < nt; tt += kRouteThreads / kWave) {
        const int t = t0 + tt;
        float v[kMaxExperts / kWave];
#pragma unroll
        for (int q = 0; q < kMaxExperts / kWave; ++q) {
            const int e = lane + q * kWave;
            v[q] = e < E ? s_logit[tt][e] : 0.0f;
            if (logits_out && e < E) logits_out[(size_t)t * E + e] = v[q];
        }
        unsigned taken = 0;  // bit q: expert lane + 64q already selected (or absent)
#pragma unroll
        for (int q = 0; q < kMaxExperts / kWave; ++q)
            if (lane + q * kWave >= E) taken |= 1u << q;
        float sel_v[kMaxTopK];
        int sel_i[kMaxTopK];
        for (int j = 0; j < k; ++j) {
            float bv = 0.0f;
            int bi = 0x7fffffff;
#pragma unroll
            for (int q = 0; q < kMaxExperts / kWave; ++q) {
                const int e = lane + q * kWave;
                if (!(taken & (1u << q)) && (bi == 0x7fffffff || v[q] > bv)) { bv = v[q]; bi = e; }
            }
            // wave arg-max: larger value wins, equal values go to the lower index
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1) {
                const float ov = __shfl_xor(bv, s, kWave);
                const int oi = __shfl_xor(bi, s, kWave);
                const bool better = (oi != 0x7fffffff) &&
                                    (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi));
                if (better) { bv = ov; bi = oi; }
            }
            sel_v[j] = bv;
            sel_i[j] = bi;
            if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
        }
        if (lane == 0) {
            // softmax over the selected logits, summed in slot order
            float ez[kMaxTopK];
            float den = 0.0f;
            for (int j = 0; j < k; ++j) {
                ez[j] = expf(sel_v[j] - sel_v[0]);
                den = den + ez[j];
            }
            for (int j = 0; j < k; ++j) {
                topk_idx[(size_t)t * k + j] = sel_i[j];
                topk_w[(size_t)t * k + j] = ez[j] / den;
            }
        }
    }
}

void launch_route(const uint16_t* x, const float* Wr, const float* bias, int T, int H, int E, int k,
                  int32_t* topk_idx, float* topk_w, float* logits, hipStream_t stream, uint8_t* xq, uint8_t* xs) {
    const int blocks = ceil_div(T, kRouteTokens);
    const bool vec4 = (E % 4 == 0) && (((uintptr_t)Wr & 15) == 0);
    if (vec4)
        hipLaunchKernelGGL(route_kernel<true>, dim3(blocks), dim3(kRouteThreads), 0, stream, x, Wr, bias, T,
                           H, E, k, topk_idx, topk_w, logits, xq, xs);
    else
        hipLaunchKernelGGL(route_kernel<false>, dim3(blocks), dim3(kRouteThreads), 0, stream, x, Wr, bias, T,
                           H, E, k, topk_idx, topk_w, logits, xq, xs);
}

// ---------------------------------------------------------------------------
// layout
// ---------------------------------------------------------------------------

constexpr int kLayoutThreads = 1024;
constexpr int kLayoutWaves = kLayoutThreads / kWave;

__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(const int32_t* __restrict__ idx, int T, int Mb,
                                                                 int E, int k, int with_shared,
                                                                 LayoutOut o, LayoutStrides st) {
    // workgroup b lays out minibatch b: tokens [b*Mb, min(T, (b+1)*Mb))
    {
        const int b = blockIdx.x;
        const int t0 = b * Mb;
        if (o.counts) o.counts += b * st.counts;
        if (o.offsets) o.offsets += b * st.offsets;
        if (o.row_token) o.row_token += b * st.row_token;
        if (o.tok_row) o.tok_row += b * st.tok_row;
        if (o.hdr) o.hdr += b * st.hdr;
        if (o.mt_start) o.mt_start += b * st.mt_start;
        if (o.prow_token) o.prow_token += b * st.prow_token;
        if (o.tok_prow) o.tok_prow += b * st.tok_prow;
        if (o.prow_slot) o.prow_slot += b * st.prow_slot;
        if (o.rows_e) o.rows_e += b * st.rows_e;
        if (o.prow_start) o.prow_start += b * st.prow_start;
        o.token_base += t0;
        idx += (int64_t)t0 * k;
    }
    const int Tm = min(Mb, T - (int)blockIdx.x * Mb);
    __shared__ int s_cnt[kLayoutWaves][kMaxExperts + 1];  // per-wave counts, then running bases
    __shared__ int s_off[kMaxExperts + 2];                 // unpadded row offsets
    __shared__ int s_poff[kMaxExperts + 2];                // padded (kSegRows-aligned) row offsets
    __shared__ int s_tot[kMaxExperts + 1];                 // rows per expert
    __shared__ int s_err;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Et = E + (with_shared ? 1 : 0);
    for (int i = tid; i < kLayoutWaves * (kMaxExperts + 1); i += kLayoutThreads) (&s_cnt[0][0])[i] = 0;
    if (tid == 0) s_err = 0;
    __syncthreads();

    // Wave w owns the contiguous token chunk [c0, c1); chunks ascend with w.
    const int chunk = ceil_div(Tm, kLayoutWaves);
    const int c0 = min(Tm, wave * chunk), c1 = min(Tm, c0 + chunk);

    // 1. count (integer atomics: the totals do not depend on their order)
    for (int t = c0 + lane; t < c1; t += kWave) {
        int ids[kMaxTopK];
        bool bad = false;
        for (int j = 0; j < k; ++j) {
            ids[j] = idx[(size_t)t * k + j];
            bad |= (unsigned)ids[j] >= (unsigned)E;
            for (int q = 0; q < j; ++q) bad |= ids[q] == ids[j];
        }
        if (bad) {
            s_err = 1;
            continue;
        }
        for (int j = 0; j < k; ++j) atomicAdd(&s_cnt[wave][ids[j]], 1);
    }
    __syncthreads();
    if (s_err) {  // report, and leave an empty tile map so no GEMM tile runs
        if (tid == 0) {
            if (o.offsets) o.offsets[E] = -1;
            if (o.hdr) { o.hdr->m_tiles = 0; o.hdr->rows = 0; o.hdr->error = 1; o.hdr->prows = 0; }
        }
        for (int e = tid; e <= Et; e += kLayoutThreads) {
            if (o.mt_start) o.mt_start[e] = 0;
            if (o.prow_start) o.prow_start[e] = 0;
            if (o.rows_e && e < Et) o.rows_e[e] = 0;
        }
        return;
    }

    // 2a. per expert: exclusive prefix over waves (each wave's first rank) and total
    for (int e = tid; e < E; e += kLayoutThreads) {
        int run = 0;
        for (int w = 0; w < kLayoutWaves; ++w) {
            const int c = s_cnt[w][e];
            s_cnt[w][e] = run;
            run += c;
        }
        s_tot[e] = run;
    }
    if (tid == 0 && with_shared) s_tot[E] = Tm;  // the shared expert takes every token
    __syncthreads();
    // 2b. offsets and tile map (one thread: at most 257 experts).  Expert e's
    // padded rows start at s_poff[e], a multiple of kSegRows; its ceil(tot/BM)
    // M tiles are BM rows, the last a half tile when it holds at most kSegRows.
    if (tid == 0) {
        int off = 0, mt = 0, poff = 0;
        for (int e = 0; e < Et; ++e) {
            const int tot = s_tot[e];
            s_off[e] = off;
            s_poff[e] = poff;
            if (o.mt_start) o.mt_start[e] = mt;
            if (o.prow_start) o.prow_start[e] = poff;
            if (o.rows_e) o.rows_e[e] = tot;
            if (e < E) {
                if (o.counts) o.counts[e] = tot;
                if (o.offsets) o.offsets[e] = off;
                off += tot;
            }
            mt += ceil_div(tot, BM);
            poff += ceil_div(tot, kSegRows) * kSegRows;
        }
        s_off[Et] = off;
        s_poff[Et] = poff;
        if (o.offsets) o.offsets[E] = off;
        if (o.mt_start) o.mt_start[Et] = mt;
        if (o.prow_start) o.prow_start[Et] = poff;
        if (o.hdr) { o.hdr->m_tiles = mt; o.hdr->rows = off; o.hdr->error = 0; o.hdr->prows = poff; }
    }
    __syncthreads();

    // 3. rank: 64 tokens at a time in lane order, experts in index order
    for (int g0 = c0; g0 < c1; g0 += kWave) {
        const int t = g0 + lane;
        const bool valid = t < c1;
        int ids[kMaxTopK];
        for (int j = 0; j < k; ++j) ids[j] = valid ? idx[(size_t)t * k + j] : -1;
        for (int e = 0; e < E; ++e) {
            int js = -1;
            for (int j = 0; j < k; ++j) js = (ids[j] == e) ? j : js;
            const uint64_t mask = __ballot(js >= 0);
            if (mask == 0) continue;
            const int base = s_cnt[wave][e];
            if (js >= 0) {
                const int rank = base + __popcll(mask & ((1ull << lane) - 1ull));
                const int row = s_off[e] + rank;
                const int prow = s_poff[e] + rank;
                if (o.row_token) o.row_token[row] = t;
                if (o.tok_row) o.tok_row[(size_t)t * k + js] = row;
                if (o.prow_token) o.prow_token[prow] = o.token_base + t;
                if (o.tok_prow) o.tok_prow[(size_t)t * o.tok_prow_ld + js] = prow;
                if (o.prow_slot) o.prow_slot[prow] = js;
            }
            if (lane == 0) s_cnt[wave][e] = base + __popcll(mask);
        }
        if (with_shared && valid) {
            const int prow = s_poff[E] + t;
            if (o.prow_token) o.prow_token[prow] = o.token_base + t;
            if (o.tok_prow) o.tok_prow[(size_t)t * o.tok_prow_ld + k] = prow;
            if (o.prow_slot) o.prow_slot[prow] = k;
        }
    }
    __syncthreads();

    // 4. padding rows of each expert's last tile repeat the expert's first token,
    //    so every GEMM input row is a real, finite row (their outputs are unused).
    if (o.prow_token) {
        for (int e = wave; e < Et; e += kLayoutWaves) {
            const int tot = (e < E) ? s_off[e + 1] - s_off[e] : Tm;
            if (tot == 0) continue;
            const int first = o.prow_token[s_poff[e]];
            for (int r = s_poff[e] + tot + lane; r < s_poff[e + 1]; r += kWave) {
                o.prow_token[r] = first;
                if (o.prow_slot) o.prow_slot[r] = -1;
            }
        }
    }
}

void launch_layout(const int32_t* idx, int Tm, int E, int k, int with_shared, const LayoutOut& o,
                   hipStream_t stream) {
    hipLaunchKernelGGL(layout_kernel, dim3(1), dim3(kLayoutThreads), 0, stream, idx, Tm, Tm, E, k,
                       with_shared, o, LayoutStrides{});
}

void launch_layout_batched(const int32_t* idx, int T, int Mb, int E, int k, int with_shared, const LayoutOut& o,
                           const LayoutStrides& st, hipStream_t stream) {
    hipLaunchKernelGGL(layout_kernel, dim3(ceil_div(T, Mb)), dim3(kLayoutThreads), 0, stream, idx, T, Mb, E, k,
                       with_shared, o, st);
}

}  // namespace moe
