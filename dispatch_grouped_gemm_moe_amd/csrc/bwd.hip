// Backward-pass data movement and reductions of the MoE layer (gfx950).
//
// Training runs the two exchanges of the layer in reverse (KuCoin flash
// "Cursor's MoK achieves 2.37x performance boost on NVIDIA GB300 NVL72",
// section 01; section 02 names them reverse-combine and reverse-dispatch).
// On one GPU they become:
//   reverse-combine: every expert row r = (token t, slot j) receives
//     dY_r = w[t,j] * dout[t], and d out / d w[t,j] = <dout[t], Y_r>;
//   reverse-dispatch: dx[t] = sum_j dX_r(t,j) (+ the shared expert's rows)
//     plus the router term sum_j dsel[t,j] * Wr[:, idx[t,j]], where
//     dsel = w * (dgate - <w, dgate>) is the softmax backward.
// Every floating-point sum has a fixed order (no atomics), so results are
// bitwise reproducible.
#include "common.hpp"
#include "kernels.hpp"
#include "mxfp8.hpp"

namespace moe {

constexpr int kTile = 64;

__device__ __forceinline__ void unpack16_bf16(const intx4* src, float* f) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const intx4 a = src[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[8 * q + 2 * e] = __builtin_bit_cast(float, (uint32_t)a[e] << 16);
            f[8 * q + 2 * e + 1] = __builtin_bit_cast(float, (uint32_t)a[e] & 0xffff0000u);
        }
    }
}

__device__ __forceinline__ void pack16_bf16(const uint16_t* v, intx4* dst) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        intx4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (int)((uint32_t)v[8 * q + 2 * e] | ((uint32_t)v[8 * q + 2 * e + 1] << 16));
        dst[q] = o;
    }
}

// One workgroup per 64 padded rows x 64 hidden columns of a minibatch.
//   row_w[prow]   = w (0 on padding rows), if row_w is set
//   dYq, sdY      = MXFP8 codes and scales of w * dout[t] (rows before padded
//                   row *dyq_row_end), if dYq is set
//   dgp[prow][hb] = sum over the block's 64 columns of dout[t][h] * Y[prow][h]
//                   (routed rows; in column order, then a fixed pair tree)
//   dsel[prow]    = 0 (filled for routed rows by the reverse-dispatch)
// MXW (MXFP8 weight gradients): a block of rows before *dyq_row_end also
// writes dY (from its fp32 values) and x (zero on padding rows), quantised
// along the padded rows, through LDS transposes.  The block of 64 rows lies
// inside one expert segment (segments start at multiples of 128 rows), so the
// choice is uniform over the workgroup.  bf16 weight gradients need neither
// copy: they read dout and x rows through the row map.
template <bool MXW>
__global__ __launch_bounds__(256) void rcomb_gather_kernel(RcombArgs p) {
    __shared__ float sY[MXW ? kTile : 1][kTile + 1];
    __shared__ uint16_t sX[MXW ? kTile : 1][kTile + 2];
    const int prow0 = blockIdx.x * kTile, h0 = blockIdx.y * kTile;
    if (prow0 >= p.hdr->prows) return;
    const int tid = threadIdx.x;
    const int r = tid >> 2, c0 = (tid & 3) * 16;
    const int prow = prow0 + r;
    const int slot = p.prow_slot[prow];
    const int t = p.prow_token[prow];
    const float w = slot < 0 ? 0.0f : (slot < p.k ? p.topk_w[(int64_t)t * p.k + slot] : 1.0f);
    float d[16];
    {
        const intx4* src = (const intx4*)(p.dout + (int64_t)t * p.H + h0 + c0);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const intx4 a = src[q];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                d[8 * q + 2 * e] = __builtin_bit_cast(float, (uint32_t)a[e] << 16);
                d[8 * q + 2 * e + 1] = __builtin_bit_cast(float, (uint32_t)a[e] & 0xffff0000u);
            }
        }
    }
    // reverse-combine partial dot product <dout[t], Y[prow]> over this block's columns
    float part = 0.0f;
    if (slot >= 0 && slot < p.k) {
        const intx4* ys = (const intx4*)(p.Y + (int64_t)prow * p.H + h0 + c0);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const intx4 yv = ys[q];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                part = __builtin_fmaf(d[8 * q + 2 * e], __builtin_bit_cast(float, (uint32_t)yv[e] << 16), part);
                part = __builtin_fmaf(d[8 * q + 2 * e + 1], __builtin_bit_cast(float, (uint32_t)yv[e] & 0xffff0000u), part);
            }
        }
    }
    part = part + __shfl_xor(part, 1, kWave);
    part = part + __shfl_xor(part, 2, kWave);
    if ((tid & 3) == 0) {
        if (slot >= 0 && slot < p.k) p.dgp[(int64_t)prow * p.nhb + blockIdx.y] = part;
        if (blockIdx.y == 0) {
            p.dsel[prow] = 0.0f;
            if (p.row_w) p.row_w[prow] = w;
        }
    }
    float dyf[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) dyf[c] = w * d[c];
    // MXFP8 operand of the down input-gradient GEMM, from the fp32 values
    if (p.dYq && prow < *p.dyq_row_end)
        mx_quant_row64(dyf, tid & 3, p.dYq + (int64_t)prow * p.H + h0, p.sdY, p.ldt, prow, h0 / 64, p.H / 64);
    if constexpr (MXW) {
        if (prow0 >= *p.dyq_row_end) return;
        float xv[16];
        unpack16_bf16((const intx4*)(p.x + (int64_t)t * p.H + h0 + c0), xv);
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            sY[c0 + c][r] = dyf[c];
            sX[c0 + c][r] = slot < 0 ? (uint16_t)0 : f32_to_bf16_rne(xv[c]);
        }
        __syncthreads();
        // transposed tiles: thread -> column h0 + tid/4, rows prow0 + 16*(tid%4) .. +16;
        // four consecutive lanes hold the column's 64 rows: two 32-row blocks
        const int hc = tid >> 2, r0 = (tid & 3) * 16;
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = sY[hc][r0 + q];
        mx_quant_row64(v, tid & 3, p.dYTq + (int64_t)(h0 + hc) * p.ldt + prow0, p.sdYT, p.H, h0 + hc,
                       prow0 / 64, (int)(p.ldt / 64));
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = __builtin_bit_cast(float, (uint32_t)sX[hc][r0 + q] << 16);
        mx_quant_row64(v, tid & 3, p.xgTq + (int64_t)(h0 + hc) * p.ldt + prow0, p.sxgT, p.H, h0 + hc,
                       prow0 / 64, (int)(p.ldt / 64));
    }
}

void launch_rcomb_gather(const RcombArgs& a, int rpad, hipStream_t stream) {
    if (a.xgTq)
        hipLaunchKernelGGL(rcomb_gather_kernel<true>, dim3(rpad / kTile, a.H / kTile), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(rcomb_gather_kernel<false>, dim3(rpad / kTile, a.H / kTile), dim3(256), 0, stream, a);
}

// SwiGLU backward, one workgroup per 64 padded rows x 64 intermediate columns.
// For the rows from *dgu_row0 on (the experts whose weight gradient, and so
// input gradient, takes bf16 operands) it writes row-major dG | dU, operand of
// the gate|up input-gradient GEMM and of the gate|up weight gradient, and
// w * h (zero on padding rows), the down weight gradient's row operand; the
// MXFP8 input gradient's rows take the quantised dG | dU.  MXW (MXFP8 weight
// gradients): a block of rows before *dgu_row0 also writes dG | dU and h as
// E4M3 codes quantised along the padded rows from their fp32 values (h zero
// on padding rows), through LDS transposes; the block lies inside one expert
// segment.
template <bool MXW>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(SwigluBwdArgs p) {
    __shared__ float sG[MXW ? kTile : 1][kTile + 1];
    __shared__ float sU[MXW ? kTile : 1][kTile + 1];
    __shared__ float sH[MXW ? kTile : 1][kTile + 1];
    const int prow0 = blockIdx.x * kTile, i0 = blockIdx.y * kTile;
    if (prow0 >= p.hdr->prows) return;
    const int tid = threadIdx.x;
    const int r = tid >> 2, c0 = (tid & 3) * 16;
    const int64_t prow = prow0 + r;
    const int I = p.I;
    float dh[16], g[16], u[16];
    if (p.dHf) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const floatx4 a = *(const floatx4*)(p.dHf + prow * I + i0 + c0 + 4 * q);
            const floatx4 b = *(const floatx4*)(p.GUf + prow * 2 * I + i0 + c0 + 4 * q);
            const floatx4 c = *(const floatx4*)(p.GUf + prow * 2 * I + I + i0 + c0 + 4 * q);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dh[4 * q + e] = a[e];
                g[4 * q + e] = b[e];
                u[4 * q + e] = c[e];
            }
        }
    } else {
        unpack16_bf16((const intx4*)(p.dH + prow * I + i0 + c0), dh);
        unpack16_bf16((const intx4*)(p.GU + prow * 2 * I + i0 + c0), g);
        unpack16_bf16((const intx4*)(p.GU + prow * 2 * I + I + i0 + c0), u);
    }
    float dgf[16], duf[16], hf[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const float sg = 1.0f / (1.0f + __expf(-g[c]));
        const float silu = g[c] * sg;
        dgf[c] = dh[c] * u[c] * (sg * (1.0f + g[c] * (1.0f - sg)));
        duf[c] = dh[c] * silu;
        hf[c] = silu * u[c];
    }
    if (prow >= (int64_t)*p.dgu_row0) {
        const float w = p.row_w[prow];
        uint16_t v[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) v[c] = f32_to_bf16_rne(dgf[c]);
        pack16_bf16(v, (intx4*)(p.dGU + prow * 2 * I + i0 + c0));
#pragma unroll
        for (int c = 0; c < 16; ++c) v[c] = f32_to_bf16_rne(duf[c]);
        pack16_bf16(v, (intx4*)(p.dGU + prow * 2 * I + I + i0 + c0));
#pragma unroll
        for (int c = 0; c < 16; ++c) v[c] = w == 0.0f ? (uint16_t)0 : f32_to_bf16_rne(w * hf[c]);
        pack16_bf16(v, (intx4*)(p.HW + prow * I + i0 + c0));
    }
    if (p.dGUq) {  // MXFP8 operand of the gate|up input-gradient GEMM, from the fp32 values
        mx_quant_row64(dgf, tid & 3, p.dGUq + prow * 2 * I + i0, p.sdGU, p.ldt, prow, i0 / 64, 2 * I / 64);
        mx_quant_row64(duf, tid & 3, p.dGUq + prow * 2 * I + I + i0, p.sdGU, p.ldt, prow, (I + i0) / 64, 2 * I / 64);
    }
    if constexpr (MXW) {
        if (prow0 >= *p.dgu_row0) return;
        // h of a padding row is zero, so it cannot raise its block's scale
        const bool pad = p.prow_slot[prow] < 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            sG[c0 + c][r] = dgf[c];
            sU[c0 + c][r] = duf[c];
            sH[c0 + c][r] = pad ? 0.0f : hf[c];
        }
        __syncthreads();
        // four consecutive lanes hold a column's 64 rows: two 32-row blocks
        const int ic = tid >> 2, r0 = (tid & 3) * 16;
        const int j = prow0 / 64, nj = (int)(p.ldt / 64);
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = sG[ic][r0 + q];
        mx_quant_row64(v, tid & 3, p.dGUTq + (int64_t)(i0 + ic) * p.ldt + prow0, p.sdGUT, 2 * I, i0 + ic, j, nj);
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = sU[ic][r0 + q];
        mx_quant_row64(v, tid & 3, p.dGUTq + (int64_t)(I + i0 + ic) * p.ldt + prow0, p.sdGUT, 2 * I, I + i0 + ic,
                       j, nj);
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = sH[ic][r0 + q];
        mx_quant_row64(v, tid & 3, p.HTq + (int64_t)(i0 + ic) * p.ldt + prow0, p.sHT, I, i0 + ic, j, nj);
    }
}

void launch_swiglu_bwd(const SwigluBwdArgs& a, int rpad, hipStream_t stream) {
    if (a.HTq)
        hipLaunchKernelGGL(swiglu_bwd_kernel<true>, dim3(rpad / kTile, a.I / kTile), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(swiglu_bwd_kernel<false>, dim3(rpad / kTile, a.I / kTile), dim3(256), 0, stream, a);
}

// One workgroup per token of a minibatch: gate gradients, softmax backward and
//   dx[t] = sum_j dX[prow_j] (+ dX[shared row]) + sum_j dsel_j * WrT[idx_j]
constexpr int kRdThreads = 128;
constexpr int kRdPartBlock = 128;  // gate-gradient partials staged per pass
constexpr int kRdBatch = 8;        // rows loaded before their adds

__global__ __launch_bounds__(kRdThreads) void rdispatch_kernel(RdispArgs p) {
    __shared__ int s_row[kMaxTopK + 1];
    __shared__ int s_idx[kMaxTopK];
    __shared__ float s_w[kMaxTopK], s_dg[kMaxTopK], s_ds[kMaxTopK];
    __shared__ float s_part[kMaxTopK][kRdPartBlock + 1];
    const int tl = blockIdx.x, t = p.t0 + tl, tid = threadIdx.x;
    const int k = p.k;
    if (tid < k + p.with_shared) s_row[tid] = p.tok_prow[(int64_t)tl * p.ld + tid];
    if (tid < k) {
        s_idx[tid] = p.topk_idx[(int64_t)t * k + tid];
        s_w[tid] = p.topk_w[(int64_t)t * k + tid];
    }
    __syncthreads();
    // d out / d w[t,j]: the block partials of slot j added in column order.
    // All threads stage them in LDS with independent loads first, so the
    // ordered sum waits on no chain of global loads.
    float g = 0.0f;
    for (int hb0 = 0; hb0 < p.nhb; hb0 += kRdPartBlock) {
        const int nb = min(kRdPartBlock, p.nhb - hb0);
        for (int i = tid; i < k * nb; i += kRdThreads) {
            const int j = i / nb, hb = i - j * nb;
            s_part[j][hb] = p.dgp[(int64_t)s_row[j] * p.nhb + hb0 + hb];
        }
        __syncthreads();
        if (tid < k)
            for (int hb = 0; hb < nb; ++hb) g = g + s_part[tid][hb];
        __syncthreads();
    }
    if (tid < k) s_dg[tid] = g;
    __syncthreads();
    if (tid == 0) {
        float dot = 0.0f;
        for (int j = 0; j < k; ++j) dot = __builtin_fmaf(s_w[j], s_dg[j], dot);
        for (int j = 0; j < k; ++j) {
            const float ds = s_w[j] * (s_dg[j] - dot);
            s_ds[j] = ds;
            p.dsel[s_row[j]] = ds;
            if (p.dgate) p.dgate[(int64_t)t * k + j] = s_dg[j];
        }
    }
    __syncthreads();
    for (int e = tid; e < p.E; e += kRdThreads) {  // dense row of d out / d logits
        float v = 0.0f;
        for (int j = 0; j < k; ++j) v = s_idx[j] == e ? s_ds[j] : v;
        p.dlogits[(int64_t)t * p.E + e] = v;
    }
    // Rows are taken kRdBatch at a time: every load of a batch is issued
    // before its first add, and the adds then run in slot order (the fixed
    // summation order), so the loads overlap without changing a bit.
    const int nrows = k + p.with_shared;
    for (int c = tid; c < p.H / 8; c += kRdThreads) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        for (int j0 = 0; j0 < nrows; j0 += kRdBatch) {
            intx4 raw[kRdBatch];
#pragma unroll
            for (int u = 0; u < kRdBatch; ++u)
                if (j0 + u < nrows) raw[u] = *(const intx4*)(p.dX + (int64_t)s_row[j0 + u] * p.H + c * 8);
#pragma unroll
            for (int u = 0; u < kRdBatch; ++u) {
                if (j0 + u >= nrows) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = acc[2 * e] + __builtin_bit_cast(float, (uint32_t)raw[u][e] << 16);
                    acc[2 * e + 1] = acc[2 * e + 1] + __builtin_bit_cast(float, (uint32_t)raw[u][e] & 0xffff0000u);
                }
            }
        }
        for (int j0 = 0; j0 < k; j0 += kRdBatch) {
            floatx4 w0[kRdBatch], w1[kRdBatch];
#pragma unroll
            for (int u = 0; u < kRdBatch; ++u)
                if (j0 + u < k) {
                    const floatx4* wr = (const floatx4*)(p.WrT + (int64_t)s_idx[j0 + u] * p.H + c * 8);
                    w0[u] = wr[0];
                    w1[u] = wr[1];
                }
#pragma unroll
            for (int u = 0; u < kRdBatch; ++u) {
                if (j0 + u >= k) break;
                const float ds = s_ds[j0 + u];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[q] = __builtin_fmaf(ds, w0[u][q], acc[q]);
                    acc[4 + q] = __builtin_fmaf(ds, w1[u][q], acc[4 + q]);
                }
            }
        }
        intx4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = (int)((uint32_t)f32_to_bf16_rne(acc[2 * e]) | ((uint32_t)f32_to_bf16_rne(acc[2 * e + 1]) << 16));
        *(intx4*)(p.dx + (int64_t)t * p.H + c * 8) = o;
    }
}

void launch_rdispatch(const RdispArgs& a, int Tm, hipStream_t stream) {
    hipLaunchKernelGGL(rdispatch_kernel, dim3(Tm), dim3(kRdThreads), 0, stream, a);
}

// Router weight gradient dWr = x^T dlogits, with dlogits [T][E] dense (zero
// outside the selected experts), read once from x: workgroup (h block of 64,
// token chunk c) sums its chunk's tokens in ascending order into
// partial[c][h][e]; a second pass adds the chunks in ascending order, so the
// sum over tokens has one fixed order.
constexpr int kDwrChunk = 512, kDwrH = 64, kDwrSub = 64;

__global__ __launch_bounds__(256) void dwr_partial_kernel(DwrArgs p) {
    __shared__ float s_d[kDwrSub][32];  // this pass's 32 experts
    __shared__ uint16_t s_x[kDwrSub][kDwrH];
    const int tid = threadIdx.x, hl = tid & 63, eg = tid >> 6;
    const int h0 = blockIdx.x * kDwrH, h = h0 + hl;
    const int t0 = blockIdx.y * kDwrChunk, t1 = min(p.T, t0 + kDwrChunk);
    for (int pass = 0; pass * 32 < p.E; ++pass) {
        const int eb = pass * 32 + eg * 8;  // this thread's 8 experts
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int ts = t0; ts < t1; ts += kDwrSub) {
            const int n = min(kDwrSub, t1 - ts);
            __syncthreads();
            for (int f = tid; f < n * 32; f += 256) {
                const int e = pass * 32 + (f & 31);
                s_d[f >> 5][f & 31] = e < p.E ? p.dlogits[(int64_t)(ts + (f >> 5)) * p.E + e] : 0.0f;
            }
            // x tile [n][64] bf16: 8 threads per token, 16 bytes each
            for (int f = tid; f < n * 8; f += 256)
                *(intx4*)&s_x[f >> 3][(f & 7) * 8] = *(const intx4*)(p.x + (int64_t)(ts + (f >> 3)) * p.H + h0 + (f & 7) * 8);
            __syncthreads();
            for (int t = 0; t < n; ++t) {
                const float xv = __builtin_bit_cast(float, (uint32_t)s_x[t][hl] << 16);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(xv, s_d[t][eg * 8 + i], acc[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (eb + i < p.E) p.partial[((int64_t)blockIdx.y * p.H + h) * p.E + eb + i] = acc[i];
    }
}

__global__ __launch_bounds__(256) void dwr_reduce_kernel(DwrArgs p, int nchunk) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)p.H * p.E) return;
    float acc = 0.0f;
    for (int c = 0; c < nchunk; ++c) acc = acc + p.partial[(int64_t)c * p.H * p.E + i];
    p.dWr[i] = acc;
}

int dwr_chunks(int T) { return ceil_div(T, kDwrChunk); }

void launch_dwr(const DwrArgs& a, hipStream_t stream) {
    const int nchunk = dwr_chunks(a.T);
    hipLaunchKernelGGL(dwr_partial_kernel, dim3(a.H / kDwrH, nchunk), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(dwr_reduce_kernel, dim3(ceil_div(a.H * a.E, 256)), dim3(256), 0, stream, a, nchunk);
}

// dst[c][r] = src[r][c] for fp32 [rows][cols] (small matrices).
__global__ __launch_bounds__(256) void transpose_f32_kernel(const float* __restrict__ src, int rows, int cols,
                                                            float* __restrict__ dst) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)rows * cols) return;
    const int r = (int)(i / cols), c = (int)(i % cols);
    dst[(int64_t)c * rows + r] = src[i];
}

void launch_transpose_f32(const float* src, int rows, int cols, float* dst, hipStream_t stream) {
    const int64_t n = (int64_t)rows * cols;
    hipLaunchKernelGGL(transpose_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, src, rows, cols,
                       dst);
}

// Row-wise concatenation of the gate and up weights for the input-gradient
// GEMM: Wgu[e][h][c] = c < I ? Wg[e][h][c] : Wu[e][h][c - I].
__global__ __launch_bounds__(256) void concat_gu_kernel(const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu,
                                                        int H, int I, uint16_t* __restrict__ Wgu) {
    const int64_t row = blockIdx.x;  // e * H + h
    for (int c = threadIdx.x * 8; c < 2 * I; c += 256 * 8) {
        const uint16_t* src = c < I ? Wg + row * I + c : Wu + row * I + (c - I);
        *(intx4*)(Wgu + row * 2 * I + c) = *(const intx4*)src;
    }
}

void launch_concat_gu(const uint16_t* Wg, const uint16_t* Wu, int E, int H, int I, uint16_t* Wgu, hipStream_t stream) {
    hipLaunchKernelGGL(concat_gu_kernel, dim3(E * H), dim3(256), 0, stream, Wg, Wu, H, I, Wgu);
}

__global__ __launch_bounds__(256) void copy16_kernel(const intx4* __restrict__ src, int64_t n16, intx4* __restrict__ dst) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) dst[i] = src[i];
}

void launch_copy(const void* src, size_t bytes, void* dst, hipStream_t stream) {
    const int64_t n16 = (int64_t)(bytes / 16);
    const int blocks = (int)((n16 + 255) / 256 < 8192 ? (n16 + 255) / 256 : 8192);
    hipLaunchKernelGGL(copy16_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream, (const intx4*)src, n16,
                       (intx4*)dst);
}

}  // namespace moe
