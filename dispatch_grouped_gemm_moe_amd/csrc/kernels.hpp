// Launch interfaces between the host runtime (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

// Outputs of the layout kernel.  NULL members are not written.
struct LayoutOut {
    int32_t* counts;      // [E]      rows per routed expert
    int32_t* offsets;     // [E+1]    unpadded row offsets (offsets[E] = -1 on bad input)
    int32_t* row_token;   // [Tm*k]   token (relative to the slice) of each unpadded row
    int32_t* tok_row;     // [Tm,k]   unpadded row of each slot
    LayoutHeader* hdr;    // tile count and error flag for the GEMM kernels
    int32_t* mt_start;    // [Et+1]   first M tile of each expert (Et = E + shared)
    int32_t* prow_start;  // [Et+1]   first padded row of each expert (a multiple of kSegRows)
    int32_t* prow_token;  // [R_pad]  token (absolute) feeding each padded GEMM row
    int32_t* tok_prow;    // [Tm, tok_prow_ld] padded row of each slot; column k = shared row
    int32_t* prow_slot;   // [R_pad]  slot j of each padded row: 0..k-1 routed, k shared, -1 padding
    int32_t* rows_e;      // [Et]     rows of each expert (the shared expert: every token)
    int32_t tok_prow_ld;
    int32_t token_base;   // added to tokens written into prow_token
};

// With xq / xs (MXFP8 dispatch), the router also writes every token row's
// E4M3 codes xq [T][H] and E8M0 scales xs in the GEMM operand scale layout
// [mx_groups(H)][T][4] (the quantisation of launch_mx_quant, bit for bit).
void launch_route(const uint16_t* x, const float* Wr, const float* bias, int T, int H, int E, int k,
                  int32_t* topk_idx, float* topk_w, float* logits, hipStream_t stream, uint8_t* xq = nullptr,
                  uint8_t* xs = nullptr);

void launch_layout(const int32_t* idx, int Tm, int E, int k, int with_shared, const LayoutOut& o,
                   hipStream_t stream);

// Element strides between consecutive minibatches' copies of each LayoutOut
// array (hdr in LayoutHeader units).
struct LayoutStrides {
    int64_t counts, offsets, row_token, tok_row, hdr, mt_start, prow_token, tok_prow, prow_slot, rows_e, prow_start;
};
// Every minibatch of Mb tokens (the last one possibly shorter) in one launch,
// one workgroup each; o holds minibatch 0's pointers.
void launch_layout_batched(const int32_t* idx, int T, int Mb, int E, int k, int with_shared, const LayoutOut& o,
                           const LayoutStrides& st, hipStream_t stream);

// Grouped GEMM over the experts of one minibatch: C[prow, n] = sum_k A[row(prow), k] * B[e][n][k].
struct GemmArgs {
    const uint16_t* A;         // activation rows (bf16)
    const int32_t* a_row_map;  // padded row -> A row, or NULL for the identity
    int64_t lda;
    const uint16_t* B;         // [Et][N][K] bf16, K contiguous
    int64_t b_stride;          // elements between experts
    uint16_t* C;               // [R_pad][ldc] bf16 output
    int64_t ldc;
    int N, K;
    const int32_t* mt_start;   // [Et+1] first M tile of each expert
    const int32_t* prow_start; // [Et+1] first padded row of each expert (M tile ml starts ml * BM after it)
    const LayoutHeader* hdr;
    int Et;
    // kEpiSwiGLU: optional [R_pad][2I] copy of g | u (kept for the backward),
    // bf16 in GU or fp32 in GUf.
    uint16_t* GU;
    int e_begin, e_end;        // experts [e_begin, e_end) are processed
    float* GUf;
    float* Cf;                 // kEpiStore, optional: fp32 output instead of C
    const int32_t* rows_e;     // optional [Et] rows of each expert: padding fragments get no MFMAs
    // Several minibatches in one launch (nmb > 1): minibatch b's tile map,
    // row starts and row counts sit b * mt_ld ints after mt_start /
    // prow_start / rows_e, its A rows (a_row_map NULL) a_mb elements, its row
    // map map_mb ints, its row scales rs_mb floats, its C / Cf rows c_mb
    // elements and its g | u rows (GU / GUf) gu_mb elements after minibatch
    // 0's; the tiles run minibatch by minibatch.
    int nmb, mt_ld;
    int64_t a_mb, c_mb, map_mb, rs_mb, gu_mb;
    // kEpiStore, optional: output row r is acc * row_scale[r] (fp32) before
    // it is rounded and stored
    const float* row_scale;
};

enum GemmEpilogue { kEpiSwiGLU = 0, kEpiStore = 1 };

// GEMM operand scale layout of MXFP8 rows of `cols` elements:
// [mx_groups(cols)][rows][4] bytes, byte b of the dword of (group g, row) the
// E8M0 scale of the row's 32-element block 4g + b (bytes past the row's last
// block zero).  One dword per row thus covers the 128 K elements a GEMM stage
// consumes, so a stage's scales of both operands are a single 4-byte load per
// lane of the workgroup.
__host__ __device__ constexpr int64_t mx_groups(int64_t cols) { return (cols + 127) / 128; }

// MXFP8 grouped GEMM: E4M3 codes with E8M0 scales on both operands.
// Codes: A rows [.][lda] bytes (gathered through a_row_map), B [Et][N][K] bytes.
// Scales in the operand scale layout (one dword per row and 128-element K
// group): SA + g * sa_kstride + row * 4 and SB + e * sb_stride + g * sb_kstride + n * 4.
struct MxGemmArgs {
    const uint8_t* A;
    const int32_t* a_row_map;
    int64_t lda;
    const uint8_t* SA;
    int64_t sa_kstride;
    const uint8_t* B;
    int64_t b_stride;
    const uint8_t* SB;
    int64_t sb_stride, sb_kstride;
    int N, K;
    const int32_t* mt_start;
    const int32_t* prow_start;
    const LayoutHeader* hdr;
    int e_begin, e_end;
    uint16_t* C;               // kEpiStore: bf16 [R_pad][ldc]
    int64_t ldc;
    uint8_t* Cq;               // kEpiSwiGLU: h codes [R_pad][N/2]
    uint8_t* Cs;               // kEpiSwiGLU: h scales, operand layout [mx_groups(N/2)][cs_rows][4]
    int64_t cs_rows;
    float* GU;                 // kEpiSwiGLU, optional: fp32 g | u [R_pad][N] kept for the backward
    float* Cf;                 // kEpiStore, optional: fp32 output instead of C
    const int32_t* rows_e;     // optional [Et] rows of each expert: padding fragments get no MFMAs
    // Several minibatches in one launch (kEpiStore, nmb > 1), as in GemmArgs;
    // a_mb and sa_mb are bytes of codes and scales, c_mb elements of C / Cf.
    int nmb, mt_ld;
    int64_t a_mb, sa_mb, c_mb;
};
void launch_mx_gemm(const MxGemmArgs& a, GemmEpilogue epi, int grid, hipStream_t stream);
// bf16 [rows][cols] -> E4M3 codes [rows][cols] and E8M0 scales; layout 0:
// [rows][cols/32], layout 1: the GEMM operand scale layout.
// With hdr, rows from hdr->prows on are skipped.
void launch_mx_quant(const uint16_t* src, int64_t rows, int cols, int layout, uint8_t* codes, uint8_t* scales,
                     hipStream_t stream, const LayoutHeader* hdr = nullptr);

// Persistent layer kernel (expert GEMMs of every minibatch + combine), see
// mega.hip.  Layouts of every minibatch are precomputed: minibatch b's header
// sits at lay0 + b * lay_bytes, its prow_token / tok_prow at + ly_prow_token /
// + ly_tok_prow, its first-tile map at mt_all + b * mt_ld.  g1/g2 (bf16) or
// m1/m2 (MXFP8) carry the per-layer operands; the per-minibatch pointers are
// filled in by the kernel.  counters: 3 * nmb + 1 ints (per-minibatch gate|up,
// down and combine progress, then the launch's abort word; zeroed by
// launch_mega).  Wait sites recorded in the status detail: 0 ring slot (down),
// 1 ring slot (combine), 2 combine input, 3 down input.
struct MegaArgs {
    int T, H, I, k, Mb, nmb, S, comm, e_end, with_shared, ld_tok_prow, mx;
    int e_mx;  // experts [0, e_mx) run MXFP8 tiles (m1/m2), the rest (the shared expert) bf16 (g1/g2)
    int group;  // minibatches per GEMM / combine phase; S is a multiple of it
    const uint8_t* lay0;
    int64_t lay_bytes, ly_prow_token, ly_tok_prow;
    const int32_t* mt_all;
    const int32_t* prs_all;   // [nmb][mt_ld] first padded row of each expert per minibatch
    const int32_t* rows_all;  // [nmb][mt_ld] rows of each expert per minibatch
    int mt_ld;
    GemmArgs g1, g2;
    MxGemmArgs m1, m2;
    uint8_t* slot0;  // ring slot s at slot0 + s * slot_bytes: h (+ hq, sh), Y
    int64_t slot_bytes, sl_h, sl_y, sl_hq, sl_sh;
    uint8_t* saved_mb0;  // NULL: Y lives in the ring; else minibatch b's g|u at + b * sv_mb, Y at + sv_y
    int64_t sv_mb, sv_y;
    const float* gw;
    uint16_t* out;
    int* counters;
    int* status;
    uint64_t spin_ticks;  // bound of every wait, in s_memrealtime ticks (100 MHz)
    int debug_drop;       // GEMM workgroup 0 skips its signal of gate|up phase 0 (watchdog test)
};
hipError_t launch_mega(const MegaArgs& a, int grid, hipStream_t stream);

// Backward SwiGLU over the padded rows of one minibatch, from dH and the saved
// g | u:  dG = dH * u * silu'(g), dU = dH * silu(g), h = silu(g) * u.
struct SwigluBwdArgs {
    const uint16_t* dH;        // [R_pad][I]
    const uint16_t* GU;        // [R_pad][2I]
    const float* row_w;        // [R_pad] each padded row's weight (0 on padding rows)
    const LayoutHeader* hdr;
    // bf16 operands of the rows from *dgu_row0 on (the experts whose weight
    // gradient, and so input gradient, takes bf16 operands):
    uint16_t* dGU;             // [R_pad][2I]  dG | dU
    uint16_t* HW;              // [R_pad][I]   w * h, zero on padding rows (the down weight gradient's row operand)
    const int32_t* dgu_row0;
    int I;
    int64_t ldt;
    // MXFP8: fp32 inputs instead of dH / GU, and dG | dU also quantised along
    // I from fp32: codes [R_pad][2I], scales in the operand layout
    // [mx_groups(2I)][ldt][4]
    const float* dHf;
    const float* GUf;
    uint8_t* dGUq;
    uint8_t* sdGU;
    // MXFP8 weight-gradient operands, optional (all or none, with dHf): for the
    // rows before *dgu_row0 (the MXFP8 experts' segments) dG | dU and h
    // quantised along the padded rows from fp32, h zero on padding rows
    // (prow_slot < 0): codes [2I][ldt] / [I][ldt], scales in the operand layout
    // [mx_groups(ldt)][2I][4] / [mx_groups(ldt)][I][4]
    const int32_t* prow_slot;
    uint8_t* dGUTq;
    uint8_t* sdGUT;
    uint8_t* HTq;
    uint8_t* sHT;
};
void launch_swiglu_bwd(const SwigluBwdArgs& a, int rpad, hipStream_t stream);

// Weight-gradient GEMM from token-major operands: C[e][m][n] = sum over expert
// e's padded rows r of every minibatch of A[r][m] * B[r][n].  Each operand is
// either a row-major [rows][lda or ldb] buffer per minibatch (a_mb / b_mb
// elements apart) or, for the one `gather` names (1: A, 2: B, 0: neither),
// the token matrix [T][ld] whose row map[b * map_mb + r] is row r of
// minibatch b.  Padding rows must hold zeros in the directly read operand
// (the gathered one then reads a real token's row).  M and N are multiples of
// 64.  Columns n < n_split go to C0 [Et][M][n_split], the rest to
// C1 [Et][M][N - n_split]; with Cs0 set, the last expert writes to Cs0/Cs1.
struct WgradArgs {
    const uint16_t* A;
    const uint16_t* B;
    int64_t lda, ldb, a_mb, b_mb;
    int gather;
    const int32_t* map;  // [nmb][map_mb] row -> token (the layouts' prow_token)
    int64_t map_mb;
    int M, N, n_split, Et, nmb, mt_ld;
    int e_begin;         // experts [e_begin, Et); C0 / C1 are still indexed by e
    const int32_t* prs;  // [nmb][mt_ld] first padded row of each expert, per minibatch
    const int32_t* rows;  // [nmb][mt_ld] rows of each expert, per minibatch: K stops at the last
                          // 64-row stage holding one (the rest of the tile is zero padding)
    float* C0;
    float* C1;
    float* Cs0;
    float* Cs1;
    int mq, nq;  // XCD blocking of each expert's tile grid (set by launch_wgrad)
};

// grid: a multiple of 8 workgroups (XCD-aware dealing).
void launch_wgrad(const WgradArgs& a, int grid, hipStream_t stream);

// MXFP8 weight gradients of experts [0, E): C[e] = A_e^T B_e over every
// padded row of expert e's segments, minibatch by minibatch in order, both
// operands E4M3 codes with E8M0 scales per 32 rows.  A [M][ld] and B [N][ld]
// codes (the padded rows along each row), scales in the operand layout
// [ld / 128][M][4] and [ld / 128][N][4]; minibatch b's copies lie a_mb / b_mb
// code bytes and sa_mb / sb_mb scale bytes after minibatch 0's.  Segments
// start at multiples of 128 rows; padding rows hold zero codes.
struct MxWgradArgs {
    const uint8_t* A;
    const uint8_t* B;
    const uint8_t* SA;
    const uint8_t* SB;
    int64_t ld, a_mb, b_mb, sa_mb, sb_mb;
    int M, N, n_split, E, nmb, mt_ld;
    const int32_t* prs;   // [nmb][mt_ld] first padded row of each expert
    const int32_t* rows;  // [nmb][mt_ld] rows of each expert: K stops at the last 128-row stage holding one
    float* C0;            // columns < n_split: [E][M][n_split]
    float* C1;            // the rest: [E][M][N - n_split], or NULL when n_split == N
    int mq, nq;           // XCD blocking (set by launch_mx_wgrad)
};
void launch_mx_wgrad(const MxWgradArgs& a, int grid, hipStream_t stream);

void launch_grouped_gemm(const GemmArgs& a, GemmEpilogue epi, int grid, hipStream_t stream);

// out[t] = sum_j w[t,j] * Y[tok_prow[t,j]]  (+ Y[tok_prow[t,k]] with the shared expert)
void launch_combine(const uint16_t* Y, int64_t ldy, const int32_t* tok_prow, int tok_prow_ld,
                    const float* w, int k, int with_shared, int H, int Tm, uint16_t* out,
                    hipStream_t stream);

// Y[prow] = x[prow_token[prow]] for every padded row (identity-expert dispatch).
void launch_gather_rows(const uint16_t* x, int H, const int32_t* prow_token, const LayoutHeader* hdr,
                        int max_rows, uint16_t* Y, int64_t ldy, hipStream_t stream);

// Backward: reverse-combine gather over the padded rows of one minibatch.
struct RcombArgs {
    const uint16_t* dout;      // [T][H]
    const uint16_t* x;         // [T][H] (read for the MXFP8 weight-gradient operands only)
    const uint16_t* Y;         // [R_pad][H] saved expert outputs of the minibatch
    const float* topk_w;       // [T][k]
    const int32_t* prow_token;
    const int32_t* prow_slot;
    const LayoutHeader* hdr;
    float* row_w;              // [R_pad], or NULL: each padded row's weight (gate weight, 1 for the shared expert, 0 on padding)
    float* dgp;                // [R_pad][nhb] partial gate gradients
    float* dsel;               // [R_pad] zeroed
    int H, k, nhb;
    int64_t ldt;
    // MXFP8, optional: dY quantised along H from fp32, codes [R_pad][H],
    // scales in the operand layout [mx_groups(H)][ldt][4]; only rows before
    // padded row *dyq_row_end (the experts whose input gradient runs in MXFP8)
    uint8_t* dYq;
    uint8_t* sdY;
    const int32_t* dyq_row_end;
    // MXFP8 weight-gradient operands, optional (both or neither, with dYq):
    // for the rows before *dyq_row_end, dY (from fp32) and x (zero on padding
    // rows) quantised along the padded rows, codes [H][ldt], scales in the
    // operand layout [mx_groups(ldt)][H][4].  (bf16 weight gradients need no
    // copy: they read dout and x through the row map.)
    uint8_t* dYTq;
    uint8_t* sdYT;
    uint8_t* xgTq;
    uint8_t* sxgT;
};
void launch_rcomb_gather(const RcombArgs& a, int rpad, hipStream_t stream);

// Backward: reverse-dispatch of one minibatch (tokens t0 .. t0+Tm-1).
struct RdispArgs {
    const uint16_t* dX;        // [R_pad][H]
    const float* dgp;          // [R_pad][nhb]
    const int32_t* tok_prow;   // [Tm][ld]
    const int32_t* topk_idx;   // [T][k]
    const float* topk_w;       // [T][k]
    const float* WrT;          // [E][H]
    float* dsel;               // [R_pad]
    float* dgate;              // [T][k] or NULL
    uint16_t* dx;              // [T][H]
    float* dlogits;            // [T][E] dense d out / d logits (0 off the selection)
    int t0, H, k, ld, with_shared, nhb, E;
};
void launch_rdispatch(const RdispArgs& a, int Tm, hipStream_t stream);

// Backward: router weight gradient dWr [H][E] = x^T dlogits, tokens summed in
// ascending order in chunks, then the chunks in order (partial: dwr_chunks(T)
// x H x E floats of scratch).
struct DwrArgs {
    const uint16_t* x;         // [T][H]
    const float* dlogits;      // [T][E]
    float* partial;
    float* dWr;                // [H][E]
    int T, H, E;
};
int dwr_chunks(int T);
void launch_dwr(const DwrArgs& a, hipStream_t stream);

void launch_transpose_f32(const float* src, int rows, int cols, float* dst, hipStream_t stream);
void launch_concat_gu(const uint16_t* Wg, const uint16_t* Wu, int E, int H, int I, uint16_t* Wgu, hipStream_t stream);
void launch_copy(const void* src, size_t bytes, void* dst, hipStream_t stream);

// Weight packing (bf16).
void launch_pack_gate_up(const uint16_t* Wg, const uint16_t* Wu, int E, int H, int I, uint16_t* W1t,
                         hipStream_t stream);
void launch_transpose(const uint16_t* src, int batches, int rows, int cols, uint16_t* dst,
                      hipStream_t stream);

}  // namespace moe
