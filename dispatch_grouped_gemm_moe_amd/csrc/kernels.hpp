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
    int32_t* mt_start;    // [Et+1]   first BM-tile of each expert (Et = E + shared)
    int32_t* prow_token;  // [R_pad]  token (absolute) feeding each padded GEMM row
    int32_t* tok_prow;    // [Tm, tok_prow_ld] padded row of each slot; column k = shared row
    int32_t tok_prow_ld;
    int32_t token_base;   // added to tokens written into prow_token
};

void launch_route(const uint16_t* x, const float* Wr, const float* bias, int T, int H, int E, int k,
                  int32_t* topk_idx, float* topk_w, float* logits, hipStream_t stream);

void launch_layout(const int32_t* idx, int Tm, int E, int k, int with_shared, const LayoutOut& o,
                   hipStream_t stream);

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
    const int32_t* mt_start;   // [Et+1]
    const LayoutHeader* hdr;
    int Et;
};

enum GemmEpilogue { kEpiSwiGLU = 0, kEpiStore = 1 };

void launch_grouped_gemm(const GemmArgs& a, GemmEpilogue epi, int grid, hipStream_t stream);

// out[t] = sum_j w[t,j] * Y[tok_prow[t,j]]  (+ Y[tok_prow[t,k]] with the shared expert)
void launch_combine(const uint16_t* Y, int64_t ldy, const int32_t* tok_prow, int tok_prow_ld,
                    const float* w, int k, int with_shared, int H, int Tm, uint16_t* out,
                    hipStream_t stream);

// Y[prow] = x[prow_token[prow]] for every padded row (identity-expert dispatch).
void launch_gather_rows(const uint16_t* x, int H, const int32_t* prow_token, const LayoutHeader* hdr,
                        int max_rows, uint16_t* Y, int64_t ldy, hipStream_t stream);

// Weight packing (bf16).
void launch_pack_gate_up(const uint16_t* Wg, const uint16_t* Wu, int E, int H, int I, uint16_t* W1t,
                         hipStream_t stream);
void launch_transpose(const uint16_t* src, int batches, int rows, int cols, uint16_t* dst,
                      hipStream_t stream);

}  // namespace moe
