/*
 * moe.h -- C ABI of the MI355X (gfx950) fused mixture-of-experts layer.
 *
 * One layer, on one GPU: top-k routing, a dispatch that gathers each expert's
 * tokens into contiguous GEMM tiles, the expert SwiGLU FFN as a grouped GEMM,
 * and a combine that forms the weighted sum back in token order, plus the
 * backward pass.  Sources of the method (cited per entry point below):
 *   [KC]  KuCoin flash, "Cursor's MoK achieves 2.37x performance boost on
 *         NVIDIA GB300 NVL72" (sections 01, 02, 03);
 *   [RW]  RuntimeWire, "Cursor open-sources MoK MoE training kernel"
 *         (sections "Cursor's benchmark claims" and "Rebuilding the MoE layer
 *         around communication").
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller (the library
 *     never allocates, frees or keeps them).  Tensors are dense row-major.
 *     "bf16" tensors are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call that takes a stream only enqueues work on it and returns;
 *     nothing synchronises with the host except moe_read_device_status.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     failed check returns a non-zero moe_status and enqueues nothing.
 *   - Calls are re-entrant.  A workspace belongs to one stream at a time.
 *   - Results are deterministic: every floating-point reduction has a fixed
 *     order and no floating-point atomics are used, so the same inputs give
 *     bitwise-identical outputs on every call ([RW], "Rebuilding the MoE layer
 *     around communication": fixed floating-point order for bitwise-identical
 *     output).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

typedef enum moe_status {
    MOE_OK = 0,
    MOE_E_INVALID = 1,     /* null/misaligned pointer, bad size or inconsistent cfg */
    MOE_E_UNSUPPORTED = 2, /* valid request outside what the kernels implement */
    MOE_E_WORKSPACE = 3,   /* workspace / saved / packed buffer smaller than required */
    MOE_E_HIP = 4,         /* a HIP runtime call failed (launch error, bad device) */
    MOE_E_DEVICE = 5       /* a kernel reported an error through the device status word */
} moe_status;

typedef enum moe_prec {
    MOE_PREC_BF16 = 0, /* bf16 operands, fp32 accumulation */
    MOE_PREC_MXFP8 = 1 /* routed experts in MXFP8: OCP E4M3 values, one E8M0 scale per
                          32 elements along each GEMM's contraction axis ([KC] 02:
                          MXFP8 activations inside dispatch / grouped GEMM / SwiGLU) */
} moe_prec;

enum moe_flags {
    /* add one always-on SwiGLU expert of the same shape, in bf16, weight 1, after
       the routed weighted sum ([RW] "Rebuilding...": shared expert kept in BF16) */
    MOE_F_SHARED_EXPERT = 1u << 0,
    /* test mode: every routed expert is the identity (y = x), so combine must
       return the weighted sum of copies of the input */
    MOE_F_IDENTITY_EXPERTS = 1u << 1,
    /* run the forward's expert GEMMs and combine as one launch per grouped GEMM
       and per combine, minibatch by minibatch, instead of the persistent layer
       kernel (same results bit for bit) */
    MOE_F_LAUNCH_PER_GEMM = 1u << 2,
    /* debug, for testing the watchdog: in the persistent layer kernel, GEMM
       workgroup 0 never signals that it has finished the first gate|up phase.
       The waits on that phase then run into their bound (2 s), the launch
       drains, the device status word records MOE_DEV_WAIT_TIMEOUT with the wait
       site as detail, and `out` is unspecified.  No effect on a forward that
       runs one launch per GEMM. */
    MOE_F_DEBUG_DROP_SIGNAL = 1u << 3,
    /* MOE_PREC_MXFP8 only (MOE_E_INVALID otherwise): the routed experts'
       weight-gradient GEMMs take the unquantised bf16 operands instead of
       MXFP8 ones (the variant that keeps only the four forward and
       input-gradient GEMMs in MXFP8).  No effect on the forward. */
    MOE_F_BF16_WGRAD = 1u << 4
};

/* Layer shape and execution choices. */
typedef struct moe_cfg {
    int32_t T;          /* tokens in this call, >= 1 */
    int32_t H;          /* hidden size: multiple of 64 */
    int32_t I;          /* expert intermediate size: multiple of 64 */
    int32_t E;          /* experts on this GPU: 1..256 */
    int32_t k;          /* experts per token: 1..min(E, 16) */
    int32_t minibatch;  /* tokens per ring slot; 0 = automatic (see moe_query_sizes) */
    int32_t ring_slots; /* ring token buffer slots (one minibatch each); 0 = automatic:
                           three groups of minibatches, a group being the
                           minibatches (~8192 tokens) whose expert GEMMs the
                           layer kernel runs as one phase */
    int32_t comm_cus;   /* workgroups (one per CU) dedicated to combine in the
                           persistent layer kernel; 0 = automatic: none, combine
                           runs as tiles of the GEMM workgroups (on one GPU
                           every GEMM phase has more tiles than CUs, and
                           dedicated combine workgroups measured slower at
                           every shape, count and minibatch tried) */
    int32_t prec;       /* moe_prec */
    uint32_t flags;     /* moe_flags */
} moe_cfg;

/* Sizes, in bytes, of the buffers the caller allocates for a cfg. */
typedef struct moe_sizes {
    size_t packed_weights; /* moe_prepare_weights output (routed + shared experts) */
    size_t workspace_fwd;  /* scratch of moe_layer_fwd */
    size_t saved;          /* what moe_layer_fwd keeps for moe_layer_bwd */
    size_t workspace_bwd;  /* scratch of moe_layer_bwd */
    int32_t minibatch;     /* effective tokens per ring slot */
    int32_t ring_slots;    /* effective ring slots */
    int32_t num_minibatches;
    int32_t comm_cus;      /* effective dedicated combine workgroups (0: combine tiles) */
} moe_sizes;

/* Device buffers of one layer's parameters. */
typedef struct moe_weights {
    const float *Wr;    /* [H, E] fp32 router weight */
    const float *bias;  /* [E] fp32 router logit bias, or NULL */
    const void *packed; /* moe_prepare_weights output */
    size_t packed_bytes;
} moe_weights;

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_string(moe_status s);

/* MOE_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

/*
 * Host-only check of a cfg (no GPU needed).  MOE_E_INVALID for T<1, E<1, k<1,
 * k>E, unknown prec or flags, MOE_F_BF16_WGRAD without MOE_PREC_MXFP8;
 * MOE_E_UNSUPPORTED for H or I not a multiple of 64, E>256, k>16, T*k>2^30,
 * or a cfg past the kernels' 32-bit operand offsets: T*H*2, R*H*2, R*4I and
 * 4*I*H bytes must stay below 4 GiB, R being a minibatch's padded rows
 * (256 * (ceil(minibatch * (k + shared) / 256) + E + shared - 1)).
 * moe_query_sizes and every layer call apply the same check.
 */
moe_status moe_validate_cfg(const moe_cfg *cfg);

/*
 * Host-only: buffer sizes and the effective minibatch / ring / CU split of a
 * cfg.  The automatic minibatch gives the GEMM role at least two full waves of
 * output tiles per minibatch ([KC] 02: a minibatch must fill the compute SMs
 * with at least two complete waves of GEMM tasks; too small starves them, too
 * large delays the first compute).
 */
moe_status moe_query_sizes(const moe_cfg *cfg, moe_sizes *out);

/*
 * Convert the caller's bf16 expert weights into the kernels' packed layout
 * (and, for MOE_PREC_MXFP8, into E4M3 codes with E8M0 block scales).
 *   Wg, Wu : [E, H, I] bf16   gate / up projections (g = x Wg[e], u = x Wu[e])
 *   Wd     : [E, I, H] bf16   down projection (y = h Wd[e])
 *   Wsg, Wsu [H, I], Wsd [I, H] bf16: shared expert; NULL unless
 *            cfg->flags has MOE_F_SHARED_EXPERT.
 *   packed : device buffer of at least moe_sizes.packed_weights bytes.
 * Runs on `stream`; the inputs may be freed once the stream has passed it.
 */
moe_status moe_prepare_weights(const moe_cfg *cfg, const uint16_t *Wg, const uint16_t *Wu,
                               const uint16_t *Wd, const uint16_t *Wsg, const uint16_t *Wsu,
                               const uint16_t *Wsd, void *packed, size_t packed_bytes,
                               void *stream);

/*
 * Router ([KC] 01: the router picks several experts for each token and
 * re-decides at every step).  For each of cfg->T tokens:
 *   logits[t,e] = sum_h x[t,h] * Wr[h,e] (+ bias[e]), fp32, summed in a fixed
 *       order: 64 lane partials p[h mod 64] accumulated with fused
 *       multiply-add for ascending h, then a halving tree p[l] += p[l+s] for
 *       s = 32, 16, ..., 1; the bias is one fp32 add after the tree;
 *   topk_idx[t,0..k-1] = the k largest logits, descending, ties to the lower
 *       expert index;
 *   topk_w[t,j] = softmax over the k selected logits (fp32).
 *   x [T,H] bf16; Wr [H,E] fp32; bias [E] fp32 or NULL;
 *   topk_idx [T,k] int32; topk_w [T,k] fp32; logits [T,E] fp32 or NULL.
 * Optionally, the MXFP8 dispatch quantisation of every token row, computed
 * from the values the router reads ([KC] 02: MXFP8 quantisation inside the
 * dispatch instead of a separate kernel; the MXFP8 forward runs exactly this):
 *   x_codes [T,H] uint8: E4M3 codes of x along H, by the rule of
 *       moe_mx_quantize (16-byte aligned);
 *   x_scales: the E8M0 scales (e + 127) in the GEMM operand layout
 *       [ceil(H/128)][T][4] bytes: byte b of dword (g, t) is the scale of
 *       token t's 32-element block 4g + b, bytes past the row's end zero;
 *   both NULL (nothing written) or both set.
 * Inputs must be finite.  MOE_E_INVALID if only one of x_codes, x_scales is
 * given, or x_codes is given and it or x is not 16-byte aligned.
 */
moe_status moe_route(const moe_cfg *cfg, const uint16_t *x, const float *Wr, const float *bias,
                     int32_t *topk_idx, float *topk_w, float *logits, uint8_t *x_codes,
                     uint8_t *x_scales, void *stream);

/*
 * Dispatch layout ([KC] 01: count the tokens of every expert, decide where each
 * lands, and keep each expert's tokens adjacent so that the grouped GEMM gets
 * ordered input; [KC] 02: the receiving side picks the placement itself).
 *   topk_idx [T,k] int32 (values in [0,E), distinct within a token)
 *   counts   [E]   rows of each expert
 *   offsets  [E+1] exclusive prefix sum of counts (offsets[E] = T*k)
 *   row_token[T*k] token of each row; rows of expert e are
 *                  offsets[e] .. offsets[e+1]-1 in ascending token order
 *   tok_row  [T,k] row holding slot j of token t (inverse of row_token)
 * Needs no workspace.  If any index lies outside [0,E), or an expert appears
 * twice among one token's k indices, the kernel writes offsets[E] = -1 and
 * leaves the other outputs unspecified (the host cannot see device data
 * without a sync, so this is the error report of this call).
 */
moe_status moe_dispatch_layout(const moe_cfg *cfg, const int32_t *topk_idx, int32_t *counts,
                               int32_t *offsets, int32_t *row_token, int32_t *tok_row,
                               void *stream);

/*
 * Layer forward: route, layout, dispatch, expert SwiGLU FFN, combine and the
 * final weighted sum ([KC] 03: the measured layer covers scheduling, dispatch,
 * expert FFN, combine and the final weighted sum), minibatch by minibatch
 * through a fixed-size ring token buffer ([KC] 02: a fixed-size ring buffer is
 * reused as soon as combine has sent a batch's results, with no CPU round trip).
 *   out[t] = sum_j topk_w[t,j] * FFN_{topk_idx[t,j]}(x[t])  (+ shared FFN(x[t]))
 *   FFN_e(v) = (silu(v Wg[e]) * (v Wu[e])) Wd[e],  silu(z) = z / (1 + exp(-z))
 *   x [T,H] bf16, out [T,H] bf16.
 *   saved: NULL, or at least moe_sizes.saved bytes that moe_layer_bwd will read.
 *       It starts with the routing of every token: topk_idx [T,k] int32 at
 *       byte 0, then topk_w [T,k] fp32 at the next 256-byte boundary; the
 *       rest (per-minibatch g|u and expert outputs, bf16) is internal.
 *   ws: at least moe_sizes.workspace_fwd bytes, 256-byte aligned.  Its first 256
 *       bytes hold the device status word: zero them once when the workspace
 *       is allocated (moe_read_device_status clears the word after reading).
 */
moe_status moe_layer_fwd(const moe_cfg *cfg, const moe_weights *w, const uint16_t *x,
                         uint16_t *out, void *saved, size_t saved_bytes, void *ws,
                         size_t ws_bytes, void *stream);

/*
 * Layer forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_layer_fwd with saved = NULL (nothing kept for a backward), whose
 * workspace is the library's own static device array of
 * MOE_STATIC_WORKSPACE_BYTES, one per GPU, held from the library's load until
 * the process ends.  Same kernels and bitwise the same `out` as moe_layer_fwd.
 *   cfg, w, x, out: as for moe_layer_fwd.
 *   status: NULL, or a device int32[2] (4-byte aligned) that receives the
 *       device status word of this call after the forward (code, detail: see
 *       moe_read_device_status; {0, 0} when no kernel reported an error).
 * Allocates nothing: the first call on a device looks up the array's device
 * address once (hipGetSymbolAddress).  The status word is cleared by a kernel
 * at the start of every call; the layer kernel's counters are cleared by the
 * forward itself.
 * MOE_E_WORKSPACE if moe_sizes.workspace_fwd of cfg exceeds
 * MOE_STATIC_WORKSPACE_BYTES (checked before any device call; choose a
 * smaller minibatch or ring).  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (on different streams, or from
 * different threads) race and give undefined results.
 */
#define MOE_STATIC_WORKSPACE_BYTES (256u << 20)
moe_status moe_layer_fwd_static(const moe_cfg *cfg, const moe_weights *w, const uint16_t *x,
                                uint16_t *out, int32_t *status, void *stream);

/*
 * Layer backward ([KC] 01: training adds two exchanges in the reverse
 * direction; [KC] 02: reverse-combine then reverse-dispatch).  Gradients of
 * sum(out * dout) with the routing of the forward held fixed:
 *   dx [T,H] bf16; dWg, dWu [E,H,I], dWd [E,I,H], dWr [H,E] fp32 (overwritten);
 *   dWs: NULL, or the shared expert's [H*I | H*I | I*H] fp32 (gate, up, down);
 *   dgate: NULL, or [T,k] fp32 = d(sum out*dout)/d topk_w.
 *   saved: what moe_layer_fwd wrote for the same cfg, weights and x.
 *   ws: at least moe_sizes.workspace_bwd bytes, 256-byte aligned.
 * The router bias is an input, not a parameter: it has no gradient.
 * Each weight gradient sums expert e's rows minibatch by minibatch in token
 * order, so results are bitwise reproducible for a given minibatch size.
 * MOE_PREC_MXFP8: every GEMM of the routed experts takes E4M3 operands with
 * E8M0 scales per 32 elements of its contraction axis (the MXFP8 routed
 * experts of [RW] "Rebuilding the MoE layer around communication"): dY and Wd
 * along H for dH = dY Wd^T; dG|dU and Wg|Wu along I for
 * dX = dG Wg^T + dU Wu^T; and for the weight gradients dWd = h^T dY,
 * dWg = x^T dG, dWu = x^T dU the operands x (the expert's token rows), h, dY,
 * dG and dU along the token rows: within each (minibatch, expert) segment in
 * blocks of 32 rows in token order, the segment's last block zero-padded.
 * Quantisation starts from the fp32 values (bf16 for x).  With
 * MOE_F_BF16_WGRAD the weight gradients use the unquantised bf16 operands
 * instead.  The shared expert stays bf16.
 * MOE_E_UNSUPPORTED in identity-expert mode.
 */
moe_status moe_layer_bwd(const moe_cfg *cfg, const moe_weights *w, const uint16_t *x,
                         const uint16_t *dout, const void *saved, size_t saved_bytes,
                         uint16_t *dx, float *dWg, float *dWu, float *dWd, float *dWr,
                         float *dWs, float *dgate, void *ws, size_t ws_bytes, void *stream);

/*
 * Read (and clear) the device status word kept at the start of a forward or
 * backward workspace: waits for `stream`, then returns MOE_OK, or MOE_E_DEVICE
 * with *code / *detail set to the first error a kernel of that workspace
 * recorded (codes are listed in moe_device_error).  The only call that
 * synchronises with the host.
 */
typedef enum moe_device_error {
    MOE_DEV_OK = 0,
    MOE_DEV_WAIT_TIMEOUT = 1 /* a bounded device-side wait expired; detail = wait site */
} moe_device_error;

moe_status moe_read_device_status(void *ws, void *stream, int32_t *code, int32_t *detail);

/*
 * The MXFP8 quantiser the layer applies to activations and weights ([KC] 02:
 * MXFP8 inside the dispatch / grouped GEMM / SwiGLU path), exposed on its own:
 * OCP Microscaling v1.0 E4M3 codes with one E8M0 scale per 32 consecutive
 * elements of a row.  The scale is 2^e for the smallest e with
 * amax <= 448 * 2^e (clamped to [-127, 127]; an all-zero block gets e = 0);
 * codes are x / 2^e rounded to nearest even, saturating at +-448.
 *   src [rows, cols] bf16 (16-byte aligned), cols a multiple of 32;
 *   codes [rows, cols] uint8 (16-byte aligned); scales [rows, cols/32] uint8 = e + 127.
 */
moe_status moe_mx_quantize(const uint16_t *src, int64_t rows, int32_t cols, uint8_t *codes,
                           uint8_t *scales, void *stream);

/*
 * Kernel timing (diagnostics, for benchmarks).  While enabled, every kernel
 * the library launches is bracketed by a pair of HIP events recorded on the
 * stream it is launched on; moe_timing_read waits for those events and
 * returns, per kernel kind, the launch count and the summed event time since
 * the last moe_timing_enable(1).  Recording costs a few microseconds per
 * launch; with timing off nothing is recorded.  Not re-entrant across threads.
 * moe_timing_enable(1) creates the HIP events (host call; never inside a
 * capture); moe_timing_enable(0) waits for the recorded launches and destroys
 * the events, so read the times before switching timing off.
 */
typedef enum moe_kernel_kind {
    MOE_K_ROUTE = 0,
    MOE_K_LAYOUT = 1,
    MOE_K_GEMM_GATE_UP = 2, /* forward grouped GEMM of gate|up with the SwiGLU epilogue */
    MOE_K_GEMM_DOWN = 3,    /* forward grouped GEMM of the down projection */
    MOE_K_COMBINE = 4,      /* combine, and the backward's reverse-dispatch */
    MOE_K_GATHER = 5,       /* elementwise passes: MXFP8 dispatch quantisation, reverse-combine, SwiGLU backward */
    MOE_K_OTHER = 6,
    MOE_K_WGRAD = 7,        /* weight-gradient grouped GEMMs of the backward (MOE_PREC_MXFP8 without
                               MOE_F_BF16_WGRAD: the routed experts' scaled-MFMA ones) */
    MOE_K_DGRAD_DOWN = 8,   /* backward: dH = dY Wd^T */
    MOE_K_DGRAD_GATE_UP = 9, /* backward: dX = dG Wg^T + dU Wu^T */
    MOE_K_SHARED_GEMM = 10, /* MOE_PREC_MXFP8: the bf16 shared expert's forward and input-gradient GEMMs,
                               and its weight-gradient GEMMs unless MOE_F_BF16_WGRAD */
    MOE_K_LAYER = 11,       /* the persistent layer kernel: every forward expert GEMM and combine */
    MOE_K_COUNT = 12
} moe_kernel_kind;

typedef struct moe_kernel_times {
    int32_t launches[MOE_K_COUNT];
    double ms[MOE_K_COUNT];
    int32_t dropped; /* launches not timed because the event pool was full */
} moe_kernel_times;

moe_status moe_timing_enable(int32_t on);
moe_status moe_timing_read(moe_kernel_times *out);

/*
 * Sustained MFMA rate (diagnostic, for benchmarks; not part of the layer).
 * Launches `blocks` workgroups of 512 threads (eight waves; one workgroup per
 * CU when blocks = 256) on `stream`; every wave issues iters x 32 independent
 * matrix instructions on eight fp32 accumulators: kind 0 = v_mfma_f32_32x32x16_bf16
 * (32768 flops each) on bf16 operands, kind 1 = v_mfma_scale_f32_32x32x64_f8f6f4
 * (131072 flops each) on OCP E4M3 codes with unit E8M0 scales.  Each lane
 * reads its operands once from `operands` (device, operand_bytes >= 16 KiB,
 * 16-byte aligned; the caller picks the values, which set how far the chip
 * lowers its clock under the load).  No memory is touched inside the loop.
 * Writes clocks[0] = shader-clock cycles and clocks[1] = 100 MHz reference
 * ticks over workgroup 0's loop (device, 8-byte aligned), and one float per
 * thread to sink [blocks * 512] (device) so the work is not elided.  The caller
 * times the launch with events on `stream`.  MOE_E_INVALID for an unknown
 * kind, null or misaligned pointers, blocks outside 1..65536, iters < 1;
 * MOE_E_HIP if the launch fails.  Allocates nothing.
 */
moe_status moe_diag_mfma_loop(int32_t kind, const void *operands, int64_t operand_bytes, int32_t blocks,
                              int32_t iters, uint64_t *clocks, float *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
