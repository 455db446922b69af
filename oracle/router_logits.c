/*
 * CPU oracle: router logits in a fixed fp32 summation order.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.
 *
 * What it computes.  Each token's router scores every local expert and the
 * expert choice is re-made at every step (KuCoin flash "Cursor's MoK achieves
 * 2.37x performance boost on NVIDIA GB300 NVL72", section 01).  The score of
 * expert e for token t is the dot product l[t,e] = sum_h x[t,h] * Wr[h,e],
 * plus an optional per-expert bias.  Because the routing decision (an
 * integer) must be reproduced bit for bit, the fp32 rounding order of that
 * dot product is fixed here rather than left to a library:
 *
 *   p[lane] = 0 for lane = 0..63
 *   for h = 0..H-1 (ascending): p[h mod 64] = fmaf(x[t,h], Wr[h,e], p[h mod 64])
 *   for s = 32, 16, 8, 4, 2, 1: p[lane] = p[lane] + p[lane + s] for lane < s
 *   l[t,e] = p[0]  (+ bias[e], one fp32 add, when a bias is given)
 *
 * fmaf is the correctly rounded fused multiply-add of C99.  H must be a
 * multiple of 64.  Inputs are plain fp32 (bf16 activations widen exactly).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define ORACLE_LANES 64

static float logit_fixed_order(const float *xrow, const float *Wr, int H, int E, int e) {
    float p[ORACLE_LANES];
    for (int lane = 0; lane < ORACLE_LANES; ++lane) p[lane] = 0.0f;
    for (int h = 0; h < H; ++h) {
        int lane = h % ORACLE_LANES;
        p[lane] = fmaf(xrow[h], Wr[(size_t)h * E + e], p[lane]);
    }
    for (int s = ORACLE_LANES / 2; s >= 1; s /= 2)
        for (int lane = 0; lane < s; ++lane) p[lane] = p[lane] + p[lane + s];
    return p[0];
}

/* logits[t*E + e] for t < T, e < E.  Returns 0, or -1 if H is not a multiple of 64. */
int oracle_router_logits(int T, int H, int E, const float *x, const float *Wr, const float *bias,
                         float *logits) {
    if (H % ORACLE_LANES != 0 || T < 0 || E <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *xrow = x + (size_t)t * H;
        for (int e = 0; e < E; ++e) {
            float l = logit_fixed_order(xrow, Wr, H, E, e);
            if (bias) l = l + bias[e];
            logits[(size_t)t * E + e] = l;
        }
    }
    return 0;
}
