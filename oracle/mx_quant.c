/*
 * CPU oracle: OCP Microscaling (MX v1.0) MXFP8 quantiser.
 *
 * TEST INFRASTRUCTURE ONLY (see router_logits.c).
 *
 * MoK runs its experts in MXFP8 (KuCoin flash "Cursor's MoK achieves 2.37x
 * performance boost on NVIDIA GB300 NVL72", section 02; RuntimeWire "Cursor
 * open-sources MoK", "Rebuilding the MoE layer around communication").  The
 * pages give no format details, so the OCP MX v1.0 MXFP8 format is taken:
 *   - elements: E4M3 ("FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits,
 *     no infinities, S.1111.111 is NaN, largest finite 448;
 *   - one E8M0 scale 2^e per 32 consecutive elements, stored as e + 127;
 *   - e is the smallest integer with amax <= 448 * 2^e (clamped to [-127, 127]),
 *     0 for an all-zero block;
 *   - each element is x / 2^e rounded to the nearest E4M3 value, ties to the
 *     even code, magnitudes above 448 saturating to 448; the sign is kept.
 * Rows of `cols` values are quantised along the row (cols a multiple of 32).
 */
#include <math.h>
#include <stdint.h>

static double e4m3_decode_pos(int code) { /* code in 0..126 */
    int ex = (code >> 3) & 0xF, m = code & 7;
    if (ex == 0) return ldexp((double)m / 8.0, -6);
    return ldexp(1.0 + (double)m / 8.0, ex - 7);
}

static int e4m3_encode_pos(double a) { /* a >= 0, finite */
    if (a > 448.0) a = 448.0;
    /* first code whose value is >= a (values increase with the code) */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi) / 2;
        if (e4m3_decode_pos(mid) >= a) hi = mid; else lo = mid + 1;
    }
    if (e4m3_decode_pos(lo) == a || lo == 0) return lo;
    double up = e4m3_decode_pos(lo) - a, dn = a - e4m3_decode_pos(lo - 1);
    if (up < dn) return lo;
    if (dn < up) return lo - 1;
    return (lo % 2 == 0) ? lo : lo - 1; /* tie: the even code */
}

static int scale_exponent(double amax) {
    if (amax == 0.0) return 0;
    int p;
    double m = frexp(amax, &p); /* amax = m 2^p, m in [0.5, 1); 448 = 0.875 2^9 */
    int e = p - 9 + (m > 0.875 ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

void oracle_mx_quantize(int64_t rows, int cols, const float *src, uint8_t *codes, uint8_t *scales) {
    const int nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const float *v = src + r * cols + b * 32;
            double amax = 0.0;
            for (int c = 0; c < 32; ++c) {
                double a = fabs((double)v[c]);
                if (a > amax) amax = a;
            }
            int e = scale_exponent(amax);
            scales[r * nb + b] = (uint8_t)(e + 127);
            for (int c = 0; c < 32; ++c) {
                double q = ldexp((double)v[c], -e);
                int code = e4m3_encode_pos(fabs(q));
                if (signbit(q)) code |= 0x80;
                codes[r * cols + b * 32 + c] = (uint8_t)code;
            }
        }
    }
}
