/*
 * NVFP4 reference oracle: a plain, slow, obviously-correct CPU implementation
 * of the NVFP4 block quantizer (absmax, MSE and four-over-six block scales),
 * dequantization,
 * and the W4A16 / W4A4 dot products, all in IEEE fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library; neither includes the other.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared
 * (no FMA contraction: every fp64 operation below rounds exactly once, in the
 * order written).
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB de laptop",
 *        section 2 "Que es realmente NVFP4": the E2M1 bitfield formula and the
 *        grid G, the hierarchical reconstruction W^ = q * s_b * s_g, the
 *        per-element argmin, the absmax scale max|W|/6 and the MSE objective
 *        (box "Derivacion del objetivo de optimizacion MSE vs Absmax").
 *   [P3] "NVFP4 en difusion: la misma cuantizacion, un motor completamente
 *        distinto", section 2 "NVFP4 sin vLLM: torch._scaled_mm a mano":
 *        packed uint8 [out, in/2] codes, float8_e4m3fn [out, in/16] scales,
 *        out = (A*s_a)(B*s_b)^T with a 16-bit output, activations quantized on
 *        every call.
 * Readings where the pages are silent (fixed identically on the GPU side):
 *   R1 nibble order: low nibble = even column.          R2 canonical +0 code.
 *   R3 s_g = fp32(amax_T / (6*448)); amax_T == 0 -> 1.  R4 ties to the even code
 *   (E2M1 and E4M3), E4M3 saturates at 448.              R5 MSE candidates: the
 *   E4M3 values in [a/2, min(2a, 448)] plus the absmax scale; error = fp64
 *   sequential sum of rounded squares; ties keep the smaller scale.
 *   R11 four-over-six: candidates max/(6 s_g) and max/(4 s_g), each rounded
 *   to E4M3; the R5 error decides, ties keep the smaller scale.
 *   R13 activation scale sweep: see oracle_act_scale_errors.
 *   R14 SVDQuant smoothing: see oracle_smooth_factors and oracle_smooth_act.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

/* ---- formats ---------------------------------------------------------- */

/* E2M1 value of a 4-bit code [P1 sec.2, piecewise formula]:
 * sign s (bit 3), exponent e (bits 2..1, bias 1), mantissa m (bit 0);
 * e = 0: 0 or the subnormal 0.5; e > 0: 2^(e-1) * (1 + m/2). */
double oracle_e2m1_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag;
    if (e == 0) mag = m ? 0.5 : 0.0;
    else mag = ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* FP8 E4M3 ("fn") value of a byte [P1 sec.2: 4 exponent + 3 mantissa bits;
 * P3 sec.2: float8_e4m3fn].  Bias 7, subnormals m * 2^-9, S.1111.111 = NaN,
 * no infinities; the bias and NaN encoding follow the OCP FP8 definition. */
double oracle_e4m3_value(int byte) {
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest non-negative finite E4M3 value to a >= 0 (codes 0..126); exact ties
 * go to the even code (even mantissa).  Values above 448 saturate to 448
 * because no larger candidate exists.  [P1 sec.2 absmax scale + reading R4] */
int oracle_e4m3_nearest(double a) {
    /* beyond the top value the top value is nearest (fp64 distances to
     * huge a would all round to the same number) */
    if (a >= 448.0) return 126;
    int best = 0;
    double bestd = fabs(a - oracle_e4m3_value(0));
    for (int c = 1; c <= 126; ++c) {
        double d = fabs(a - oracle_e4m3_value(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) { best = c; bestd = d; }
    }
    return best;
}

/* Nearest E2M1 grid value to x, as a code: q = argmin_{q in G} |x - q|
 * [P1 sec.2, "Fundamento matematico"].  G has 15 distinct values; code 8
 * (-0) is never produced (reading R2).  Exact ties go to the even code. */
int oracle_e2m1_nearest(double x) {
    /* beyond +-6 the end value is nearest (see oracle_e4m3_nearest) */
    if (x >= 6.0) return 7;
    if (x <= -6.0) return 15;
    int best = 0;
    double bestd = fabs(x - 0.0);
    for (int c = 1; c < 16; ++c) {
        if (c == 8) continue;
        double d = fabs(x - oracle_e2m1_value(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) { best = c; bestd = d; }
    }
    return best;
}

/* ---- second-level (per-tensor) scale --------------------------------- */

float oracle_amax(const float* x, int64_t n) {
    double m = 0.0;
    for (int64_t i = 0; i < n; ++i) { double v = fabs((double)x[i]); if (v > m) m = v; }
    return (float)m;
}

/* s_g = fp32(amax_T / 2688), 2688 = 6 * 448: the largest block's absmax scale
 * then lands on the top E4M3 value.  [P1 sec.2: the block scale covers the
 * block's range relative to the tensor; FP32 tensor scale; reading R3]
 * The fp64 quotient rounded to fp32 is the correctly rounded fp32 quotient. */
float oracle_global_scale(float amax_t) {
    if (amax_t == 0.0f) return 1.0f;
    return (float)((double)amax_t / 2688.0);
}

/* ---- one 16-element block -------------------------------------------- */

/* Element codes of a block for a given block scale value sb (reading R2:
 * every code is 0 when the scale is 0). */
static void encode_block(const float* w, double sb, float sg, uint8_t code[16]) {
    double denom = sb * (double)sg;            /* exact: <= 4 + 24 significant bits */
    for (int k = 0; k < 16; ++k) {
        if (sb == 0.0) { code[k] = 0; continue; }
        code[k] = (uint8_t)oracle_e2m1_nearest((double)w[k] / denom);
    }
}

static double block_amax(const float* w) {
    double m = 0.0;
    for (int k = 0; k < 16; ++k) { double v = fabs((double)w[k]); if (v > m) m = v; }
    return m;
}

/* Absmax block scale code: s_b = nearest E4M3 to max|W_k| / (6 * s_g)
 * [P1 sec.2: s_absmax = max_k |W_k| / 6.0, here relative to s_g]. */
int oracle_absmax_scale_code(const float* w, float sg) {
    double a = block_amax(w) / (6.0 * (double)sg);
    return oracle_e4m3_nearest(a);
}

/* Squared reconstruction error of a block for scale value sb, summed in fp64
 * in element order with one rounding per operation [P1 sec.2, MSE objective:
 * sum_k (W_k - s_b s_g Q(W_k / (s_b s_g)))^2; reading R5 fixes the
 * arithmetic]. */
double oracle_block_error(const float* w, float sg, int scale_code) {
    uint8_t code[16];
    double sb = oracle_e4m3_value(scale_code);
    encode_block(w, sb, sg, code);
    double e = 0.0;
    for (int k = 0; k < 16; ++k) {
        double p = (sb * (double)sg) * oracle_e2m1_value(code[k]);   /* exact */
        double d = (double)w[k] - p;
        double sq = d * d;
        e = e + sq;
    }
    return e;
}

/* MSE block scale code [P1 sec.2 MSE objective and the algorithm table:
 * several scales are tried and the one with the least reconstruction error
 * of the block wins].  Candidates (reading R5): the absmax scale plus every positive
 * E4M3 value c with a/2 <= c <= min(2a, 448), a = max|W|/(6 s_g); visited in
 * ascending order, replaced only on a strictly smaller error. */
int oracle_mse_scale_code(const float* w, float sg) {
    double a = block_amax(w) / (6.0 * (double)sg);
    int abs_code = oracle_e4m3_nearest(a);
    int best = -1;
    double best_err = 0.0;
    for (int c = 0; c <= 126; ++c) {
        double v = oracle_e4m3_value(c);
        int in_window = (c >= 1) && (a / 2.0 <= v) && (v <= 2.0 * a);
        if (!in_window && c != abs_code) continue;
        double err = oracle_block_error(w, sg, c);
        if (best < 0 || err < best_err) { best = c; best_err = err; }
    }
    return best;
}

/* Four-over-six block scale code [P1 sec.2, algorithm table: each block
 * chooses between two possible largest values, 4 or 6, whichever gives the
 * smaller error].  Reading R11: the two candidates are the nearest E4M3
 * values to max|W| / (6 s_g) (the absmax scale: the block maximum lands on
 * 6) and to max|W| / (4 s_g) (it lands on 4); the error is the MSE
 * objective's (R5) and a tie keeps the smaller scale, i.e. the first. */
int oracle_4o6_scale_code(const float* w, float sg) {
    double m = block_amax(w);
    int c6 = oracle_e4m3_nearest(m / (6.0 * (double)sg));
    int c4 = oracle_e4m3_nearest(m / (4.0 * (double)sg));
    if (c4 == c6) return c6;
    double e6 = oracle_block_error(w, sg, c6);
    double e4 = oracle_block_error(w, sg, c4);
    return e4 < e6 ? c4 : c6;
}

/* ---- whole tensors ---------------------------------------------------- */

/* Quantize a row-major [rows, cols] fp32 tensor (cols % 16 == 0; bf16 inputs
 * are passed here widened to fp32, which is exact).
 *   method 0 = absmax, 1 = MSE, 2 = four-over-six.
 *   *sg: if sg_given, read; else written with oracle_global_scale(amax).
 *   codes [rows, cols/2]: byte i = code(W[2i]) | code(W[2i+1]) << 4 (R1).
 *   scales [rows, cols/16]: E4M3 byte of each block's scale.
 * Returns 0, or -1 on a bad shape. */
int oracle_quantize(int method, const float* x, int64_t rows, int64_t cols,
                    int sg_given, float* sg, uint8_t* codes, uint8_t* scales, int threads) {
    if (rows < 0 || cols < 0 || cols % 16 != 0) return -1;
    int64_t n = rows * cols;
    if (!sg_given) *sg = oracle_global_scale(oracle_amax(x, n));
    float s_g = *sg;
    int64_t nblocks = n / 16;
    #pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t b = 0; b < nblocks; ++b) {
        const float* w = x + 16 * b;
        int sc = method == 0 ? oracle_absmax_scale_code(w, s_g)
               : method == 1 ? oracle_mse_scale_code(w, s_g) : oracle_4o6_scale_code(w, s_g);
        uint8_t code[16];
        encode_block(w, oracle_e4m3_value(sc), s_g, code);
        scales[b] = (uint8_t)sc;
        for (int i = 0; i < 8; ++i) codes[8 * b + i] = (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));
    }
    return 0;
}

/* Dequantize: W^ = q * s_b * s_g [P1 sec.2], returned as the fp32 rounding of
 * the exact value (q * s_b * s_g has <= 30 significant bits, exact in fp64). */
int oracle_dequant(const uint8_t* codes, const uint8_t* scales, float sg,
                   int64_t rows, int64_t cols, float* out) {
    if (rows < 0 || cols < 0 || cols % 16 != 0) return -1;
    int64_t n = rows * cols;
    for (int64_t i = 0; i < n; ++i) {
        int code = (i & 1) ? (codes[i / 2] >> 4) : (codes[i / 2] & 15);
        double v = oracle_e2m1_value(code) * oracle_e4m3_value(scales[i / 16]) * (double)sg;
        out[i] = (float)v;
    }
    return 0;
}

/* Exact dequantized element as an fp64 (no rounding). */
static double wq(const uint8_t* codes, const uint8_t* scales, float sg, int64_t row, int64_t K, int64_t k) {
    int64_t i = row * K + k;
    int code = (i & 1) ? (codes[i / 2] >> 4) : (codes[i / 2] & 15);
    return oracle_e2m1_value(code) * oracle_e4m3_value(scales[i / 16]) * (double)sg;
}

/* W4A16 dot products [P1 sec.2: in W4A16 the weights stay in 4 bits and are
 * widened to 16 bits for the multiply]: y*[m,n] = sum_k x[m,k] * W^[n,k] in fp64 for each
 * requested (m, n) pair, with tau = 1e-5 * sum_k |x[m,k]| |W^[n,k]|. */
int oracle_dot_w4a16(const float* x, const uint8_t* w_codes, const uint8_t* w_scales, float sgw,
                     int64_t K, const int64_t* pm, const int64_t* pn, int64_t npairs,
                     double* y, double* tau, int threads) {
    if (K % 16 != 0) return -1;
    #pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t p = 0; p < npairs; ++p) {
        double s = 0.0, t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = (double)x[pm[p] * K + k];
            double b = wq(w_codes, w_scales, sgw, pn[p], K, k);
            s = s + a * b;
            t = t + fabs(a) * fabs(b);
        }
        y[p] = s;
        tau[p] = 1e-5 * t;
    }
    return 0;
}

/* W4A4 dot products [P3 sec.2: out = (A s_a)(B s_b)^T]: both operands are
 * NVFP4 tensors (activation codes from oracle_quantize with method 0, the
 * per-call activation quantization of P3 sec.2).  y*[m,n] = sum_k A^[m,k] W^[n,k]
 * in fp64, tau = 1e-5 * sum_k |A^||W^|. */
int oracle_dot_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, float sga,
                    const uint8_t* w_codes, const uint8_t* w_scales, float sgw,
                    int64_t K, const int64_t* pm, const int64_t* pn, int64_t npairs,
                    double* y, double* tau, int threads) {
    if (K % 16 != 0) return -1;
    #pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t p = 0; p < npairs; ++p) {
        double s = 0.0, t = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = wq(a_codes, a_scales, sga, pm[p], K, k);
            double b = wq(w_codes, w_scales, sgw, pn[p], K, k);
            s = s + a * b;
            t = t + fabs(a) * fabs(b);
        }
        y[p] = s;
        tau[p] = 1e-5 * t;
    }
    return 0;
}

/* Low-rank branch of a fused LoRA layer [P3 sec.3: y = W_4bit x + B (A x),
 * the second term in 16 bits with rank r in the tens, added to the quantized
 * product before the layer returns].  x [M, K], A [r, K], B [N, r] hold the
 * 16-bit (bf16) values widened to fp32.  For each requested (m, n):
 *   L*_j = sum_k x[m,k] A[j,k] (fp64),  y*_L = sum_j L*_j B[n,j] (fp64),
 *   tau_L = 2^-8 sum_j |L*_j| |B[n,j]| + 1e-5 sum_j (sum_k |x[m,k] A[j,k]|) |B[n,j]|
 * (reading R12: L is held in bf16 between the two products -- one rounding,
 * at most 2^-8 relative -- and the 1e-5 term is the product tolerance of R9
 * applied to the down-projection sums). */
int oracle_lora_term(const float* x, const float* A, const float* B, int64_t r, int64_t K,
                     const int64_t* pm, const int64_t* pn, int64_t npairs,
                     double* y, double* tau, int threads) {
    if (r <= 0 || K <= 0) return -1;
    #pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int64_t p = 0; p < npairs; ++p) {
        const float* xr = x + pm[p] * K;
        const float* br = B + pn[p] * r;
        double s = 0.0, t = 0.0;
        for (int64_t j = 0; j < r; ++j) {
            const float* ar = A + j * K;
            double l = 0.0, la = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double v = (double)xr[k] * (double)ar[k];
                l = l + v;
                la = la + fabs(v);
            }
            double b = (double)br[j];
            s = s + l * b;
            t = t + ldexp(fabs(l) * fabs(b), -8) + 1e-5 * la * fabs(b);
        }
        y[p] = s;
        tau[p] = t;
    }
    return 0;
}

/* ---- static activation tensor scale: FP8 candidate sweep --------------- */

/* Errors of the candidate static activation tensor scales over one batch of
 * calibration activations, added to err[0..16].
 * [P1 sec.1, "Tres preguntas", question 3: activation scales have to be
 * calibrated on real activations whose ranges are recorded; P1 sec.2, box
 * "En tu proyecto": the MSE calibration also sweeps candidate activation
 * scales in FP8.]  Reading R13: candidate c (0..16) puts the block scale of
 * the calibration set's largest block on the E4M3 value v_c = E4M3(126 - c),
 * i.e. 448 down to 112, so s_c = fp32(amax / (6 v_c)) (s_c = 1 for every c
 * when amax == 0; c = 0 is the dynamic rule's s_g).  A candidate's error is
 * the sum over every block, in order, of the absmax-quantized block's squared
 * error (R5 arithmetic) under s_c, accumulated across batches in call order.
 * n must be a multiple of 16. */
int oracle_act_scale_errors(const float* x, int64_t n, float amax, double* err, int threads) {
    if (n % 16 != 0) return -1;
    #pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
    for (int c = 0; c < 17; ++c) {
        float s = amax == 0.0f ? 1.0f : (float)((double)amax / (6.0 * oracle_e4m3_value(126 - c)));
        double e = err[c];
        for (int64_t b = 0; b < n / 16; ++b) {
            const float* w = x + 16 * b;
            e = e + oracle_block_error(w, s, oracle_absmax_scale_code(w, s));
        }
        err[c] = e;
    }
    return 0;
}

/* ---- SVDQuant smoothing ------------------------------------------------ */

/* Nearest bf16 value (8 significant bits, fp32's exponent range) to x, ties
 * to the even significand: x = f 2^e with f in [0.5, 1), so the spacing of
 * bf16 values around x is 2^(e - 8) (2^-133 below the normal range). */
static double bf16_nearest(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(x, &e);
    int q = (e < -125 ? -125 : e) - 8;
    return ldexp(nearbyint(ldexp(x, -q)), q);
}

/* Per-input-channel smoothing factors [P3 sec.3: SVDQuant first moves the
 * activation outliers into the weights by scaling channel by channel].
 * Reading R14: lambda_k = sqrt(a_k / w_k) (migration strength 1/2), a_k the
 * calibration max |x| of channel k, w_k the max |W| of input column k, each
 * operation in fp64 and the result rounded to fp32; lambda_k = 1 when a_k or
 * w_k is 0.  mult_k = fp32(1 / lambda_k) is what the activation is
 * multiplied by. */
void oracle_smooth_factors(const float* a_amax, const float* w_amax, int64_t K, float* lambda, float* mult) {
    for (int64_t k = 0; k < K; ++k) {
        double a = (double)a_amax[k], w = (double)w_amax[k];
        float l = (a == 0.0 || w == 0.0) ? 1.0f : (float)sqrt(a / w);
        lambda[k] = l;
        mult[k] = (float)(1.0 / (double)l);
    }
}

/* Smoothed activation x^_{m,k} = bf16(fp32(x_{m,k} mult_k)) (reading R14:
 * the layer's 16-bit input after the folded per-channel scale; the product
 * of a bf16 and an fp32 is exact in fp64, so the fp32 rounding is the
 * correctly rounded product). */
void oracle_smooth_act(const float* x, const float* mult, int64_t M, int64_t K, float* out) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float p = (float)((double)x[m * K + k] * (double)mult[k]);
            out[m * K + k] = (float)bf16_nearest((double)p);
        }
}
