/*
 * nvfp4_oracle.c -- plain, slow, scalar CPU oracle for NVFP4 quantization, expansion and
 * percentile calibration.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load this library.  The product path (the HIP library under
 * bit_gemm_nvfp4_amd/) never calls it, never links it and shares no code, header, table or
 * constant generator with it.
 *
 * Sources (cited by page title and section; no line numbers):
 *   [ADA]  "Qwen-Image NVFP4 on a 16 GB Ada GPU: NVFP4 vs NF4, weight error, speed and the NF4
 *          grain" (efraingaray.com/en/blog/qwen-image-nvfp4-ada/), with its Spanish twin.
 *          [ADA What]   section "What NVFP4 is and how it differs from NF4": E2M1 with values 0..6,
 *                       an FP8 scale per 16 weights, one FP32 global scale per matrix, the stored
 *                       block figure "First NVFP4 block, as stored in the file" and the formula
 *                       weight = E2M1 x block scale x global scale; 4.5 bits per weight.
 *          [ADA Run]    section "Running the NVFP4 weights on Ada": the byte-table expander and
 *                       the nibble-order control.
 *          [ADA Error]  section "Quality: the error of each matrix": percentiles by nearest rank.
 *   [AIO]  "Qwen-Rapid-AIO-NVFP4" (app.alphaneural.io): section "Why This Exists" (FP8 weights
 *          upcast to FP32 before re-quantizing; text-encoder layers without weight_scale) and
 *          "Recommended Model" (p99.9 percentile calibration versus max aggregation).
 *   [VL]   "Qwen3-VL-8B-Instruct-heretic-NVFP4" model card, "Quantization Details": activations
 *          quantized at run time with a per-tensor amax, no baked input scale.
 *
 * Readings where the pages leave a step open (each is a choice, listed with its reason in the
 * design notes of the repository):
 *   R1  global scale g = fl(amax / 2688), 2688 = 6 * 448 (largest E2M1 times largest E4M3).
 *   R2  block scale byte = E4M3 nearest (ties to even mantissa, saturating at 448) of
 *       t = fl(bamax / fl(6 * g)); a zero g gives scale byte 0.
 *   R3  element: d = fl(s * g), r = fl(1 / d), y = fl(|v| * r); magnitude = nearest E2M1
 *       (ties to the even code index, saturating at 6); sign bit = sign bit of v (so -0 and
 *       small negatives give code 0b1000).  s = 0 gives magnitude 0; a non-finite r gives
 *       magnitude 0 for v = 0 and 7 otherwise (y = |v| * inf).
 *   R4  the 16-element block runs along a row (the K / in-features axis); scales are stored
 *       row-major [rows][cols/16]; codes row-major [rows][cols/2], element 2j in the low nibble.
 *   R5  FP8 source: v = fl(e4m3(b) * src_scale), a missing scale meaning 1.0.
 *   R6  expansion: w = fl(e2m1 * s * g) with one rounding (e2m1 * s is exact).
 *   R7  percentile: nearest rank, k = clamp(ceil(p * n / 100), 1, n), over |x| per channel.
 *   R9  matrix statistics ([ADA Error]): relative error = ||W - W_hat||_F / ||W||_F with W_hat the
 *       exact expansion; kurtosis = excess kurtosis m4 / m2^2 - 3 with population central
 *       moments; block ratio = mean over blocks of 64 consecutive elements (row-major order, the
 *       last block possibly shorter) of max|w| / population std of the block, blocks with std 0
 *       left out.
 *   R8  FP8 tensorwise ([VL] "Quantization Details": float8_e4m3fn, tensorwise, round to
 *       nearest; "Runtime / hardware": FP4 weights against dynamically quantized FP8
 *       activations): scale = fl(amax / 448), 448 the largest E4M3, and 1 when amax = 0;
 *       byte = sign bit of v | E4M3 nearest (ties to even, saturating at 448) of fl(|v| / scale).
 *       Dequantized value = e4m3(byte) x scale.
 *   R10 low-rank branch ("Qwen Image 2.1: INT4 + FP4", "What I quantized": FP4 weights with BF16
 *       rank-128 branches): C = A_hat . W_hat^T + (A . V^T) . U^T with U [N x r], V [r x K] bf16
 *       and the branch on the bf16 activations.  Plain float64 matrix products (Python side).
 *
 * Arithmetic precision: every fp32 step above is carried out in IEEE binary32 (the pages fix
 * an FP32 global scale, so the decisions that pick codes are taken in fp32).  Grid rounding is
 * done by enumerating every grid value and comparing distances exactly in double: near a tie
 * the operands share an exponent range, so the double subtractions are exact there.
 * Build: gcc -O2 -std=c99 -fno-fast-math -ffp-contract=off (no fused multiply-add).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* E2M1: sign, 2 exponent bits, 1 mantissa bit.  Magnitudes by code index 0..7 ([ADA What]).   */
/* ------------------------------------------------------------------------------------------ */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double ref_e2m1_value(int code) {
    double m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* Nearest magnitude index for y >= 0 (y not NaN).  Ties go to the even index; anything past 6
 * (including +inf) saturates to index 7.  The explicit test keeps huge y, whose distances to the
 * grid points all round to the same double, out of the enumeration. */
int ref_e2m1_index(double y) {
    if (y > 6.0) return 7;
    int best = 0;
    double bd = fabs(y - E2M1_MAG[0]);
    for (int k = 1; k < 8; k++) {
        double d = fabs(y - E2M1_MAG[k]);
        if (d < bd || (d == bd && (k % 2) == 0)) {
            best = k;
            bd = d;
        }
    }
    return best;
}

/* ------------------------------------------------------------------------------------------ */
/* FP8 E4M3 (OCP e4m3fn): bias 7, no infinity, S.1111.111 is NaN, subnormal step 2^-9.          */
/* ------------------------------------------------------------------------------------------ */
double ref_e4m3_value(int b) {
    int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Nearest non-negative finite E4M3 code for t >= 0 (ties to the even code, i.e. even mantissa;
 * anything past 448 saturates to 0x7E; 0x7F is never produced). */
int ref_e4m3_encode(float t) {
    if (t > 448.0f) return 0x7E; /* saturation; also keeps huge t out of the enumeration */
    int best = 0;
    double bd = fabs((double)t);
    for (int b = 1; b <= 0x7E; b++) {
        double d = fabs((double)t - ref_e4m3_value(b));
        if (d < bd || (d == bd && (b % 2) == 0)) {
            best = b;
            bd = d;
        }
    }
    return best;
}

/* ------------------------------------------------------------------------------------------ */
/* Widening of source formats to fp32 ([AIO Why]: FP8 weights upcast to FP32 before requant).  */
/* ------------------------------------------------------------------------------------------ */
float ref_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float ref_f16_to_f32(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp((double)(1024 + m), e - 25);
    return (float)(s ? -v : v);
}

/* v = fl(e4m3(b) * src_scale), a missing scale meaning 1.0 (R5). */
float ref_e4m3_upcast(uint8_t b, float src_scale) {
    float dec = (float)ref_e4m3_value(b); /* exact: every E4M3 value is an fp32 value */
    return dec * src_scale;
}

/* dtype: 0 fp32, 1 bf16 bits, 2 fp16 bits, 3 e4m3 bytes.  Row stride ld in elements. */
void ref_widen(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ld, const float *src_scale,
               float *out) {
    float sc = src_scale ? *src_scale : 1.0f;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < cols; c++) {
            int64_t i = r * ld + c;
            float v;
            switch (dtype) {
            case 0: v = ((const float *)x)[i]; break;
            case 1: v = ref_bf16_to_f32(((const uint16_t *)x)[i]); break;
            case 2: v = ref_f16_to_f32(((const uint16_t *)x)[i]); break;
            default: v = ref_e4m3_upcast(((const uint8_t *)x)[i], sc); break;
            }
            out[r * cols + c] = v;
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Quantization of fp32 values [rows x cols] (dense, cols % 16 == 0) to NVFP4.                  */
/* Returns flags: bit0 = a non-finite input was seen (outputs are then unspecified).           */
/* ------------------------------------------------------------------------------------------ */
float ref_global_scale(float amax) { return amax / 2688.0f; /* R1 */ }

int ref_block_scale_byte(float bamax, float g) { /* R2 */
    if (g == 0.0f) return 0;
    float six_g = 6.0f * g;
    float t = bamax / six_g;
    return ref_e4m3_encode(t);
}

/* Code of one element given its block's decoded scale s and the global scale g (R3). */
int ref_element_code(float v, float s, float g) {
    int sign = signbit(v) ? 8 : 0;
    if (s == 0.0f) return sign;
    float d = s * g;
    float r = 1.0f / d;
    float y = fabsf(v) * r;
    if (isnan(y)) return sign; /* v = 0 against an infinite reciprocal */
    return sign | ref_e2m1_index((double)y);
}

int ref_quantize_f32(const float *v, int64_t rows, int64_t cols, const float *amax_in, uint8_t *codes,
                     uint8_t *scales, float *g_out) {
    int flags = 0;
    int64_t n = rows * cols;
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        if (!isfinite(v[i])) flags |= 1;
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax_in) amax = *amax_in;
    float g = ref_global_scale(amax);
    *g_out = g;
    int64_t nb = cols / 16;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *blk = v + r * cols + b * 16;
            float bamax = 0.0f;
            for (int j = 0; j < 16; j++) {
                float a = fabsf(blk[j]);
                if (a > bamax) bamax = a;
            }
            int sb = ref_block_scale_byte(bamax, g);
            scales[r * nb + b] = (uint8_t)sb;
            float s = (float)ref_e4m3_value(sb);
            for (int j = 0; j < 16; j += 2) {
                int lo = ref_element_code(blk[j], s, g);
                int hi = ref_element_code(blk[j + 1], s, g);
                codes[r * (cols / 2) + b * 8 + j / 2] = (uint8_t)(lo | (hi << 4)); /* R4: low nibble first */
            }
        }
    }
    return flags;
}

/* ------------------------------------------------------------------------------------------ */
/* FP8 tensorwise quantization of fp32 values [rows x cols] (dense), R8.  Returns flags (bit0 =  */
/* a non-finite input was seen).  amax_in: static amax (values beyond it saturate), or NULL.    */
/* ------------------------------------------------------------------------------------------ */
float ref_fp8_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }

int ref_fp8_byte(float v, float scale) {
    int sign = signbit(v) ? 0x80 : 0;
    float t = fabsf(v) / scale;
    return sign | ref_e4m3_encode(t);
}

int ref_quantize_fp8_f32(const float *v, int64_t rows, int64_t cols, const float *amax_in, uint8_t *out,
                         float *scale_out) {
    int flags = 0;
    int64_t n = rows * cols;
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        if (!isfinite(v[i])) flags |= 1;
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax_in) amax = *amax_in;
    float scale = ref_fp8_scale(amax);
    *scale_out = scale;
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)ref_fp8_byte(v[i], scale);
    return flags;
}

/* ------------------------------------------------------------------------------------------ */
/* Expansion ("expander", [ADA Run]): w = e2m1 x block scale x global scale ([ADA What]).       */
/* ------------------------------------------------------------------------------------------ */
/* Exact value in double: e2m1*s has at most 6 significant bits, times g at most 30 (< 53). */
void ref_dequantize_f64(const uint8_t *codes, const uint8_t *scales, float g, int64_t rows, int64_t cols,
                        double *out) {
    int64_t nb = cols / 16;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < cols; c++) {
            uint8_t byte = codes[r * (cols / 2) + c / 2];
            int code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
            double s = ref_e4m3_value(scales[r * nb + c / 16]);
            out[r * cols + c] = ref_e2m1_value(code) * s * (double)g;
        }
    }
}

/* fp32 output: one rounding of the exact product (R6). */
void ref_dequantize_f32(const uint8_t *codes, const uint8_t *scales, float g, int64_t rows, int64_t cols,
                        float *out) {
    int64_t nb = cols / 16;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < cols; c++) {
            uint8_t byte = codes[r * (cols / 2) + c / 2];
            int code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
            double s = ref_e4m3_value(scales[r * nb + c / 16]);
            out[r * cols + c] = (float)(ref_e2m1_value(code) * s * (double)g);
        }
    }
}

/* bf16 by round-to-nearest-even of an fp32 value (NaN kept quiet). */
uint16_t ref_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

void ref_dequantize_bf16(const uint8_t *codes, const uint8_t *scales, float g, int64_t rows, int64_t cols,
                         uint16_t *out) {
    int64_t n = rows * cols;
    float *tmp = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    ref_dequantize_f32(codes, scales, g, rows, cols, tmp);
    for (int64_t i = 0; i < n; i++) out[i] = ref_f32_to_bf16(tmp[i]);
    free(tmp);
}

/* ------------------------------------------------------------------------------------------ */
/* Percentile calibration ([AIO Recommended]: p99.9 vs max; [ADA Error]: nearest rank).        */
/* ------------------------------------------------------------------------------------------ */
int64_t ref_rank(double p, int64_t n) { /* R7 */
    double kk = ceil(p * (double)n / 100.0);
    int64_t k = (int64_t)kk;
    if (k < 1) k = 1;
    if (k > n) k = n;
    return k;
}

static int cmp_float(const void *a, const void *b) {
    float x = *(const float *)a, y = *(const float *)b;
    return (x > y) - (x < y);
}

/* x: fp32 [rows x cols] dense.  per_channel = 1: one result per column; 0: one for the whole
 * tensor.  out_max may be NULL.  |x| with -0 counted as +0. */
void ref_amax_percentile(const float *x, int64_t rows, int64_t cols, double p, int per_channel, float *out_pct,
                         float *out_max) {
    if (per_channel) {
        float *buf = (float *)malloc(sizeof(float) * (size_t)(rows > 0 ? rows : 1));
        int64_t k = ref_rank(p, rows);
        for (int64_t c = 0; c < cols; c++) {
            for (int64_t r = 0; r < rows; r++) buf[r] = fabsf(x[r * cols + c]);
            qsort(buf, (size_t)rows, sizeof(float), cmp_float);
            out_pct[c] = buf[k - 1];
            if (out_max) out_max[c] = buf[rows - 1];
        }
        free(buf);
    } else {
        int64_t n = rows * cols;
        float *buf = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
        for (int64_t i = 0; i < n; i++) buf[i] = fabsf(x[i]);
        qsort(buf, (size_t)n, sizeof(float), cmp_float);
        int64_t k = ref_rank(p, n);
        out_pct[0] = buf[k - 1];
        if (out_max) out_max[0] = buf[n - 1];
        free(buf);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Quality statistics of one matrix ([ADA Error]; R9).  w: fp32 [rows x cols] dense; codes /    */
/* scales / g: its NVFP4 form (used when has_q).  out[0] relative error (NaN without q),         */
/* out[1] excess kurtosis, out[2] mean block ratio, out[3] mean, out[4] population std,          */
/* out[5] max |w|, out[6] number of blocks in out[2].  Two passes, the plain definitions.        */
/* ------------------------------------------------------------------------------------------ */
void ref_matrix_stats(const float *w, int64_t rows, int64_t cols, const uint8_t *codes, const uint8_t *scales,
                      float g, int has_q, double *out) {
    int64_t n = rows * cols;
    double sum = 0.0, amax = 0.0;
    for (int64_t i = 0; i < n; i++) {
        sum += (double)w[i];
        if (fabs((double)w[i]) > amax) amax = fabs((double)w[i]);
    }
    double mu = sum / (double)n;
    double m2 = 0.0, m4 = 0.0;
    for (int64_t i = 0; i < n; i++) {
        double d = (double)w[i] - mu;
        m2 += d * d;
        m4 += d * d * d * d;
    }
    m2 /= (double)n;
    m4 /= (double)n;
    out[1] = m4 / (m2 * m2) - 3.0;
    out[3] = mu;
    out[4] = sqrt(m2);
    out[5] = amax;
    if (has_q) {
        double *wh = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        ref_dequantize_f64(codes, scales, g, rows, cols, wh);
        double num = 0.0, den = 0.0;
        for (int64_t i = 0; i < n; i++) {
            double d = (double)w[i] - wh[i];
            num += d * d;
            den += (double)w[i] * (double)w[i];
        }
        out[0] = sqrt(num) / sqrt(den);
        free(wh);
    } else {
        out[0] = NAN;
    }
    double rsum = 0.0;
    int64_t cnt = 0;
    for (int64_t b = 0; b < n; b += 64) {
        int64_t e = b + 64 < n ? b + 64 : n;
        double bs = 0.0, bmax = 0.0;
        for (int64_t i = b; i < e; i++) {
            bs += (double)w[i];
            if (fabs((double)w[i]) > bmax) bmax = fabs((double)w[i]);
        }
        double bmu = bs / (double)(e - b), v = 0.0;
        for (int64_t i = b; i < e; i++) v += ((double)w[i] - bmu) * ((double)w[i] - bmu);
        double sd = sqrt(v / (double)(e - b));
        if (sd > 0.0) {
            rsum += bmax / sd;
            cnt++;
        }
    }
    out[2] = cnt > 0 ? rsum / (double)cnt : NAN;
    out[6] = (double)cnt;
}

/* ------------------------------------------------------------------------------------------ */
/* Array forms of the scalar rounding rules, for exhaustive and sampled checks.                 */
/* ------------------------------------------------------------------------------------------ */
void ref_e2m1_index_array(const float *y, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)ref_e2m1_index((double)y[i]);
}

void ref_e4m3_encode_array(const float *t, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)ref_e4m3_encode(t[i]);
}

void ref_f32_to_bf16_array(const float *x, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; i++) out[i] = ref_f32_to_bf16(x[i]);
}
