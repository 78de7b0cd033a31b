/*
 * CPU oracle for the W8A8 MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plainly written
 * definition that the GPU path is checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links or calls it, and it shares no code, header,
 * table or helper with the HIP sources.
 *
 * Every routine is the definition written out with plain loops (OpenMP only
 * splits independent rows/tokens across threads; it never reorders a sum).
 * Floating-point precision follows the pages where they fix it, else fp64,
 * except where a float decides an integer (a quantised code), where the
 * decision is taken in fp32 exactly as the method states it.
 *
 * Sources (web pages, cited by title and section):
 *  [K100AI]  "W8A8 quantisation of MiniMax-M3 on K100AI: an MoE inference
 *            deployment guide" (mhpn.cn) -- sec. 2.1 quantisation maths,
 *            sec. 3.1 batching small expert GEMMs, sec. 3.2 routing buffers.
 *  [HUNYUAN] "Tencent Hunyuan AI Infra: inference optimisation of a 100B
 *            model on Hopper GPUs" (pnsm.cn) -- sec. 1.3 FusedMoE stages.
 *  [DSV4]    "DeepSeek V4 '950' unified FP8 dataflow on H100" (lpnh.cn) --
 *            sec. 2.3 low-precision in / wide accumulator / requantised out,
 *            sec. 2.4 per-output-channel weight scales, sec. 4.1 fp32 router.
 *  [STRATA]  "125B MoE on one RTX 3090" (hncyxsy.com) -- sec. 3.3 grouping
 *            same-expert tokens into one GEMM.
 *
 * Parity pins: every function here is pinned by the CPU tests (hand-worked
 * values, brute force against numpy, closed forms, invariants).  None is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Symmetric INT8 quantisation of one row, [K100AI] sec. 2.1:               */
/*   s = max|x| / 127,  q = clamp(round(x / s), -128, 127),  x ~= q * s.    */
/* Reading adopted (pages silent): round half to even, IEEE fp32 division,  */
/* an all-zero row gives s = 0 and q = 0.                                   */
/* ------------------------------------------------------------------------ */
static void quantize_one_row(const float* x, int64_t cols, int8_t* q, float* s_out) {
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
        float a = fabsf(x[c]);
        if (a > amax) amax = a;
    }
    float s = amax / 127.0f;
    *s_out = s;
    for (int64_t c = 0; c < cols; ++c) {
        if (s == 0.0f) {
            q[c] = 0;
            continue;
        }
        float v = x[c] / s;
        float r = nearbyintf(v); /* default rounding mode: to nearest, ties to even */
        if (r > 127.0f) r = 127.0f;
        if (r < -128.0f) r = -128.0f;
        q[c] = (int8_t)r;
    }
}

/* Per-row quantisation of a [rows][ld] fp32 matrix (first `cols` columns).
 * Used per token for activations and per output channel for weights
 * ([DSV4] sec. 2.4: one weight scale per output channel). */
ORACLE_API void oracle_quantize_rows(const float* x, int64_t rows, int64_t cols, int64_t ld,
                                     int8_t* q, float* scale) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        quantize_one_row(x + r * ld, cols, q + r * cols, scale + r);
}

/* ------------------------------------------------------------------------ */
/* Integer GEMM: acc[m][n] = sum_k a[m][k] * b[n][k], exact in int32.        */
/* b is stored [N][K]: one row per output channel.  [K100AI] sec. 2.1 gives  */
/* the shape [A,K] x [K,N]; storing the second operand transposed is a       */
/* layout choice, not a change of the product.                               */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_gemm_i32(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K,
                                int32_t* acc) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int32_t)a[m * K + k] * (int32_t)b[n * K + k];
            acc[m * N + n] = sum;
        }
    }
}

/* Dense W8A8 GEMM with the scale outer product applied to the int32 result,
 * [K100AI] sec. 2.1: activation scale [A,1], weight scale [1,N].
 * out = ((float)acc * s_a[m]) * s_b[n]  (fp32, this association). */
ORACLE_API void oracle_dense_w8a8(const int8_t* a, const float* s_a, const int8_t* b,
                                  const float* s_b, int64_t M, int64_t N, int64_t K, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int32_t)a[m * K + k] * (int32_t)b[n * K + k];
            float v = (float)sum * s_a[m];
            out[m * N + n] = v * s_b[n];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Router logits on the unquantised activations, [DSV4] sec. 4.1 (the router */
/* stays in full precision).  The oracle accumulates in fp64:                */
/*   l[t][e] = sum_h x[t][h] * wr[e][h]  + bias[e]                           */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_router_logits(const float* x, const float* wr, const float* bias, int64_t T,
                                     int64_t H, int64_t E, double* logits) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double sum = 0.0;
            for (int64_t h = 0; h < H; ++h) sum += (double)x[t * H + h] * (double)wr[e * H + h];
            if (bias) sum += (double)bias[e];
            logits[t * E + e] = sum;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Gate -> top-k -> weights, [HUNYUAN] sec. 1.3 stage list.  Steps:          */
/*  1. softmax over all E experts (fp64, max-subtracted);                   */
/*  2. pick the k experts of largest logit (the order of the probabilities, */
/*     which softmax preserves, but decided on the logits so that           */
/*     probabilities that underflow to zero do not tie), in descending      */
/*     order, a tie going to the lower expert index;                        */
/*  3. renormalise the k picked probabilities to sum to one.                */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_topk_softmax(const double* logits, int64_t T, int64_t E, int64_t k,
                                    int32_t* ids, float* w) {
#pragma omp parallel
    {
        double* p = (double*)malloc((size_t)E * sizeof(double));
        unsigned char* taken = (unsigned char*)malloc((size_t)E);
        double* sel = (double*)malloc((size_t)k * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* l = logits + t * E;
            double lmax = l[0];
            for (int64_t e = 1; e < E; ++e)
                if (l[e] > lmax) lmax = l[e];
            double z = 0.0;
            for (int64_t e = 0; e < E; ++e) {
                p[e] = exp(l[e] - lmax);
                z += p[e];
            }
            for (int64_t e = 0; e < E; ++e) p[e] /= z;

            memset(taken, 0, (size_t)E);
            double sel_sum = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                int64_t best = -1;
                for (int64_t e = 0; e < E; ++e) {
                    if (taken[e]) continue;
                    if (best < 0 || l[e] > l[best]) best = e; /* strict: tie keeps lower index */
                }
                taken[best] = 1;
                ids[t * k + j] = (int32_t)best;
                sel[j] = p[best];
                sel_sum += p[best];
            }
            for (int64_t j = 0; j < k; ++j) w[t * k + j] = (float)(sel[j] / sel_sum);
        }
        free(p);
        free(taken);
        free(sel);
    }
}

/* ------------------------------------------------------------------------ */
/* Permute: contiguous per-expert row segments ([HUNYUAN] sec. 1.3: each     */
/* expert's output gets a contiguous reserved region; [STRATA] sec. 3.3:     */
/* tokens routed to one expert form one group).  Within an expert, rows are  */
/* in ascending token order.  Entries are assignment ids a = t*k + j.        */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_permute(const int32_t* ids, int64_t T, int64_t k, int64_t E, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_assign) {
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < T * k; ++a) counts[ids[a]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t pos = 0;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t j = 0; j < k; ++j)
                if (ids[t * k + j] == e) sorted_assign[pos++] = (int32_t)(t * k + j);
}

/* SiLU(g) = g / (1 + exp(-g)), fp32 arithmetic.  The pages never name the
 * expert non-linearity; the SwiGLU reading is SiLU(gate) * up.  The
 * exponential is taken correctly rounded to fp32 (the double-precision exp
 * rounded once); division and addition are IEEE fp32. */
ORACLE_API float oracle_silu(float g) {
    float e = (float)exp(-(double)g);
    float den = 1.0f + e;
    return g / den;
}

/* ------------------------------------------------------------------------ */
/* Expert FFN for a list of assignments (token t, expert e, weight w):       */
/*  gate-up: acc[i] = sum_h xq[t][h] * wgu[e][i][h], i < 2I (int32),          */
/*           rows 0..I-1 are gate, rows I..2I-1 are up;                      */
/*  dequant in the epilogue ([K100AI] sec. 2.1):                             */
/*           g = ((float)acc[i] * s_x[t]) * s_gu[e][i],                       */
/*           u = ((float)acc[I+i] * s_x[t]) * s_gu[e][I+i];                   */
/*  h = SiLU(g) * u (fp32), requantised per row ([DSV4] sec. 2.3) with the   */
/*  same formula as the activations;                                         */
/*  down:    accd[n] = sum_i hq[i] * wd[e][n][i] (int32);                    */
/*  o[n] = w * (((float)accd[n] * s_h) * s_d[e][n])  -- the routing weight   */
/*  applied before the combine ([HUNYUAN] sec. 1.3 weighted aggregation).    */
/* Optional outputs may be NULL.                                             */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_expert_ffn(int64_t n_assign, const int64_t* a_token, const int32_t* a_expert,
                                  const float* a_weight, const int8_t* x_q, const float* s_x,
                                  int64_t H, int64_t I, const int8_t* w_gu, const float* s_gu,
                                  const int8_t* w_d, const float* s_d, int32_t* acc_gu, float* h_out,
                                  int8_t* h_q, float* s_h, int32_t* acc_d, float* o) {
#pragma omp parallel
    {
        int32_t* acc = (int32_t*)malloc((size_t)(2 * I) * sizeof(int32_t));
        float* h = (float*)malloc((size_t)I * sizeof(float));
        int8_t* hq = (int8_t*)malloc((size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t a = 0; a < n_assign; ++a) {
            const int64_t t = a_token[a];
            const int64_t e = a_expert[a];
            const int8_t* xr = x_q + t * H;
            const int8_t* wg = w_gu + e * (2 * I) * H;
            for (int64_t i = 0; i < 2 * I; ++i) {
                int32_t sum = 0;
                for (int64_t hh = 0; hh < H; ++hh) sum += (int32_t)xr[hh] * (int32_t)wg[i * H + hh];
                acc[i] = sum;
            }
            if (acc_gu) memcpy(acc_gu + a * 2 * I, acc, (size_t)(2 * I) * sizeof(int32_t));
            for (int64_t i = 0; i < I; ++i) {
                float g = ((float)acc[i] * s_x[t]) * s_gu[e * 2 * I + i];
                float u = ((float)acc[I + i] * s_x[t]) * s_gu[e * 2 * I + I + i];
                h[i] = oracle_silu(g) * u;
            }
            if (h_out) memcpy(h_out + a * I, h, (size_t)I * sizeof(float));
            float sh;
            quantize_one_row(h, I, hq, &sh);
            s_h[a] = sh;
            memcpy(h_q + a * I, hq, (size_t)I);
            const int8_t* wdn = w_d + e * H * I;
            for (int64_t n = 0; n < H; ++n) {
                int32_t sum = 0;
                for (int64_t i = 0; i < I; ++i) sum += (int32_t)hq[i] * (int32_t)wdn[n * I + i];
                if (acc_d) acc_d[a * H + n] = sum;
                float v = ((float)sum * sh) * s_d[e * H + n];
                o[a * H + n] = a_weight[a] * v;
            }
        }
        free(acc);
        free(h);
        free(hq);
    }
}

/* Combine: y[t][n] = sum over j = 0..k-1, in that order, of o[t*k+j][n]
 * (fp32), [HUNYUAN] sec. 1.3 weighted aggregation at the end. */
ORACLE_API void oracle_combine(const float* o, int64_t T, int64_t k, int64_t H, float* y) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < H; ++n) {
            float sum = 0.0f;
            for (int64_t j = 0; j < k; ++j) sum += o[(t * k + j) * H + n];
            y[t * H + n] = sum;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 codes, [DSV4] sec. 2.1: the forward weights and activations use  */
/* E4M3 (4 exponent bits, 3 mantissa bits, range about +-448); sec. 2.3:     */
/* fp8 inputs, an fp32 (here: exact) accumulator, the output requantised.   */
/* Layout (the OCP "E4M3FN" format that the +-448 range implies): sign bit,  */
/* 4-bit exponent with bias 7, 3-bit mantissa; exponent 0 holds subnormals   */
/* m * 2^-9; there are no infinities and S.1111.111 is NaN, so the largest   */
/* finite magnitude is 1.75 * 2^8 = 448.                                     */
/* Reading adopted (the pages give no rounding rule): round to the nearest   */
/* finite value, a tie going to the even mantissa; magnitudes beyond 448     */
/* therefore map to 448 (saturation).                                        */
/* ------------------------------------------------------------------------ */
ORACLE_API double oracle_e4m3_decode(uint8_t c) {
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (c & 0x80) ? -mag : mag;
}

/* Nearest finite E4M3 value by a walk over the 127 non-negative finite codes
 * in increasing order (codes 0x00 .. 0x7E increase with the value): the
 * magnitude lies between two consecutive values, and the midpoint decides. */
ORACLE_API uint8_t oracle_e4m3_encode(float v) {
    if (isnan(v)) return 0x7F;
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double a = fabs((double)v);
    uint8_t best = 0x7E; /* beyond the largest value: saturate */
    for (int c = 0; c < 0x7E; ++c) {
        const double lo = oracle_e4m3_decode((uint8_t)c), hi = oracle_e4m3_decode((uint8_t)(c + 1));
        if (a > hi) continue;
        const double mid = 0.5 * (lo + hi); /* exact: both have at most 4 significant bits */
        if (a < mid) best = (uint8_t)c;
        else if (a > mid) best = (uint8_t)(c + 1);
        else best = (c % 2 == 0) ? (uint8_t)c : (uint8_t)(c + 1); /* tie: even mantissa */
        break;
    }
    return (uint8_t)(sign | best);
}

/* Per-row FP8 quantisation, the same scheme as the INT8 one with the E4M3
 * range: s = max|x| / 448 (fp32 division), code = E4M3(x / s) (the quotient
 * an IEEE fp32 division, then rounded as above); an all-zero row gives s = 0
 * and code 0x00. */
ORACLE_API void oracle_quantize_rows_fp8(const float* x, int64_t rows, int64_t cols, int64_t ld,
                                         uint8_t* q, float* scale) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * ld;
        float amax = 0.0f;
        for (int64_t c = 0; c < cols; ++c)
            if (fabsf(xr[c]) > amax) amax = fabsf(xr[c]);
        const float s = amax / 448.0f;
        scale[r] = s;
        for (int64_t c = 0; c < cols; ++c) q[r * cols + c] = (s == 0.0f) ? 0x00 : oracle_e4m3_encode(xr[c] / s);
    }
}

/* ------------------------------------------------------------------------ */
/* Activation scales beyond the per-token absmax.                            */
/*                                                                          */
/* [K100AI] sec. 2.2 (SmoothQuant): a per-channel factor reshapes the        */
/* activations so that their outlier channels flatten, and the weights take  */
/* the inverse factor on the same input channel, which leaves the product    */
/* unchanged.  Here the factor is a given vector col_mul[cols] (choosing it  */
/* needs calibration data): x'[c] = x[c] * col_mul[c] (one fp32 product)     */
/* before the scale is taken; the weights are quantised with 1/col_mul.      */
/*                                                                          */
/* [K100AI] sec. 2.2 and [DSV4] sec. 3.1: a calibrated bound (a high         */
/* percentile times a safety factor) in place of the row maximum; [DSV4]     */
/* sec. 3.1 keeps a static part (that bound) and a dynamic part (the         */
/* per-token scale computed at run time).  Readings adopted:                 */
/*   mode 0, dynamic:  s = max|x'| / Q                                       */
/*   mode 1, clipped:  s = min(max|x'|, clip) / Q   (the static bound caps   */
/*                     the dynamic per-token scale)                          */
/*   mode 2, static:   s = clip / Q for every row                            */
/* with Q = 127 (INT8) or 448 (FP8 E4M3).  Values beyond the scale's range   */
/* saturate: INT8 clamps to [-128, 127], E4M3 to +-448.                      */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_quantize_rows_ex(const float* x, int64_t rows, int64_t cols, int64_t ld,
                                        const float* col_mul, int mode, float clip, int fp8,
                                        void* q_out, float* scale) {
#pragma omp parallel
    {
        float* xs = (float*)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            const float* xr = x + r * ld;
            float amax = 0.0f;
            for (int64_t c = 0; c < cols; ++c) {
                xs[c] = col_mul ? xr[c] * col_mul[c] : xr[c];
                if (fabsf(xs[c]) > amax) amax = fabsf(xs[c]);
            }
            float base = amax;
            if (mode == 1 && clip < amax) base = clip;
            if (mode == 2) base = clip;
            const float s = base / (fp8 ? 448.0f : 127.0f);
            scale[r] = s;
            for (int64_t c = 0; c < cols; ++c) {
                if (fp8) {
                    uint8_t* q = (uint8_t*)q_out + r * cols;
                    q[c] = (s == 0.0f) ? 0x00 : oracle_e4m3_encode(xs[c] / s);
                } else {
                    int8_t* q = (int8_t*)q_out + r * cols;
                    if (s == 0.0f) {
                        q[c] = 0;
                        continue;
                    }
                    float v = nearbyintf(xs[c] / s);
                    if (v > 127.0f) v = 127.0f;
                    if (v < -128.0f) v = -128.0f;
                    q[c] = (int8_t)v;
                }
            }
        }
        free(xs);
    }
}

/* FP8 GEMM accumulator: acc[m][n] = sum_k E4M3(a[m][k]) * E4M3(b[n][k]) in
 * fp64.  Products of two E4M3 values have at most 8 significant bits and
 * magnitudes in [2^-18, 448^2]; a sum of up to 2^13 of them needs at most 49
 * bits, so this fp64 sum is exact for K <= 8192. */
ORACLE_API void oracle_gemm_fp8(const uint8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                                double* acc) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) sum += oracle_e4m3_decode(a[m * K + k]) * oracle_e4m3_decode(b[n * K + k]);
            acc[m * N + n] = sum;
        }
}

/* Dense W8A8 GEMM with FP8 codes: out = ((float)acc * s_a[m]) * s_b[n], the
 * exact accumulator rounded once to fp32, then the scale outer product. */
ORACLE_API void oracle_dense_fp8(const uint8_t* a, const float* s_a, const uint8_t* b, const float* s_b,
                                 int64_t M, int64_t N, int64_t K, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) sum += oracle_e4m3_decode(a[m * K + k]) * oracle_e4m3_decode(b[n * K + k]);
            const float v = (float)sum * s_a[m];
            out[m * N + n] = v * s_b[n];
        }
}

/* Expert FFN with FP8 codes: the INT8 definition above with E4M3 codes, the
 * exact accumulators rounded once to fp32, and h requantised per row to E4M3
 * (s_h = max|h| / 448). */
ORACLE_API void oracle_expert_ffn_fp8(int64_t n_assign, const int64_t* a_token, const int32_t* a_expert,
                                      const float* a_weight, const uint8_t* x_q, const float* s_x,
                                      int64_t H, int64_t I, const uint8_t* w_gu, const float* s_gu,
                                      const uint8_t* w_d, const float* s_d, double* acc_gu, float* h_out,
                                      uint8_t* h_q, float* s_h, double* acc_d, float* o) {
#pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)(2 * I) * sizeof(double));
        float* h = (float*)malloc((size_t)I * sizeof(float));
        uint8_t* hq = (uint8_t*)malloc((size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t a = 0; a < n_assign; ++a) {
            const int64_t t = a_token[a];
            const int64_t e = a_expert[a];
            const uint8_t* xr = x_q + t * H;
            const uint8_t* wg = w_gu + e * (2 * I) * H;
            for (int64_t i = 0; i < 2 * I; ++i) {
                double sum = 0.0;
                for (int64_t hh = 0; hh < H; ++hh)
                    sum += oracle_e4m3_decode(xr[hh]) * oracle_e4m3_decode(wg[i * H + hh]);
                acc[i] = sum;
            }
            if (acc_gu) memcpy(acc_gu + a * 2 * I, acc, (size_t)(2 * I) * sizeof(double));
            for (int64_t i = 0; i < I; ++i) {
                float g = ((float)acc[i] * s_x[t]) * s_gu[e * 2 * I + i];
                float u = ((float)acc[I + i] * s_x[t]) * s_gu[e * 2 * I + I + i];
                h[i] = oracle_silu(g) * u;
            }
            if (h_out) memcpy(h_out + a * I, h, (size_t)I * sizeof(float));
            float sh;
            oracle_quantize_rows_fp8(h, 1, I, I, hq, &sh);
            s_h[a] = sh;
            memcpy(h_q + a * I, hq, (size_t)I);
            const uint8_t* wdn = w_d + e * H * I;
            for (int64_t n = 0; n < H; ++n) {
                double sum = 0.0;
                for (int64_t i = 0; i < I; ++i) sum += oracle_e4m3_decode(hq[i]) * oracle_e4m3_decode(wdn[n * I + i]);
                if (acc_d) acc_d[a * H + n] = sum;
                float v = ((float)sum * sh) * s_d[e * H + n];
                o[a * H + n] = a_weight[a] * v;
            }
        }
        free(acc);
        free(h);
        free(hq);
    }
}

ORACLE_API int oracle_max_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
