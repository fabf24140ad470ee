/*
 * Plain CPU oracle for the BitLinear forward path with I2_S ternary weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline
 * leg of the benchmark may load this code.  It shares nothing with the GPU
 * library (no headers, helpers or tables): it is written from the pages'
 * definitions, step by step, single-threaded, without SIMD, in double
 * precision wherever the pages leave the precision open.
 *
 * Sources (web pages, cited by title and section):
 *   [EMB]  "BitNet Embeddings GGUF Conversion Implementation",
 *          section 1 "Background" (the per-projection pattern and the model
 *          table with rms_norm_eps), section 3 "I2_S Ternary Packing",
 *          section 4.5 "load_tensors" (RMSNorm then multiply by the norm weight).
 *   [INF]  "BitNet Inference Framework" (doc-search digest), sections
 *          "Quantization and Encoding", "Data Layout", "Quantization (W1.58A8)",
 *          "Architectural Details".
 *   [GEMV] "gguf-gemv", sections on supported block types and "Requirements"
 *          (128-element I2_S blocks, one f32 tensor-wide scale, K a multiple of
 *          128).
 *   [EMB s3 types, s6.1] norm weights are stored as float16 (the tensor type
 *          table of section 3) and multiplied into the f32 activations
 *          elementwise (section 6.1, F16 norm weight support).
 *   [EMB s4.5 FFN] the FFN per-projection norms: act(gate) * up, then the
 *          down projection's RMSNorm and norm weight, then down; the
 *          activation per model from the [EMB s1] table (SiLU for Qwen3,
 *          gelu_pytorch_tanh for Gemma3).
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   R1  Weight W is row-major [N][K] (output x input); 128-value blocks run
 *       along K inside a row.
 *   R2  In-block order: byte j (0..31) of a block holds elements j, j+32,
 *       j+64, j+96 of the block in fields c0, c1, c2, c3 (bits 7:6, 5:4, 3:2,
 *       1:0).
 *   R3  round() is round-half-to-even.
 *   R4  sum |w| is accumulated in double in memory order; the scale is
 *       rounded to float32 once (the appended value) and the weight codes are
 *       decided with a float32 multiply by that stored scale.  An all-zero
 *       tensor packs as all-zero codes (code 1) with scale 1.0f.
 *   R5  Activation quantization is symmetric: s = 127/absmax, codes clamped to
 *       [-127, 127]; absmax is taken after the norm-weight multiply; an
 *       all-zero row gives zero codes and factor 0.
 *   R6  RMSNorm: x / sqrt(mean(x^2) + eps) * norm_w, norm_w used as given.
 *   R7  Epilogue: y = acc * (absmax/127) / scale, no bias.
 *   R8  SiLU(z) = z / (1 + exp(-z)); gelu_pytorch_tanh is the tanh
 *       approximation of GELU, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
 *       (Hendrycks and Gimpel's published form); the glue product and the
 *       down projection's input steps run in double.
 *   R9  A projection without a norm weight (norm_w NULL; [EMB s4.5]: the
 *       projection's input is the shared input itself when its norm tensor
 *       is absent) is quantized from x unnormalised: codes from max|x|,
 *       factor = max|x| / 127.
 *   R10 A float16 norm weight is widened to its exact value (every binary16
 *       number is exactly representable in float32 and double) and then used
 *       as a float32 norm weight.  NaN and infinite halves decode as such.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_OK 0
#define REF_ERR_ARG -1
#define REF_ERR_CODE3 -2
#define REF_ERR_OVERFLOW -3
#define REF_ERR_NOMEM -4
#define REF_ERR_NONFINITE -5

#define BLOCK 128 /* values per I2_S block [EMB s3], [INF "Data Layout"] */

/* Bytes of an I2_S buffer: N*K/4 code bytes plus the appended f32 scale
 * [EMB s3], [INF "Data Layout"]. */
int64_t ref_i2s_packed_bytes(int64_t K, int64_t N) {
    if (K <= 0 || N <= 0 || K % BLOCK != 0) return 0;
    return N * K / 4 + 4;
}

/* Where element (n, k) lives (R1, R2): byte index and bit shift. */
static void ref_locate(int64_t K, int64_t n, int64_t k, int64_t* byte, int* shift) {
    int64_t block = k / BLOCK;  /* block along K in row n */
    int64_t within = k % BLOCK; /* 0..127 */
    int64_t field = within / 32;/* c0..c3 */
    int64_t j = within % 32;    /* byte inside the block */
    *byte = n * (K / 4) + block * 32 + j;
    *shift = 6 - 2 * (int)field; /* c0 at bits 7:6 ... c3 at bits 1:0 */
}

/* Absmean ternary quantization and I2_S packing [EMB s3], [INF "Quantization
 * and Encoding"]: scale = 1/mean|w|, q = round(w*scale) clamped to [-1,1],
 * code = q + 1 (-1 -> 0, 0 -> 1, +1 -> 2), then four codes per byte. */
/* IEEE 754 binary16 -> float, from the format's definition: 1 sign bit, 5
 * exponent bits with bias 15, 10 fraction bits; exponent 0 holds zero and the
 * subnormals f * 2^-24, exponent 31 infinity (f = 0) or NaN. */
void ref_half_to_float(const uint16_t* h, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) {
        const int sign = (h[i] >> 15) & 1;
        const int e = (h[i] >> 10) & 31;
        const int f = h[i] & 1023;
        double v;
        if (e == 0) v = ldexp((double)f, -24);
        else if (e == 31) v = f == 0 ? INFINITY : NAN;
        else v = ldexp((double)(1024 + f), e - 25);
        out[i] = (float)(sign ? -v : v);
    }
}

int ref_i2s_pack(const float* w, int64_t K, int64_t N, uint8_t* out, float* scale_out) {
    if (!w || !out || K <= 0 || N <= 0 || K % BLOCK != 0) return REF_ERR_ARG;
    int64_t total = N * K;
    double sum_abs = 0.0;
    for (int64_t i = 0; i < total; ++i) {
        if (!isfinite(w[i])) return REF_ERR_NONFINITE;
        sum_abs += fabs((double)w[i]);
    }
    double mean = sum_abs / (double)total;
    float scale = (mean == 0.0) ? 1.0f : (float)(1.0 / mean);

    memset(out, 0, (size_t)(total / 4));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            float t = w[n * K + k] * scale;      /* one f32 rounding */
            float r = nearbyintf(t);             /* half to even (R3) */
            int q = (r > 1.0f) ? 1 : (r < -1.0f) ? -1 : (int)r;
            int code = q + 1;
            int64_t byte;
            int shift;
            ref_locate(K, n, k, &byte, &shift);
            out[byte] |= (uint8_t)(code << shift);
        }
    }
    memcpy(out + total / 4, &scale, 4); /* appended little-endian f32 */
    if (scale_out) *scale_out = scale;
    return REF_OK;
}

/* Inverse of the packing: ternary values q in {-1,0,1} as int8 [N][K] and the
 * stored scale.  A field holding 3 is not a valid code. */
int ref_i2s_unpack(const uint8_t* packed, int64_t K, int64_t N, int8_t* q_out, float* scale_out) {
    if (!packed || !q_out || K <= 0 || N <= 0 || K % BLOCK != 0) return REF_ERR_ARG;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t byte;
            int shift;
            ref_locate(K, n, k, &byte, &shift);
            int code = (packed[byte] >> shift) & 3;
            if (code == 3) return REF_ERR_CODE3;
            q_out[n * K + k] = (int8_t)(code - 1);
        }
    }
    if (scale_out) memcpy(scale_out, packed + N * K / 4, 4);
    return REF_OK;
}

/* Per-projection RMSNorm [EMB s1, s4.5] followed by per-token absmax int8
 * quantization [INF "Quantization (W1.58A8)"], for each row m:
 *   r     = 1 / sqrt(mean_k x^2 + eps)
 *   xhat  = x * r * norm_w
 *   a     = max |xhat|
 *   q     = clamp(round(xhat * 127 / a), -127, 127)
 *   factor= a / 127       (the activation dequantization factor)
 * All arithmetic in double. */
/* One row of the steps above, on a row given in double.  norm_w NULL: no
 * RMSNorm (R9), xhat = x. */
static void quant_row(const double* row, const float* norm_w, int64_t K, float eps, int8_t* q,
                      double* factor) {
    double r = 1.0;
    if (norm_w) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) ss += row[k] * row[k];
        r = 1.0 / sqrt(ss / (double)K + (double)eps);
    }

    double a = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double xhat = norm_w ? row[k] * r * (double)norm_w[k] : row[k];
        if (fabs(xhat) > a) a = fabs(xhat);
    }
    if (a == 0.0) {
        for (int64_t k = 0; k < K; ++k) q[k] = 0;
        *factor = 0.0;
        return;
    }
    double s = 127.0 / a;
    for (int64_t k = 0; k < K; ++k) {
        double xhat = norm_w ? row[k] * r * (double)norm_w[k] : row[k];
        double v = nearbyint(xhat * s);
        if (v > 127.0) v = 127.0;
        if (v < -127.0) v = -127.0;
        q[k] = (int8_t)v;
    }
    *factor = a / 127.0;
}

int ref_quant(const float* x, const float* norm_w, int64_t M, int64_t K, float eps,
              int8_t* q_out, double* factor_out) {
    if ((M > 0 && (!x || !q_out || !factor_out)) || M < 0 || K <= 0) return REF_ERR_ARG;
    double* row = (double*)malloc((size_t)K * sizeof(double));
    if (!row) return REF_ERR_NOMEM;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) row[k] = (double)x[m * K + k];  /* exact */
        quant_row(row, norm_w, K, eps, q_out + m * K, factor_out + m);
    }
    free(row);
    return REF_OK;
}

/* FFN glue [EMB s4.5 FFN]: the activation of the gate projection's output. */
#define REF_ACT_SILU 0
#define REF_ACT_GELU_TANH 1
double ref_act(int act, double z) {
    if (act == REF_ACT_SILU) return z / (1.0 + exp(-z));
    const double c = sqrt(2.0 / acos(-1.0));
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

/* h = act(gate) * up, elementwise, in double. */
int ref_glu(const float* gate, const float* up, int act, int64_t n, double* h_out) {
    if (n < 0 || (n > 0 && (!gate || !up || !h_out))) return REF_ERR_ARG;
    if (act != REF_ACT_SILU && act != REF_ACT_GELU_TANH) return REF_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) h_out[i] = ref_act(act, (double)gate[i]) * (double)up[i];
    return REF_OK;
}

/* The down projection's input steps on the glue product: per row,
 * h = act(gate) * up, then RMSNorm with the down norm weight and the
 * absmax int8 quantization above, all in double. */
int ref_glu_quant(const float* gate, const float* up, int act, const float* norm_w, int64_t M,
                  int64_t K, float eps, int8_t* q_out, double* factor_out) {
    if ((M > 0 && (!gate || !up || !q_out || !factor_out)) || M < 0 || K <= 0)
        return REF_ERR_ARG;
    double* row = (double*)malloc((size_t)K * sizeof(double));
    if (!row) return REF_ERR_NOMEM;
    int rc = REF_OK;
    for (int64_t m = 0; m < M && rc == REF_OK; ++m) {
        rc = ref_glu(gate + m * K, up + m * K, act, K, row);
        if (rc == REF_OK) quant_row(row, norm_w, K, eps, q_out + m * K, factor_out + m);
    }
    free(row);
    return rc;
}

/* Integer product of the int8 activations with the ternary weights decoded
 * straight from the packed bytes: acc[m][n] = sum_k q[m][k] * (code[n][k] - 1),
 * accumulated in 64-bit and required to fit int32. */
int ref_matmul_i32(const int8_t* xq, const uint8_t* packed, int64_t M, int64_t K, int64_t N,
                   int32_t* acc_out) {
    if (M < 0 || K <= 0 || N <= 0 || K % BLOCK != 0) return REF_ERR_ARG;
    if (M > 0 && (!xq || !packed || !acc_out)) return REF_ERR_ARG;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t byte;
                int shift;
                ref_locate(K, n, k, &byte, &shift);
                int code = (packed[byte] >> shift) & 3;
                if (code == 3) return REF_ERR_CODE3;
                s += (int64_t)xq[m * K + k] * (int64_t)(code - 1);
            }
            if (s > INT32_MAX || s < INT32_MIN) return REF_ERR_OVERFLOW;
            acc_out[m * N + n] = (int32_t)s;
        }
    }
    return REF_OK;
}

/* Scale-only epilogue ([INF "Architectural Details"]: no bias):
 * y = acc * factor_m / scale, in double, rounded once to f32. */
void ref_epilogue(const int32_t* acc, const double* factor, float scale, int64_t M, int64_t N,
                  float* y) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (float)((double)acc[m * N + n] * factor[m] / (double)scale);
}

/* The whole path for M rows: quantize, integer product, epilogue.  The scale
 * is the one stored at the end of the packed buffer. */
int ref_bitlinear(const float* x, const float* norm_w, const uint8_t* packed, int64_t M, int64_t K,
                  int64_t N, float eps, float* y) {
    if (M < 0 || K <= 0 || N <= 0 || K % BLOCK != 0) return REF_ERR_ARG;
    if (M == 0) return REF_OK;
    int8_t* q = (int8_t*)malloc((size_t)(M * K));
    double* factor = (double*)malloc((size_t)M * sizeof(double));
    int32_t* acc = (int32_t*)malloc((size_t)(M * N) * sizeof(int32_t));
    int rc = REF_ERR_NOMEM;
    if (q && factor && acc) {
        rc = ref_quant(x, norm_w, M, K, eps, q, factor);
        if (rc == REF_OK) rc = ref_matmul_i32(q, packed, M, K, N, acc);
        if (rc == REF_OK) {
            float scale;
            memcpy(&scale, packed + N * K / 4, 4);
            ref_epilogue(acc, factor, scale, M, N, y);
        }
    }
    free(q);
    free(factor);
    free(acc);
    return rc;
}

/* The down projection fed by the glue: glue + quantization, integer
 * product, epilogue. */
int ref_glu_bitlinear(const float* gate, const float* up, int act, const float* norm_w,
                      const uint8_t* packed, int64_t M, int64_t K, int64_t N, float eps, float* y) {
    if (M < 0 || K <= 0 || N <= 0 || K % BLOCK != 0) return REF_ERR_ARG;
    if (M == 0) return REF_OK;
    int8_t* q = (int8_t*)malloc((size_t)(M * K));
    double* factor = (double*)malloc((size_t)M * sizeof(double));
    int32_t* acc = (int32_t*)malloc((size_t)(M * N) * sizeof(int32_t));
    int rc = REF_ERR_NOMEM;
    if (q && factor && acc) {
        rc = ref_glu_quant(gate, up, act, norm_w, M, K, eps, q, factor);
        if (rc == REF_OK) rc = ref_matmul_i32(q, packed, M, K, N, acc);
        if (rc == REF_OK) {
            float scale;
            memcpy(&scale, packed + N * K / 4, 4);
            ref_epilogue(acc, factor, scale, M, N, y);
        }
    }
    free(q);
    free(factor);
    free(acc);
    return rc;
}
