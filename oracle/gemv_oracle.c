/*
 * CPU oracle for dense GEMV  y = A·x (+ bias)  and its small-batch form
 * Y = A·X (+ bias).  TEST INFRASTRUCTURE ONLY: the product library never
 * links, loads or calls this file; only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * helper with the HIP path.
 *
 * What it computes, and where that is defined:
 *   - y[m] is the dot product of row m of A with x: page "SGEMV CUDA代码学习",
 *     section "问题定义: 一行一个点积" (problem definition: one dot product per
 *     output row, A is M×K, x is K×1, y is M×1).
 *   - an optional per-row bias is added, and a missing (NULL) bias counts as
 *     zero: page "第 3 课：GEMV 与行级并行", section "核心心智模型" item 1
 *     (the y = A x + bias definition) and section "3. 正确性边界与指针安全性"
 *     (bias may be absent).
 *   - several right-hand vectors share one pass over A (the small-batch decode
 *     case): page "GEMM、GEMV、dtype 与算术强度", section "可运行 CUDA 实验"
 *     (the m = 16 small_batch_decode run), and page "第 3 课", section
 *     "4. 性能与工程权舍" (batch B below 16~32 is still GEMV territory).
 *   - reduced-precision inputs are accumulated in a wider type and checked
 *     against a higher-precision recomputation: page "GEMM、GEMV、dtype 与算术
 *     强度", sections "dtype 改变什么" and "可运行 CUDA 实验".
 *   - the gated pair h = silu(A_gate·x) ⊙ (A_up·x): the FFN of the lqnn.cn
 *     NPU MatMul essay, sections 1.1 (an up-projection, an activation, a
 *     down-projection) and 4.2 / 5.1 (fusing the FFN's MatMuls with the
 *     activation).  The essay names no activation; SiLU,
 *     silu(g) = g / (1 + e^(-g)), is the gated one of the decode shapes here
 *     (gate and up projections of equal shape).
 *   - weight-only int8: y[m] = scale[m] · Σ_k q[m,k]·x[k] (+ bias[m]), the
 *     weights stored as int8 with one fp32 scale per output row
 *     ("per-channel"), the activations still in a float encoding and the
 *     accumulation wide: the lqnn.cn NPU MatMul essay, sections 1.2
 *     (quantised MatMul: int8 weights, fp16 activations, fp32 accumulator),
 *     4.2 (int8 weights with a per-channel scale) and 5.2 (bytes halve,
 *     fp32 accumulation).  No zero point: the scale alone is the
 *     per-channel compensation the essay applies.
 *
 * The oracle is that definition written out: every stored element is decoded
 * exactly to double, products and the running sum are taken in double, in
 * increasing k, and the bias is added once after the sum.  A product of two
 * decoded fp32/fp16/bf16 values is exact in double (at most 24+24 significant
 * bits), so the only rounding is in the k-ordered double sum.
 *
 * Beside y it returns, per output, the sum over k of |A[m,k]·x[k]| (also in
 * double), which scales the tolerance a faster, differently ordered fp32
 * implementation is allowed.
 *
 * Layouts (element offsets, all 64-bit):
 *   A     row-major, element (m,k) at A[m*lda + k], lda >= K; elements
 *         k = K..lda-1 of a row are never read.
 *   X     column j at X[j*ldx + k], ldx >= K (nvec = 1 is plain GEMV).
 *   bias  bias[m], fp32, or NULL.
 *   Y     element (m,j) at Y[j*M + m], double; ABS has the same layout.
 *
 * Input element encodings (dtype codes):
 *   0  IEEE binary32 words
 *   1  IEEE binary16 bit patterns (uint16)
 *   2  bfloat16 bit patterns (uint16): the upper half of a binary32 word
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2

/* binary32 word -> double (exact). */
static double decode_f32_bits(uint32_t w) {
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* bfloat16 keeps the sign, the 8 exponent bits and the top 7 fraction bits of
 * a binary32 value, so its bits placed in the high half of a 32-bit word (low
 * half zero) are that binary32 value. */
static double decode_bf16_bits(uint16_t h) {
    return decode_f32_bits((uint32_t)h << 16);
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-24
 *   exponent 1..30  : normal, value = (1024 + fraction) * 2^(exponent - 25)
 *   exponent 31     : infinity (fraction 0) or NaN */
static double decode_f16_bits(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);
    } else if (expo == 31) {
        mag = frac == 0 ? INFINITY : NAN;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -mag : mag;
}

/* Element i of an array stored with the given encoding, as a double. */
static double load_elem(int dtype, const void *base, int64_t i) {
    if (dtype == ORACLE_F32) {
        uint32_t w;
        memcpy(&w, (const char *)base + 4 * i, sizeof w);
        return decode_f32_bits(w);
    }
    const uint16_t h = ((const uint16_t *)base)[i];
    return dtype == ORACLE_F16 ? decode_f16_bits(h) : decode_bf16_bits(h);
}

/* Returns 0 on success, -1 if the arguments cannot describe a valid problem. */
int oracle_gemv(int dtype, const void *A, int64_t lda, const void *X,
                int64_t ldx, const float *bias, int64_t M, int64_t K,
                int64_t nvec, double *Y, double *ABS) {
    if (dtype < ORACLE_F32 || dtype > ORACLE_BF16) return -1;
    if (M < 0 || K < 0 || nvec < 1 || lda < K || ldx < K) return -1;
    if (M > 0 && (Y == NULL || ABS == NULL)) return -1;
    if (M > 0 && K > 0 && (A == NULL || X == NULL)) return -1;

#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < nvec; ++j) {
            double sum = 0.0;
            double abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = load_elem(dtype, A, m * lda + k);
                const double x = load_elem(dtype, X, j * ldx + k);
                sum += a * x;
                abs_sum += fabs(a * x);
            }
            if (bias != NULL) sum += (double)bias[m];
            Y[j * M + m] = sum;
            ABS[j * M + m] = abs_sum;
        }
    }
    return 0;
}

/* A two's-complement byte as a double: bytes 0..127 are themselves, bytes
 * 128..255 are byte - 256. */
static double decode_i8(uint8_t b) {
    return b < 128 ? (double)b : (double)b - 256.0;
}

/* Y[j*M+m] = scale[m] · Σ_k q[m,k]·x_j[k] (+ bias[m]) and
 * ABS[j*M+m] = |scale[m]| · Σ_k |q[m,k]·x_j[k]|, in double: the sum over k
 * first, in k order, then the scale, then the bias.  Q is row-major int8
 * with row stride ldq (bytes K..ldq-1 of a row never read); x_j is column j
 * of X (stride ldx) in encoding xdtype; scale has M fp32 values.  Returns 0,
 * or -1 for bad arguments. */
int oracle_gemv_q8(int xdtype, const uint8_t *Q, int64_t ldq, const float *scale,
                   const void *X, int64_t ldx, const float *bias, int64_t M,
                   int64_t K, int64_t nvec, double *Y, double *ABS) {
    if (xdtype < ORACLE_F32 || xdtype > ORACLE_BF16) return -1;
    if (M < 0 || K < 0 || nvec < 1 || ldq < K || ldx < K) return -1;
    if (M > 0 && (Y == NULL || ABS == NULL || scale == NULL)) return -1;
    if (M > 0 && K > 0 && (Q == NULL || X == NULL)) return -1;

#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const double s = (double)scale[m];
        for (int64_t j = 0; j < nvec; ++j) {
            double sum = 0.0;
            double abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double q = decode_i8(Q[m * ldq + k]);
                const double x = load_elem(xdtype, X, j * ldx + k);
                sum += q * x;
                abs_sum += fabs(q * x);
            }
            double y = s * sum;
            if (bias != NULL) y += (double)bias[m];
            Y[j * M + m] = y;
            ABS[j * M + m] = fabs(s) * abs_sum;
        }
    }
    return 0;
}

/* h[m] = silu(g[m]) * u[m] with g = A_gate·x and u = A_up·x (both M×K with
 * row stride lda, same encoding), in double; G, U, ABS_G, ABS_U receive g, u
 * and the sums of |A·x| of each product.  Returns 0, or -1 for bad arguments. */
int oracle_gated_silu(int dtype, const void *Ag, const void *Au, int64_t lda,
                      const void *X, int64_t M, int64_t K, double *H, double *G,
                      double *U, double *ABS_G, double *ABS_U) {
    if (oracle_gemv(dtype, Ag, lda, X, K, NULL, M, K, 1, G, ABS_G) != 0) return -1;
    if (oracle_gemv(dtype, Au, lda, X, K, NULL, M, K, 1, U, ABS_U) != 0) return -1;
    for (int64_t m = 0; m < M; ++m) {
        const double g = G[m];
        H[m] = g / (1.0 + exp(-g)) * U[m];
    }
    return 0;
}

/* Number of threads the parallel loop above runs on (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
