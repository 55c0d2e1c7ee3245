/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the fused
 * fp16 GEMM + elementwise epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code, header,
 * table or constant with the HIP library under dense_gemm_elementwise_amd/;
 * the epilogue kind numbers below are the public enum values of the boundary,
 * written out again here on purpose.
 *
 * What it computes (all citations are to the three pages the method comes
 * from):
 *   - acc[l][i][j] = sum_k A[l][i][k] * B[l][k][j], the batched product that
 *     the CUTLASS Operator API tutorial "Custom epilogue fusions for GEMMs"
 *     builds in cell [2] (A is (L,M,K), B is (L,K,N), C is (L,M,N), fp16,
 *     accumulator type fp32 in cell [4]).
 *   - the epilogue functions of the accumulator that the pages define:
 *       LINCOMB       D = alpha*acc + beta*C
 *                     (CUTLASS Python examples article, "Basic GEMM" NumPy
 *                     check, and "Epilogue" default identity activation)
 *       AUX_SCALE     Aux = alpha*acc + beta*C ; D = s*Aux
 *                     (tutorial cell [2], my_epilogue)
 *       LINCOMB_X_ACC Y = acc ; D = alpha*acc + beta*C + s*X
 *                     (Custom Epilogue Example, "Basic Example: Alpha-Beta
 *                     Scaling", epilogue_operation)
 *       RELU          D = ReLU(alpha*acc + beta*C)
 *                     (Custom Epilogue Example, "Activation Functions")
 *       SQUARE        D = alpha*acc + beta*C ; E = D*D
 *                     (Custom Epilogue Example, "Multiple Outputs"; the page
 *                     form is alpha = beta = 1)
 *       RELU_SQUARE   D = ReLU(alpha*acc + beta*C) ; E = D*D
 *                     ("Activation Functions" followed by "Multiple Outputs")
 *       RELU_AUX_STORE F = alpha*acc + beta*C ; D = ReLU(F)
 *                     (tutorial cell [6], relu_aux_store, whose beta is the
 *                     constant 2.0; cell [8] is the same with alpha = 1,
 *                     beta = 0.5)
 *       RELU_SCALE_ACC F = ReLU(alpha*acc + beta*C) ; D = s*F ; and the
 *                     accumulator itself as an fp32 output
 *                     (tutorial cell [7], relu_scale_return_acc)
 *       BIAS_ROW_COL  D = (alpha*acc + row_bias[j]) + col_bias[i]
 *                     (tutorial cell [9], broadcast_epilogue: row_bias has
 *                     shape (N,), col_bias (M, 1); C is not read)
 *       SIGMOID, TANH, GELU, SILU, LEAKY_RELU, HARDSWISH
 *                     D = act(alpha*acc + beta*C) with the activations the
 *                     Python examples article's "Epilogue" section lists as
 *                     built in (besides identity = LINCOMB and relu = RELU;
 *                     the Custom Epilogue Example's "Supported Operations"
 *                     names the same family).  The pages give no formulas;
 *                     the standard definitions are used:
 *                       sigmoid(t)    = 1 / (1 + e^-t)
 *                       tanh(t)       = the hyperbolic tangent (C library)
 *                       gelu(t)       = t * Phi(t), Phi the standard normal
 *                                       distribution function, written
 *                                       0.5 * t * erfc(-t / sqrt 2) (Hendrycks
 *                                       and Gimpel's exact form, not the tanh
 *                                       approximation)
 *                       silu(t)       = t * sigmoid(t)
 *                       leaky_relu(t) = t > 0 ? t : s * t, the slope s given
 *                                       as the third scalar
 *                       hardswish(t)  = t * min(max(t + 3, 0), 6) / 6
 *                                       (Howard et al., MobileNetV3)
 *     The second output (Aux, Y, E or F) goes to the Aux buffer; the biases
 *     are shared by every batch entry.
 *
 * Precision (readings where the pages are silent):
 *   - fp16 inputs are decoded exactly to double by oracle_f16_decode() below;
 *     the same definition runs on bfloat16 tensors (the Custom Epilogue
 *     Example's "Data Type Support": BF16 inputs and outputs) through
 *     oracle_gemm_epi_typed(), with oracle_bf16_decode() and
 *     oracle_bf16_encode() in place of the fp16 codec;
 *   - every sum runs in double, k strictly increasing, starting from +0.0
 *     (the textbook i-k-j triple loop; the loop order does not change the
 *     order in which any one element is summed);
 *   - the epilogue runs in double from the unrounded acc (Aux, D feed the next
 *     operation unrounded, as the epilogue DAG's SSA values do);
 *   - every output is rounded once, double -> fp16, round to nearest, ties to
 *     even, overflow to +-inf (oracle_f16_encode() below; oracle_bf16_encode()
 *     for bfloat16); the fp32 accumulator
 *     output is the exact sum rounded once to fp32 (nearest, ties to even);
 *   - ReLU(t) = t > 0 ? t : +0.0 (the "where(d > 0, d, 0)" form);
 *   - gelu(t) and silu(t) for t > 0 where the double factor rounds to 1 are
 *     rounded to odd below t (below_to_odd()), so that their one rounding to
 *     the output format is the exact value's.
 * Build with -ffp-contract=off so that no multiply-add is fused.
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_LINCOMB 0
#define ORACLE_AUX_SCALE 1
#define ORACLE_LINCOMB_X_ACC 2
#define ORACLE_RELU 3
#define ORACLE_SQUARE 4
#define ORACLE_RELU_SQUARE 5
#define ORACLE_RELU_AUX_STORE 6
#define ORACLE_RELU_SCALE_ACC 7
#define ORACLE_BIAS_ROW_COL 8
#define ORACLE_SIGMOID 9
#define ORACLE_TANH 10
#define ORACLE_GELU 11
#define ORACLE_SILU 12
#define ORACLE_LEAKY_RELU 13
#define ORACLE_HARDSWISH 14

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 holds zero and the subnormals f * 2^-24; exponent 31 holds
 * inf (f == 0) and NaN. */
double oracle_f16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* double -> binary16, round to nearest, ties to even, in one step (no
 * intermediate fp32, so no double rounding). */
uint16_t oracle_f16_encode(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00);
    double a = fabs(x);
    if (a >= 65520.0) /* 65520 is the midpoint between 65504 and 2^16 */
        return (uint16_t)(sign | 0x7C00);
    if (a < 0x1p-14) {
        /* subnormal (or zero): the quantum is 2^-24; a * 2^24 is exact.
         * A result of 1024 is the smallest normal, 0x0400, as it should be. */
        double q = nearbyint(a * 0x1p24);
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e2;
    double m = frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    double q = nearbyint(ldexp(m, 11)); /* 11 significant bits, in [1024, 2048] */
    int E = e2 - 1 + 15;               /* biased exponent of a */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E >= 31)
        return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)(E << 10) | (uint16_t)((int)q - 1024));
}

/* bfloat16 (brain floating point; the upper half of an IEEE 754 binary32):
 * 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.  Exponent 0 holds
 * zero and the subnormals f * 2^-133; exponent 255 holds inf (f == 0) and
 * NaN. */
double oracle_bf16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 255;
    int f = h & 127;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);
    return sign ? -v : v;
}

/* double -> bfloat16, round to nearest, ties to even, in one step. */
uint16_t oracle_bf16_encode(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0);
    double a = fabs(x);
    /* (2 - 2^-8) * 2^127 is the midpoint between the largest finite value,
     * (2 - 2^-7) * 2^127, and 2^128; the tie goes to the even neighbour, inf */
    if (a >= ldexp(2.0 - 0x1p-8, 127))
        return (uint16_t)(sign | 0x7F80);
    if (a < 0x1p-126) {
        /* subnormal (or zero): the quantum is 2^-133; a * 2^133 is exact.  A
         * result of 128 is the smallest normal, 0x0080. */
        double q = nearbyint(a * 0x1p133);
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e2;
    double m = frexp(a, &e2);         /* a = m * 2^e2, m in [0.5, 1) */
    double q = nearbyint(ldexp(m, 8)); /* 8 significant bits, in [128, 256] */
    int E = e2 - 1 + 127;             /* biased exponent of a */
    if (q == 256.0) {
        q = 128.0;
        E += 1;
    }
    if (E >= 255)
        return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | (uint16_t)(E << 7) | (uint16_t)((int)q - 128));
}

/* Element types of the 16-bit tensors (A, B, C, X, the biases, D, Aux): the
 * boundary's public enum values, written out again here. */
#define ORACLE_DTYPE_F16 0
#define ORACLE_DTYPE_BF16 1
typedef double (*decode_fn)(uint16_t);
typedef uint16_t (*encode_fn)(double);

int oracle_kind_valid(int kind) { return kind >= ORACLE_LINCOMB && kind <= ORACLE_HARDSWISH; }
int oracle_kind_has_aux(int kind)
{
    return kind == ORACLE_AUX_SCALE || kind == ORACLE_LINCOMB_X_ACC || kind == ORACLE_SQUARE ||
           kind == ORACLE_RELU_SQUARE || kind == ORACLE_RELU_AUX_STORE || kind == ORACLE_RELU_SCALE_ACC;
}
int oracle_kind_reads_x(int kind) { return kind == ORACLE_LINCOMB_X_ACC; }
int oracle_kind_reads_c(int kind) { return kind != ORACLE_BIAS_ROW_COL; }
int oracle_kind_reads_bias(int kind) { return kind == ORACLE_BIAS_ROW_COL; }
int oracle_kind_has_acc_out(int kind) { return kind == ORACLE_RELU_SCALE_ACC; }

static double relu(double t) { return t > 0.0 ? t : 0.0; }
static double sigmoid(double t) { return 1.0 / (1.0 + exp(-t)); }
/* gelu(t) and silu(t) are t times a factor below 1.  Far right that factor
 * rounds to 1 in double and the product comes out as t itself, while the
 * exact value lies below t by less than one double ulp.  Rounding t to the
 * output format would then settle a tie that the exact value does not have,
 * where t is a rounding midpoint of that format.  Rounded to odd instead
 * (t if its last bit is odd, else the next double below it), the value stays
 * on the exact value's side of every rounding boundary of fp16, bfloat16 and
 * fp32 (all far coarser than double), so the one final rounding is still the
 * exact value's. */
static double below_to_odd(double t, double r)
{
    if (!(t > 0.0) || r != t || isinf(t)) return r;
    uint64_t b;
    memcpy(&b, &t, sizeof b);
    b -= ~b & 1u;
    memcpy(&r, &b, sizeof r);
    return r;
}
static double gelu(double t) { return below_to_odd(t, 0.5 * t * erfc(-t / sqrt(2.0))); }
static double silu(double t) { return below_to_odd(t, t * sigmoid(t)); }
static double leaky_relu(double t, double slope) { return t > 0.0 ? t : slope * t; }
static double hardswish(double t) { return t * fmin(fmax(t + 3.0, 0.0), 6.0) / 6.0; }

/* The epilogue of one element, in double, from the unrounded accumulator.
 * rb / cb are the row-broadcast bias of the element's column and the
 * column-broadcast bias of its row.  Writes the unrounded first output to *d
 * and the unrounded second output (if the kind has one) to *aux. */
static void epilogue(int kind, double acc, double c, double x, double rb, double cb, double alpha, double beta,
                     double s, double *d, double *aux)
{
    double t;
    switch (kind) {
    case ORACLE_LINCOMB:
        *d = alpha * acc + beta * c;
        break;
    case ORACLE_AUX_SCALE:
        t = alpha * acc + beta * c;
        *aux = t;
        *d = s * t;
        break;
    case ORACLE_LINCOMB_X_ACC:
        *aux = acc;
        *d = (alpha * acc + beta * c) + s * x;
        break;
    case ORACLE_RELU:
        *d = relu(alpha * acc + beta * c);
        break;
    case ORACLE_SQUARE:
        t = alpha * acc + beta * c;
        *d = t;
        *aux = t * t;
        break;
    case ORACLE_RELU_SQUARE:
        t = relu(alpha * acc + beta * c);
        *d = t;
        *aux = t * t;
        break;
    case ORACLE_RELU_AUX_STORE:
        t = alpha * acc + beta * c;
        *aux = t;
        *d = relu(t);
        break;
    case ORACLE_RELU_SCALE_ACC:
        t = relu(alpha * acc + beta * c);
        *aux = t;
        *d = s * t;
        break;
    case ORACLE_BIAS_ROW_COL:
        *d = (alpha * acc + rb) + cb;
        break;
    case ORACLE_SIGMOID:
        *d = sigmoid(alpha * acc + beta * c);
        break;
    case ORACLE_TANH:
        *d = tanh(alpha * acc + beta * c);
        break;
    case ORACLE_GELU:
        *d = gelu(alpha * acc + beta * c);
        break;
    case ORACLE_SILU:
        *d = silu(alpha * acc + beta * c);
        break;
    case ORACLE_LEAKY_RELU:
        *d = leaky_relu(alpha * acc + beta * c, s);
        break;
    case ORACLE_HARDSWISH:
        *d = hardswish(alpha * acc + beta * c);
        break;
    }
}

/* Checks shared by the entry points.  Returns 0 when the call is valid. */
static int check_args(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                      const uint16_t *C, const uint16_t *X, const uint16_t *RB, const uint16_t *CB,
                      const float *scalars, int kind, uint16_t *D, uint16_t *Aux, float *Acc)
{
    if (L < 1 || M < 1 || N < 1 || K < 1)
        return 1;
    if (!A || !B || !scalars)
        return 2;
    if (!oracle_kind_valid(kind))
        return 4;
    if ((oracle_kind_reads_c(kind) && !C) || (oracle_kind_reads_x(kind) && !X) ||
        (oracle_kind_reads_bias(kind) && (!RB || !CB)))
        return 2;
    if (!D || (oracle_kind_has_aux(kind) && !Aux) || (oracle_kind_has_acc_out(kind) && !Acc))
        return 3;
    return 0;
}

/*
 * Full product.  Host arrays, packed row-major:
 *   A[l][i][k] at (l*M + i)*K + k, B[l][k][j] at (l*K + k)*N + j,
 *   C, X, D, Aux, Acc [l][i][j] at (l*M + i)*N + j,
 *   RB[j] (N entries), CB[i] (M entries), shared by every batch entry.
 * scalars = {alpha, beta, s} with s = extra_scalar (AUX_SCALE), x_factor
 * (LINCOMB_X_ACC), scale (RELU_SCALE_ACC) or the negative slope (LEAKY_RELU);
 * unused otherwise.  Inputs a kind
 * does not read and outputs it does not write may be NULL.  D64 / Aux64 /
 * Acc64, when not NULL, receive the unrounded double outputs (Acc64: the
 * exact accumulator, for every kind).  Returns 0, or a nonzero code for
 * invalid arguments.  OpenMP splits the rows; each element's sum is the same
 * whatever the thread count.
 */
int oracle_gemm_epi_typed2(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                           const uint16_t *C, const uint16_t *X, const uint16_t *RB, const uint16_t *CB,
                           const float *scalars, int kind, uint16_t *D, uint16_t *Aux, float *Acc, double *D64,
                           double *Aux64, double *Acc64, int ab_dtype, int cd_dtype);

int oracle_gemm_epi_typed(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                          const uint16_t *C, const uint16_t *X, const uint16_t *RB, const uint16_t *CB,
                          const float *scalars, int kind, uint16_t *D, uint16_t *Aux, float *Acc, double *D64,
                          double *Aux64, double *Acc64, int dtype)
{
    return oracle_gemm_epi_typed2(L, M, N, K, A, B, C, X, RB, CB, scalars, kind, D, Aux, Acc, D64, Aux64, Acc64,
                                  dtype, dtype);
}

/*
 * The same with separate 16-bit element types for A, B (ab_dtype) and for
 * C, X, RB, CB, D, Aux (cd_dtype): the Custom Epilogue Example's "Data Type
 * Support" lists FP16 and BF16 among both the input types and the output
 * types.  Each tensor is decoded with its own type's decoder and each output
 * encoded once with the epilogue type's encoder; nothing else changes.
 */
int oracle_gemm_epi_typed2(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                           const uint16_t *C, const uint16_t *X, const uint16_t *RB, const uint16_t *CB,
                           const float *scalars, int kind, uint16_t *D, uint16_t *Aux, float *Acc, double *D64,
                           double *Aux64, double *Acc64, int ab_dtype, int cd_dtype)
{
    int rc = check_args(L, M, N, K, A, B, C, X, RB, CB, scalars, kind, D, Aux, Acc);
    if (rc)
        return rc;
    if ((ab_dtype != ORACLE_DTYPE_F16 && ab_dtype != ORACLE_DTYPE_BF16) ||
        (cd_dtype != ORACLE_DTYPE_F16 && cd_dtype != ORACLE_DTYPE_BF16))
        return 8;
    const decode_fn dec = ab_dtype == ORACLE_DTYPE_BF16 ? oracle_bf16_decode : oracle_f16_decode;
    const decode_fn dec_cd = cd_dtype == ORACLE_DTYPE_BF16 ? oracle_bf16_decode : oracle_f16_decode;
    const encode_fn enc = cd_dtype == ORACLE_DTYPE_BF16 ? oracle_bf16_encode : oracle_f16_encode;
    const double alpha = scalars[0], beta = scalars[1], s = scalars[2];
    double *Bd = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
    if (!Bd)
        return 7;
    for (int64_t l = 0; l < L; l++) {
        const uint16_t *Al = A + l * M * K;
        const uint16_t *Bl = B + l * K * N;
        for (int64_t q = 0; q < K * N; q++)
            Bd[q] = dec(Bl[q]);
        int fail = 0;
#pragma omp parallel
        {
            double *acc = (double *)malloc(sizeof(double) * (size_t)N);
            if (!acc) {
#pragma omp atomic write
                fail = 1;
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < M; i++) {
                if (!acc)
                    continue;
                for (int64_t j = 0; j < N; j++)
                    acc[j] = 0.0;
                for (int64_t k = 0; k < K; k++) {
                    const double a = dec(Al[i * K + k]);
                    const double *brow = Bd + k * N;
                    for (int64_t j = 0; j < N; j++)
                        acc[j] = acc[j] + a * brow[j];
                }
                const int64_t row = (l * M + i) * N;
                const double cb = oracle_kind_reads_bias(kind) ? dec_cd(CB[i]) : 0.0;
                for (int64_t j = 0; j < N; j++) {
                    double c = oracle_kind_reads_c(kind) ? dec_cd(C[row + j]) : 0.0;
                    double x = oracle_kind_reads_x(kind) ? dec_cd(X[row + j]) : 0.0;
                    double rb = oracle_kind_reads_bias(kind) ? dec_cd(RB[j]) : 0.0;
                    double d = 0.0, aux = 0.0;
                    epilogue(kind, acc[j], c, x, rb, cb, alpha, beta, s, &d, &aux);
                    D[row + j] = enc(d);
                    if (D64)
                        D64[row + j] = d;
                    if (oracle_kind_has_aux(kind)) {
                        Aux[row + j] = enc(aux);
                        if (Aux64)
                            Aux64[row + j] = aux;
                    }
                    if (oracle_kind_has_acc_out(kind))
                        Acc[row + j] = (float)acc[j]; /* one rounding, nearest-even */
                    if (Acc64)
                        Acc64[row + j] = acc[j];
                }
            }
            free(acc);
        }
        if (fail) {
            free(Bd);
            return 7;
        }
    }
    free(Bd);
    return 0;
}

/*
 * fp32 epilogue tensors (the Custom Epilogue Example's "Data Type Support"
 * lists FP32 among the C and D types, with FP16 or BF16 A and B and an FP32
 * accumulator).  A and B are 16-bit of type ab_dtype (ORACLE_DTYPE_F16 or
 * ORACLE_DTYPE_BF16); C, X, RB, CB are IEEE binary32, widened exactly to
 * double; D and Aux are binary32, each rounded once from the unrounded double
 * (C's conversion from double to float rounds to nearest, ties to even, and
 * gives +-inf past the largest finite float).  Everything else as
 * oracle_gemm_epi_typed, whose product and epilogue this repeats.
 */
int oracle_gemm_epi_f32e(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                         const float *C, const float *X, const float *RB, const float *CB, const float *scalars,
                         int kind, float *D, float *Aux, float *Acc, double *D64, double *Aux64, double *Acc64,
                         int ab_dtype)
{
    if (L < 1 || M < 1 || N < 1 || K < 1)
        return 1;
    if (!A || !B || !scalars)
        return 2;
    if (!oracle_kind_valid(kind))
        return 4;
    if ((oracle_kind_reads_c(kind) && !C) || (oracle_kind_reads_x(kind) && !X) ||
        (oracle_kind_reads_bias(kind) && (!RB || !CB)))
        return 2;
    if (!D || (oracle_kind_has_aux(kind) && !Aux) || (oracle_kind_has_acc_out(kind) && !Acc))
        return 3;
    if (ab_dtype != ORACLE_DTYPE_F16 && ab_dtype != ORACLE_DTYPE_BF16)
        return 8;
    const decode_fn dec = ab_dtype == ORACLE_DTYPE_BF16 ? oracle_bf16_decode : oracle_f16_decode;
    const double alpha = scalars[0], beta = scalars[1], s = scalars[2];
    double *Bd = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
    if (!Bd)
        return 7;
    for (int64_t l = 0; l < L; l++) {
        const uint16_t *Al = A + l * M * K;
        const uint16_t *Bl = B + l * K * N;
        for (int64_t q = 0; q < K * N; q++)
            Bd[q] = dec(Bl[q]);
        int fail = 0;
#pragma omp parallel
        {
            double *acc = (double *)malloc(sizeof(double) * (size_t)N);
            if (!acc) {
#pragma omp atomic write
                fail = 1;
            }
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < M; i++) {
                if (!acc)
                    continue;
                for (int64_t j = 0; j < N; j++)
                    acc[j] = 0.0;
                for (int64_t k = 0; k < K; k++) {
                    const double a = dec(Al[i * K + k]);
                    const double *brow = Bd + k * N;
                    for (int64_t j = 0; j < N; j++)
                        acc[j] = acc[j] + a * brow[j];
                }
                const int64_t row = (l * M + i) * N;
                const double cb = oracle_kind_reads_bias(kind) ? (double)CB[i] : 0.0;
                for (int64_t j = 0; j < N; j++) {
                    double c = oracle_kind_reads_c(kind) ? (double)C[row + j] : 0.0;
                    double x = oracle_kind_reads_x(kind) ? (double)X[row + j] : 0.0;
                    double rb = oracle_kind_reads_bias(kind) ? (double)RB[j] : 0.0;
                    double d = 0.0, aux = 0.0;
                    epilogue(kind, acc[j], c, x, rb, cb, alpha, beta, s, &d, &aux);
                    D[row + j] = (float)d;
                    if (D64)
                        D64[row + j] = d;
                    if (oracle_kind_has_aux(kind)) {
                        Aux[row + j] = (float)aux;
                        if (Aux64)
                            Aux64[row + j] = aux;
                    }
                    if (oracle_kind_has_acc_out(kind))
                        Acc[row + j] = (float)acc[j];
                    if (Acc64)
                        Acc64[row + j] = acc[j];
                }
            }
            free(acc);
        }
        if (fail) {
            free(Bd);
            return 7;
        }
    }
    free(Bd);
    return 0;
}

/* fp16 tensors (the boundary's default element type). */
int oracle_gemm_epi_ext(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                        const uint16_t *C, const uint16_t *X, const uint16_t *RB, const uint16_t *CB,
                        const float *scalars, int kind, uint16_t *D, uint16_t *Aux, float *Acc, double *D64,
                        double *Aux64, double *Acc64)
{
    return oracle_gemm_epi_typed(L, M, N, K, A, B, C, X, RB, CB, scalars, kind, D, Aux, Acc, D64, Aux64, Acc64,
                                 ORACLE_DTYPE_F16);
}

/* The entry point without bias inputs or accumulator output (kinds 0-6). */
int oracle_gemm_epi(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                    const uint16_t *C, const uint16_t *X, const float *scalars, int kind, uint16_t *D,
                    uint16_t *Aux, double *D64, double *Aux64)
{
    return oracle_gemm_epi_ext(L, M, N, K, A, B, C, X, NULL, NULL, scalars, kind, D, Aux, NULL, D64, Aux64,
                               NULL);
}

/*
 * The same definition for a list of single output elements (l[p], i[p],
 * j[p]), each summed on its own over k in increasing order, so a full-size
 * problem can be checked at sampled points.  Outputs are indexed by p:
 * D[p], Aux[p], Acc[p], D64[p], Aux64[p], Acc64[p] (all but D may be NULL).
 */
int oracle_gemm_epi_points_typed(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A,
                                 const uint16_t *B, const uint16_t *C, const uint16_t *X, const uint16_t *RB,
                                 const uint16_t *CB, const float *scalars, int kind, int64_t npts,
                                 const int64_t *pl, const int64_t *pi, const int64_t *pj, uint16_t *D,
                                 uint16_t *Aux, float *Acc, double *D64, double *Aux64, double *Acc64, int dtype)
{
    /* the per-point outputs are optional: check the inputs with stand-ins */
    uint16_t dummy16 = 0;
    float dummy32 = 0.0f;
    int rc = check_args(L, M, N, K, A, B, C, X, RB, CB, scalars, kind, D, &dummy16, &dummy32);
    if (rc)
        return rc;
    if (npts < 0 || (npts > 0 && (!pl || !pi || !pj)))
        return 1;
    if (dtype != ORACLE_DTYPE_F16 && dtype != ORACLE_DTYPE_BF16)
        return 8;
    const decode_fn dec = dtype == ORACLE_DTYPE_BF16 ? oracle_bf16_decode : oracle_f16_decode;
    const encode_fn enc = dtype == ORACLE_DTYPE_BF16 ? oracle_bf16_encode : oracle_f16_encode;
    for (int64_t p = 0; p < npts; p++)
        if (pl[p] < 0 || pl[p] >= L || pi[p] < 0 || pi[p] >= M || pj[p] < 0 || pj[p] >= N)
            return 1;
    const double alpha = scalars[0], beta = scalars[1], s = scalars[2];
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; p++) {
        const int64_t l = pl[p], i = pi[p], j = pj[p];
        double acc = 0.0;
        for (int64_t k = 0; k < K; k++)
            acc = acc + dec(A[(l * M + i) * K + k]) * dec(B[(l * K + k) * N + j]);
        const int64_t o = (l * M + i) * N + j;
        double c = oracle_kind_reads_c(kind) ? dec(C[o]) : 0.0;
        double x = oracle_kind_reads_x(kind) ? dec(X[o]) : 0.0;
        double rb = oracle_kind_reads_bias(kind) ? dec(RB[j]) : 0.0;
        double cb = oracle_kind_reads_bias(kind) ? dec(CB[i]) : 0.0;
        double d = 0.0, aux = 0.0;
        epilogue(kind, acc, c, x, rb, cb, alpha, beta, s, &d, &aux);
        D[p] = enc(d);
        if (D64)
            D64[p] = d;
        if (oracle_kind_has_aux(kind)) {
            if (Aux)
                Aux[p] = enc(aux);
            if (Aux64)
                Aux64[p] = aux;
        }
        if (Acc && oracle_kind_has_acc_out(kind))
            Acc[p] = (float)acc;
        if (Acc64)
            Acc64[p] = acc;
    }
    return 0;
}

int oracle_gemm_epi_points_ext(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A,
                               const uint16_t *B, const uint16_t *C, const uint16_t *X, const uint16_t *RB,
                               const uint16_t *CB, const float *scalars, int kind, int64_t npts, const int64_t *pl,
                               const int64_t *pi, const int64_t *pj, uint16_t *D, uint16_t *Aux, float *Acc,
                               double *D64, double *Aux64, double *Acc64)
{
    return oracle_gemm_epi_points_typed(L, M, N, K, A, B, C, X, RB, CB, scalars, kind, npts, pl, pi, pj, D, Aux,
                                        Acc, D64, Aux64, Acc64, ORACLE_DTYPE_F16);
}

int oracle_gemm_epi_points(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                           const uint16_t *C, const uint16_t *X, const float *scalars, int kind, int64_t npts,
                           const int64_t *pl, const int64_t *pi, const int64_t *pj, uint16_t *D, uint16_t *Aux,
                           double *D64, double *Aux64)
{
    return oracle_gemm_epi_points_ext(L, M, N, K, A, B, C, X, NULL, NULL, scalars, kind, npts, pl, pi, pj, D,
                                      Aux, NULL, D64, Aux64, NULL);
}

/* Bulk codec helpers for the tests: decode n halves / encode n doubles. */
void oracle_f16_decode_n(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t q = 0; q < n; q++)
        out[q] = oracle_f16_decode(h[q]);
}

void oracle_f16_encode_n(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t q = 0; q < n; q++)
        out[q] = oracle_f16_encode(x[q]);
}

void oracle_bf16_decode_n(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t q = 0; q < n; q++)
        out[q] = oracle_bf16_decode(h[q]);
}

void oracle_bf16_encode_n(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t q = 0; q < n; q++)
        out[q] = oracle_bf16_encode(x[q]);
}

/* The rounding mode the encoder relies on (FE_TONEAREST); the tests check it. */
int oracle_rounding_mode_is_nearest(void) { return fegetround() == FE_TONEAREST; }
