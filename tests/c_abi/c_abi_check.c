/*
 * c_abi_check.c -- the C ABI of libgemm_epi.so used from plain C (no Python,
 * no torch): device buffers from the HIP runtime, one call per case (the
 * typed, mixed and workspace entry points), results compared bit for bit
 * with the CPU oracle (liboracle.so, test infrastructure).
 *
 * Inputs are small integers drawn by a seeded linear congruential
 * generator, so every product and partial sum is exact and the final
 * rounding is the only one on either side: the outputs must be
 * bit-identical (+0 and -0 compare equal).  Exit status 0 when every case
 * passes.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gemm_epi.h"

/* the oracle's typed entry points (oracle/oracle.c) */
int oracle_gemm_epi_typed2(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                           const uint16_t *C, const uint16_t *X, const uint16_t *RB, const uint16_t *CB,
                           const float *scalars, int kind, uint16_t *D, uint16_t *Aux, float *Acc, double *D64,
                           double *Aux64, double *Acc64, int ab_dtype, int cd_dtype);
int oracle_gemm_epi_f32e(int64_t L, int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                         const float *C, const float *X, const float *RB, const float *CB, const float *scalars,
                         int kind, float *D, float *Aux, float *Acc, double *D64, double *Aux64, double *Acc64,
                         int ab_dtype);

#define CHECK_HIP(x)                                                                        \
    do {                                                                                    \
        hipError_t e_ = (x);                                                                \
        if (e_ != hipSuccess) {                                                             \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_));      \
            exit(2);                                                                        \
        }                                                                                   \
    } while (0)

/* bit patterns of the integers -3..3 in binary16 and in bfloat16 */
static const uint16_t kF16[7] = {0xC200, 0xC000, 0xBC00, 0x0000, 0x3C00, 0x4000, 0x4200};
static const uint16_t kBF16[7] = {0xC040, 0xC000, 0xBF80, 0x0000, 0x3F80, 0x4000, 0x4040};

static uint64_t lcg_state;
static int next_int(void) /* uniform in -3..3 */
{
    lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (int)((lcg_state >> 33) % 7) - 3;
}

static uint16_t *draw(size_t n, int dtype)
{
    uint16_t *h = (uint16_t *)malloc(n * 2);
    for (size_t i = 0; i < n; i++) h[i] = (dtype == GEMM_EPI_BF16 ? kBF16 : kF16)[next_int() + 3];
    return h;
}

static void *upload_bytes(const void *h, size_t bytes)
{
    void *d = NULL;
    if (!h) return NULL;
    CHECK_HIP(hipMalloc(&d, bytes));
    CHECK_HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}

static void *upload(const uint16_t *h, size_t n) { return upload_bytes(h, n * 2); }

static float *draw_f32(size_t n) /* the same small integers, as fp32 */
{
    float *h = (float *)malloc(n * 4);
    for (size_t i = 0; i < n; i++) h[i] = (float)next_int();
    return h;
}

static const char *type_name(int dtype)
{
    return dtype == GEMM_EPI_BF16 ? "bf16" : dtype == GEMM_EPI_F32 ? "f32" : "f16";
}

static int same_bits(const uint16_t *g, const uint16_t *w, size_t n, const char *what)
{
    size_t bad = 0;
    for (size_t i = 0; i < n; i++)
        if (g[i] != w[i] && ((g[i] | w[i]) & 0x7FFF) != 0) bad++;
    if (bad) fprintf(stderr, "  %s: %zu of %zu outputs differ\n", what, bad, n);
    return bad == 0;
}

/* A, B of type dtype; C, X, D, Aux of the 16-bit type epi (gemm_epi_run_mixed).  With staged != 0 (epi ==
 * dtype, a shape off the fast path's 16-byte rule) the call is gemm_epi_run_ws_typed with the workspace
 * gemm_epi_plan_ws reports, which must stage the operands for the fast kernel. */
static int run_case(int kind, int dtype, int epi, int64_t L, int64_t M, int64_t N, int64_t K, const float sc[3],
                    int staged)
{
    const int has_aux = kind == GEMM_EPI_AUX_SCALE || kind == GEMM_EPI_LINCOMB_X_ACC || kind == GEMM_EPI_SQUARE ||
                        kind == GEMM_EPI_RELU_SQUARE || kind == GEMM_EPI_RELU_AUX_STORE;
    const int reads_x = kind == GEMM_EPI_LINCOMB_X_ACC;
    const size_t na = (size_t)(L * M * K), nb = (size_t)(L * K * N), nc = (size_t)(L * M * N);
    lcg_state = 0x9E3779B97F4A7C15ULL ^ (uint64_t)(kind * 131 + dtype * 7 + M);
    uint16_t *A = draw(na, dtype), *B = draw(nb, dtype), *C = draw(nc, epi);
    uint16_t *X = reads_x ? draw(nc, epi) : NULL;
    void *dA = upload(A, na), *dB = upload(B, nb), *dC = upload(C, nc), *dX = upload(X, nc);
    void *dD = NULL, *dAux = NULL;
    CHECK_HIP(hipMalloc(&dD, nc * 2));
    if (has_aux) CHECK_HIP(hipMalloc(&dAux, nc * 2));

    int ok = 1, rc;
    void *ws = NULL;
    if (staged) {
        int64_t plan[7];
        rc = gemm_epi_plan_ws(L, M, N, K, dA, dB, dC, dX, NULL, NULL, kind, dD, dAux, NULL, plan);
        if (rc == GEMM_EPI_OK && !(plan[3] == 1 && plan[6] > 16384)) {
            fprintf(stderr, "  no staging planned (vec %lld, workspace %lld)\n", (long long)plan[3], (long long)plan[6]);
            ok = 0;
        }
        if (rc == GEMM_EPI_OK) {
            CHECK_HIP(hipMalloc(&ws, (size_t)plan[6]));
            CHECK_HIP(hipMemset(ws, 0, (size_t)plan[6]));
            rc = gemm_epi_run_ws_typed(L, M, N, K, dA, dB, dC, dX, NULL, NULL, sc, kind, dD, dAux, NULL, ws,
                                       (size_t)plan[6], dtype, NULL);
        }
    } else {
        rc = epi == dtype
                 ? gemm_epi_run_typed(L, M, N, K, dA, dB, dC, dX, NULL, NULL, sc, kind, dD, dAux, NULL, dtype, NULL)
                 : gemm_epi_run_mixed(L, M, N, K, dA, dB, dC, dX, NULL, NULL, sc, kind, dD, dAux, NULL, dtype, epi, NULL);
    }
    if (rc != GEMM_EPI_OK) {
        fprintf(stderr, "  the call returned %d (%s)\n", rc, gemm_epi_status_string(rc));
        ok = 0;
    } else {
        CHECK_HIP(hipDeviceSynchronize());
        uint16_t *D = (uint16_t *)malloc(nc * 2), *Aux = has_aux ? (uint16_t *)malloc(nc * 2) : NULL;
        uint16_t *Dref = (uint16_t *)malloc(nc * 2), *Auxref = has_aux ? (uint16_t *)malloc(nc * 2) : NULL;
        CHECK_HIP(hipMemcpy(D, dD, nc * 2, hipMemcpyDeviceToHost));
        if (has_aux) CHECK_HIP(hipMemcpy(Aux, dAux, nc * 2, hipMemcpyDeviceToHost));
        const int orc = oracle_gemm_epi_typed2(L, M, N, K, A, B, C, X, NULL, NULL, sc, kind, Dref, Auxref, NULL, NULL,
                                               NULL, NULL, dtype, epi);
        if (orc != 0) {
            fprintf(stderr, "  the oracle rejected the case (%d)\n", orc);
            ok = 0;
        } else {
            ok = same_bits(D, Dref, nc, "D") && (!has_aux || same_bits(Aux, Auxref, nc, "Aux"));
        }
        free(D);
        free(Aux);
        free(Dref);
        free(Auxref);
    }
    printf("%s kind=%d dtype=%s epi=%s L=%lld M=%lld N=%lld K=%lld%s\n", ok ? "PASS" : "FAIL", kind,
           type_name(dtype), type_name(epi), (long long)L, (long long)M, (long long)N, (long long)K,
           staged ? " staged" : "");
    fflush(stdout);
    hipFree(ws);
    hipFree(dA);
    hipFree(dB);
    hipFree(dC);
    hipFree(dX);
    hipFree(dD);
    hipFree(dAux);
    free(A);
    free(B);
    free(C);
    free(X);
    return ok;
}

/* A, B of type dtype; C, X, D, Aux fp32 (gemm_epi_run_mixed with GEMM_EPI_F32) */
static int run_case_f32(int kind, int dtype, int64_t L, int64_t M, int64_t N, int64_t K, const float sc[3])
{
    const int has_aux = kind == GEMM_EPI_AUX_SCALE || kind == GEMM_EPI_LINCOMB_X_ACC || kind == GEMM_EPI_SQUARE ||
                        kind == GEMM_EPI_RELU_SQUARE || kind == GEMM_EPI_RELU_AUX_STORE;
    const int reads_x = kind == GEMM_EPI_LINCOMB_X_ACC;
    const size_t na = (size_t)(L * M * K), nb = (size_t)(L * K * N), nc = (size_t)(L * M * N);
    lcg_state = 0x243F6A8885A308D3ULL ^ (uint64_t)(kind * 131 + dtype * 7 + M);
    uint16_t *A = draw(na, dtype), *B = draw(nb, dtype);
    float *C = draw_f32(nc), *X = reads_x ? draw_f32(nc) : NULL;
    void *dA = upload(A, na), *dB = upload(B, nb), *dC = upload_bytes(C, nc * 4);
    void *dX = X ? upload_bytes(X, nc * 4) : NULL;
    void *dD = NULL, *dAux = NULL;
    CHECK_HIP(hipMalloc(&dD, nc * 4));
    if (has_aux) CHECK_HIP(hipMalloc(&dAux, nc * 4));
    int ok = 1;
    const int rc = gemm_epi_run_mixed(L, M, N, K, dA, dB, dC, dX, NULL, NULL, sc, kind, dD, dAux, NULL, dtype,
                                      GEMM_EPI_F32, NULL);
    if (rc != GEMM_EPI_OK) {
        fprintf(stderr, "  gemm_epi_run_mixed returned %d (%s)\n", rc, gemm_epi_status_string(rc));
        ok = 0;
    } else {
        CHECK_HIP(hipDeviceSynchronize());
        float *D = (float *)malloc(nc * 4), *Aux = has_aux ? (float *)malloc(nc * 4) : NULL;
        float *Dref = (float *)malloc(nc * 4), *Auxref = has_aux ? (float *)malloc(nc * 4) : NULL;
        CHECK_HIP(hipMemcpy(D, dD, nc * 4, hipMemcpyDeviceToHost));
        if (has_aux) CHECK_HIP(hipMemcpy(Aux, dAux, nc * 4, hipMemcpyDeviceToHost));
        if (oracle_gemm_epi_f32e(L, M, N, K, A, B, C, X, NULL, NULL, sc, kind, Dref, Auxref, NULL, NULL, NULL, NULL,
                                 dtype) != 0) {
            fprintf(stderr, "  the oracle rejected the case\n");
            ok = 0;
        } else {
            /* integer inputs: every value is exact, so the fp32 outputs are equal (+0 and -0 alike) */
            size_t bad = 0;
            for (size_t i = 0; i < nc; i++) {
                if (D[i] != Dref[i]) bad++;
                if (has_aux && Aux[i] != Auxref[i]) bad++;
            }
            if (bad) fprintf(stderr, "  %zu fp32 outputs differ\n", bad);
            ok = bad == 0;
        }
        free(D);
        free(Aux);
        free(Dref);
        free(Auxref);
    }
    printf("%s kind=%d dtype=%s epi=f32 L=%lld M=%lld N=%lld K=%lld\n", ok ? "PASS" : "FAIL", kind, type_name(dtype),
           (long long)L, (long long)M, (long long)N, (long long)K);
    fflush(stdout);
    hipFree(dA);
    hipFree(dB);
    hipFree(dC);
    hipFree(dX);
    hipFree(dD);
    hipFree(dAux);
    free(A);
    free(B);
    free(C);
    free(X);
    return ok;
}

int main(void)
{
    const float lin[3] = {1.0f, 2.0f, 0.0f}, aux[3] = {1.0f, 2.0f, 0.5f}, xacc[3] = {2.0f, 1.0f, 3.0f};
    int fails = 0;
    for (int dtype = GEMM_EPI_F16; dtype <= GEMM_EPI_BF16; dtype++) {
        fails += !run_case(GEMM_EPI_LINCOMB, dtype, dtype, 1, 256, 512, 128, lin, 0);
        fails += !run_case(GEMM_EPI_AUX_SCALE, dtype, dtype, 2, 200, 136, 264, aux, 0);
        fails += !run_case(GEMM_EPI_LINCOMB_X_ACC, dtype, dtype, 1, 520, 776, 88, xacc, 0);
        fails += !run_case(GEMM_EPI_RELU_SQUARE, dtype, dtype, 3, 77, 45, 61, lin, 0); /* general kernel: K, N % 8 != 0 */
        /* the same kind of shapes staged through a workspace for the fast kernel */
        fails += !run_case(GEMM_EPI_RELU_SQUARE, dtype, dtype, 3, 77, 45, 61, lin, 1);
        fails += !run_case(GEMM_EPI_LINCOMB_X_ACC, dtype, dtype, 1, 300, 517, 139, xacc, 1);
    }
    /* the other element-type pairs of gemm_epi_run_mixed */
    fails += !run_case(GEMM_EPI_AUX_SCALE, GEMM_EPI_F16, GEMM_EPI_BF16, 2, 200, 136, 264, aux, 0);
    fails += !run_case(GEMM_EPI_LINCOMB_X_ACC, GEMM_EPI_BF16, GEMM_EPI_F16, 1, 520, 776, 88, xacc, 0);
    fails += !run_case_f32(GEMM_EPI_LINCOMB_X_ACC, GEMM_EPI_F16, 1, 520, 776, 88, xacc);
    fails += !run_case_f32(GEMM_EPI_RELU_SQUARE, GEMM_EPI_BF16, 3, 77, 45, 61, lin);
    /* an argument error comes back as a status code, before any launch */
    const int bad = gemm_epi_run_typed(1, 8, 8, 8, NULL, NULL, NULL, NULL, NULL, NULL, lin, 0, NULL, NULL, NULL,
                                       GEMM_EPI_F16, NULL);
    if (bad != GEMM_EPI_ERR_NULL_INPUT) {
        fprintf(stderr, "expected GEMM_EPI_ERR_NULL_INPUT, got %d\n", bad);
        fails++;
    }
    printf("%s: %d failing case(s)\n", fails ? "FAIL" : "PASS", fails);
    return fails ? 1 : 0;
}
