/*
 * gemm_epi.h -- C ABI of the fused fp16 GEMM + elementwise epilogue library
 * (libgemm_epi.so) for AMD Instinct MI355X (gfx950).
 *
 * One call computes, in ONE kernel launch,
 *
 *     acc[l][m][n] = sum_k A[l][m][k] * B[l][k][n]      (fp16 x fp16 -> fp32)
 *
 * and applies an elementwise epilogue to acc before anything is written, so
 * C (and X) are read once and D (and the second output) written once, with
 * no intermediate tensor in HBM.  This is the GEMM-with-fused-epilogue
 * operation of the CUTLASS Operator API tutorial "Custom epilogue fusions for
 * GEMMs" (cells [2]-[5]: batched A (L,M,K), B (L,K,N), C (L,M,N), fp16
 * operands, fp32 accumulator, outputs preallocated by the caller) and of the
 * CUTLASS "Custom Epilogue Example" page (Overview: three kernels fused into
 * one; Basic Example: batched GEMM with a custom epilogue).
 *
 * Layout: every tensor is packed, row-major and batched:
 *     A[l][m][k] at element (l*M + m)*K + k
 *     B[l][k][n] at element (l*K + k)*N + n
 *     C, X, D, Aux [l][m][n] at element (l*M + m)*N + n
 * (all epilogue tensors share one major order, as the "Constraints" section
 * of the Custom Epilogue Example requires).  Offsets are 64-bit.
 *
 * Arithmetic: fp16 inputs (or bfloat16, through gemm_epi_run_typed), fp32
 * accumulation (the tutorial's accumulator_type=torch.float32;
 * "--acc_dtype Float32" on the example's command line), epilogue in fp32
 * ("--epi_dtype Float32") from the unrounded accumulator, scalars in fp32
 * (the example's 'float' scalars), each output converted once to fp16 (or
 * bfloat16) with round-to-nearest-even (overflow gives inf).  The order of
 * the K summation is not specified; the epilogue's roundings are:
 * alpha*acc + beta*C is fma(alpha, acc, beta*C), + s*X one more fma, every
 * other operation rounded on its own, so every entry point gives the same
 * bits for the same accumulator.
 */
#ifndef GEMM_EPI_H
#define GEMM_EPI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Epilogue kinds.  s = scalars[2] (extra_scalar, x_factor, scale or a slope); the
 * second output (Aux, Y, E or F) is written to the Aux buffer.
 *
 * GEMM_EPI_LINCOMB        D = alpha*acc + beta*C
 *     (CUTLASS Python examples article: the "Basic GEMM" NumPy check and the
 *     default identity epilogue of the "Epilogue" example)
 * GEMM_EPI_AUX_SCALE      Aux = alpha*acc + beta*C ; D = s*Aux
 *     (tutorial cell [2], my_epilogue: alpha, beta, extra_scalar)
 * GEMM_EPI_LINCOMB_X_ACC  Y = acc ; D = alpha*acc + beta*C + s*X
 *     (Custom Epilogue Example, "Basic Example: Alpha-Beta Scaling",
 *     epilogue_operation: alpha, beta, x_factor)
 * GEMM_EPI_RELU           D = ReLU(alpha*acc + beta*C), ReLU(t) = t > 0 ? t : 0
 *     (Custom Epilogue Example, "Activation Functions")
 * GEMM_EPI_SQUARE         D = alpha*acc + beta*C ; E = D*D
 *     (Custom Epilogue Example, "Multiple Outputs", with alpha = beta = 1
 *     giving the page's D = acc + C)
 * GEMM_EPI_RELU_SQUARE    D = ReLU(alpha*acc + beta*C) ; E = D*D
 *     ("Activation Functions" followed by "Multiple Outputs")
 * GEMM_EPI_RELU_AUX_STORE F = alpha*acc + beta*C ; D = ReLU(F)
 *     (tutorial cell [6], relu_aux_store, whose beta is the constant 2.0;
 *     cell [8] is the same function with alpha = 1, beta = 0.5); F goes to
 *     the Aux buffer.
 * GEMM_EPI_RELU_SCALE_ACC F = ReLU(alpha*acc + beta*C) ; D = s*F, and acc
 *     itself as an fp32 output (tutorial cell [7], relu_scale_return_acc,
 *     with s = scale); F goes to the Aux buffer, acc to acc_out.  Needs
 *     gemm_epi_run_ext.
 * GEMM_EPI_BIAS_ROW_COL   D = (alpha*acc + row_bias[n]) + col_bias[m]
 *     (tutorial cell [9], broadcast_epilogue: row_bias has one value per
 *     column, shape (N,), col_bias one per row, shape (M, 1)); C is not read.
 *     Needs gemm_epi_run_ext.
 * GEMM_EPI_SIGMOID, GEMM_EPI_TANH, GEMM_EPI_GELU, GEMM_EPI_SILU,
 * GEMM_EPI_LEAKY_RELU, GEMM_EPI_HARDSWISH
 *                         D = act(alpha*acc + beta*C): the built-in
 *     activations of the Python examples article's "Epilogue" section
 *     (identity and relu are LINCOMB and RELU above).  sigmoid 1/(1+e^-t);
 *     tanh; gelu t*Phi(t) in its exact (erf) form; silu t*sigmoid(t);
 *     leaky_relu t > 0 ? t : s*t with the slope s = scalars[2]; hardswish
 *     t*min(max(t+3, 0), 6)/6.  Computed in fp32 (about 1e-6 relative or a
 *     few fp32 ulps), D rounded once to fp16.  No second output.
 *
 * The intermediate values (Aux before the scaling, D before the square, F
 * before the scaling) are used unrounded.
 */
typedef enum {
    GEMM_EPI_LINCOMB = 0,
    GEMM_EPI_AUX_SCALE = 1,
    GEMM_EPI_LINCOMB_X_ACC = 2,
    GEMM_EPI_RELU = 3,
    GEMM_EPI_SQUARE = 4,
    GEMM_EPI_RELU_SQUARE = 5,
    GEMM_EPI_RELU_AUX_STORE = 6,
    GEMM_EPI_RELU_SCALE_ACC = 7,
    GEMM_EPI_BIAS_ROW_COL = 8,
    GEMM_EPI_SIGMOID = 9,
    GEMM_EPI_TANH = 10,
    GEMM_EPI_GELU = 11,
    GEMM_EPI_SILU = 12,
    GEMM_EPI_LEAKY_RELU = 13,
    GEMM_EPI_HARDSWISH = 14
} gemm_epi_kind;

/*
 * Status codes.  The library never aborts; every error is a return value.
 * The argument checks run on the host before any HIP call, so they can be
 * exercised without a GPU.  They mirror the argument errors the tutorial's
 * "Failure examples" raise (cells [10]-[13]: an output or argument that is
 * not provided) and the "friendly errors" of the Python examples article
 * ("Basic GEMM", error handling).
 */
typedef enum {
    GEMM_EPI_OK = 0,
    GEMM_EPI_ERR_SHAPE = 1,       /* L, M, N or K < 1, or an element count overflows int64 */
    GEMM_EPI_ERR_NULL_INPUT = 2,  /* A, B or scalars NULL; C NULL for a kind that reads it (all but
                                     BIAS_ROW_COL); X NULL for LINCOMB_X_ACC; row_bias or col_bias
                                     NULL for BIAS_ROW_COL */
    GEMM_EPI_ERR_NULL_OUTPUT = 3, /* D NULL; Aux NULL for a kind with a second output; acc_out NULL
                                     for RELU_SCALE_ACC */
    GEMM_EPI_ERR_KIND = 4,        /* unknown epilogue kind */
    GEMM_EPI_ERR_ALIGN = 5,       /* a 16-bit tensor is not 2-byte aligned, or acc_out (or an fp32
                                     epilogue tensor) is not 4-byte aligned */
    GEMM_EPI_ERR_HIP = 6,         /* the launch failed; see gemm_epi_last_hip_error() */
    GEMM_EPI_ERR_WORKSPACE = 7,   /* the workspace is NULL or smaller than the call needs
                                     (gemm_epi_run_unfused, gemm_epi_run_ws) */
    GEMM_EPI_ERR_DTYPE = 8        /* unknown element type or combination (the *_typed entry points,
                                     gemm_epi_run_mixed) */
} gemm_epi_status;

/*
 * Element types of the tensors (A, B, C, X, row_bias, col_bias, D, Aux), for
 * the *_typed entry points (one 16-bit type for all of them) and
 * gemm_epi_run_mixed (fp32 epilogue tensors): the Custom Epilogue Example's
 * "Data Type Support" lists FP16 and BF16 among the input types (A, B) and
 * FP32, FP16 and BF16 among the output types (C, D).  Accumulation and the
 * epilogue stay fp32; acc_out stays fp32.
 */
typedef enum {
    GEMM_EPI_F16 = 0,  /* IEEE 754 binary16 */
    GEMM_EPI_BF16 = 1, /* bfloat16: 1 sign, 8 exponent and 7 fraction bits (the upper half of a binary32) */
    GEMM_EPI_F32 = 2   /* IEEE 754 binary32 (epilogue tensors only) */
} gemm_epi_dtype;

/*
 * gemm_epi_run -- launch the fused GEMM + epilogue on `stream`.
 *
 *   L, M, N, K  batch count and problem sizes, each >= 1.
 *   A, B        device pointers, fp16 (IEEE binary16), layout above.
 *   C           device pointer, fp16, read by every kind but BIAS_ROW_COL
 *               (also when beta = 0); may be NULL for BIAS_ROW_COL.
 *   X           device pointer, fp16; read only by GEMM_EPI_LINCOMB_X_ACC,
 *               may be NULL otherwise.
 *   scalars     HOST pointer to 3 floats {alpha, beta, s}; read during the
 *               call and passed by value to the kernel, so the caller may
 *               reuse the memory as soon as the call returns.
 *   epilogue_kind  a gemm_epi_kind value.
 *   D           device pointer, fp16 output.
 *   Aux         device pointer, fp16 second output (Aux, Y, E or F) for
 *               AUX_SCALE, LINCOMB_X_ACC, SQUARE, RELU_SQUARE, RELU_AUX_STORE
 *               and RELU_SCALE_ACC; may be NULL for the other kinds.
 *   stream      a hipStream_t (0 = the null stream).
 *
 * Ownership: the caller allocates, owns and frees every buffer.  The library
 * allocates no device memory, frees nothing and does not synchronise: the
 * launch is asynchronous on `stream`, and the outputs are ready once the
 * stream reaches that point.  Outputs must not overlap each other or any
 * input (the result is undefined otherwise).
 *
 * Fast path: when K % 8 == 0, N % 8 == 0 and A, B, C, X, D, Aux are 16-byte
 * aligned (the "Constraints" section's 16-byte rule), and A and B of one batch
 * entry each span less than 2 GiB, the kernel moves 16-byte vectors;
 * otherwise a general kernel with element-wise edge handling runs.  Both
 * compute the same definition; their fp32 sums run in different orders, so
 * the results are identical on integer-valued inputs and can differ in the
 * last bits otherwise.  gemm_epi_run_ws, given a workspace, runs the fast
 * kernel on copies of such operands instead.
 *
 * Returns GEMM_EPI_OK, or a gemm_epi_status error code; on an error before
 * the launch nothing is queued on the stream.  RELU_SCALE_ACC and
 * BIAS_ROW_COL need operands this entry point does not take: use
 * gemm_epi_run_ext (here they return GEMM_EPI_ERR_NULL_OUTPUT and
 * GEMM_EPI_ERR_NULL_INPUT).
 */
int gemm_epi_run(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                 const void *X, const float *scalars, int epilogue_kind, void *D, void *Aux, void *stream);

/*
 * gemm_epi_run_ext -- gemm_epi_run with the operands of the broadcast and
 * accumulator-returning kinds (tutorial cells [7] and [9]); every kind can be
 * launched through it.  The arguments shared with gemm_epi_run mean the
 * same; in addition:
 *
 *   row_bias    device pointer, fp16, N values (one per output column),
 *               shared by every batch entry; read only by BIAS_ROW_COL, may
 *               be NULL otherwise.
 *   col_bias    device pointer, fp16, M values (one per output row), shared
 *               by every batch entry; read only by BIAS_ROW_COL, may be NULL
 *               otherwise.
 *   acc_out     device pointer, fp32 (IEEE binary32), (L,M,N) packed
 *               row-major like D: the accumulator itself, written only by
 *               RELU_SCALE_ACC; may be NULL otherwise.
 *
 * Ownership, asynchrony and the status codes are those of gemm_epi_run.  The
 * fast path additionally needs row_bias and acc_out 16-byte aligned.
 */
int gemm_epi_run_ext(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                     const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                     int epilogue_kind, void *D, void *Aux, void *acc_out, void *stream);

/*
 * gemm_epi_run_typed -- gemm_epi_run_ext with the element type of the 16-bit
 * tensors as an argument: dtype is GEMM_EPI_F16 (then the call is exactly
 * gemm_epi_run_ext) or GEMM_EPI_BF16, in which case A, B, C, X, row_bias,
 * col_bias, D and Aux all hold bfloat16 values with the same shapes, layouts
 * and alignment rules.  bfloat16 products are exact in fp32, the accumulator
 * and the epilogue are fp32 as for fp16, and every bfloat16 output is
 * rounded once, to nearest with ties to even.  The tile choice
 * (gemm_epi_plan_ext) does not depend on dtype.  Status codes as
 * gemm_epi_run_ext, plus GEMM_EPI_ERR_DTYPE for another dtype value.
 */
int gemm_epi_run_typed(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                       const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                       int epilogue_kind, void *D, void *Aux, void *acc_out, int dtype, void *stream);

/*
 * gemm_epi_run_mixed -- the fused call with separate element types for A, B
 * (ab_dtype: GEMM_EPI_F16 or GEMM_EPI_BF16) and for the epilogue tensors C, X,
 * row_bias, col_bias, D and Aux (epi_dtype: GEMM_EPI_F16, GEMM_EPI_BF16 or
 * GEMM_EPI_F32; equal to ab_dtype, the call is exactly gemm_epi_run_typed).
 * The example lists FP16 and BF16 as input types and FP32, FP16 and BF16 as
 * C and D types.  The same fp32 epilogue runs whatever the types: C, X and
 * the biases are widened exactly, and each 16-bit output is rounded once to
 * nearest-even; fp32 outputs are stored without a further rounding.  fp32
 * tensors must be 4-byte aligned (16-byte aligned, with K % 8 == N % 8 == 0
 * and 16-byte aligned A, B, for the vector kernels); shapes and layouts are
 * unchanged.  Status codes as gemm_epi_run_ext, plus GEMM_EPI_ERR_DTYPE for
 * any other combination.
 */
int gemm_epi_run_mixed(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                       const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                       int epilogue_kind, void *D, void *Aux, void *acc_out, int ab_dtype, int epi_dtype,
                       void *stream);

/*
 * gemm_epi_run_unfused -- the same operation as gemm_epi_run_ext, NOT fused:
 * one launch computes the GEMM and writes the fp32 accumulator to HBM, a
 * second, elementwise launch reads it back with C / X / the biases and
 * writes the outputs.  This is the composition the pages' fusion replaces
 * (Custom Epilogue Example, Overview: matmul, then scale/add, then the
 * activation as separate kernels, with intermediates in global memory); it
 * is here to measure what the fusion saves.  Its outputs equal those of
 * gemm_epi_run_ext bit for bit (the same accumulator, the same fp32
 * epilogue arithmetic) whenever both take the same GEMM kernel: its GEMM
 * launch chooses the fast or the general kernel from A, B and the workspace
 * alone, the fused call from every tensor.  On integer-valued inputs they
 * are equal in any case.
 *
 *   workspace        device pointer to at least L*M*N*4 bytes (4-byte
 *                    aligned; 16-byte aligned for the vector path) that
 *                    receives the fp32 accumulator; owned by the caller.
 *                    RELU_SCALE_ACC writes its accumulator to acc_out
 *                    instead and may pass NULL.
 *   workspace_bytes  its size in bytes.
 *
 * The other arguments, the ownership rules and the status codes are those of
 * gemm_epi_run_ext; GEMM_EPI_ERR_WORKSPACE when the workspace is missing or
 * too small.  The two launches are queued on `stream` in order.
 */
int gemm_epi_run_unfused(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                         const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                         int epilogue_kind, void *D, void *Aux, void *acc_out, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * gemm_epi_run_unfused_typed -- gemm_epi_run_unfused with the element type
 * of the 16-bit tensors as an argument, as in gemm_epi_run_typed (the
 * workspace stays fp32).  With GEMM_EPI_F16 it is exactly
 * gemm_epi_run_unfused; with GEMM_EPI_BF16 its outputs equal those of
 * gemm_epi_run_typed with GEMM_EPI_BF16 bit for bit.  Status codes as
 * gemm_epi_run_unfused, plus GEMM_EPI_ERR_DTYPE.
 */
int gemm_epi_run_unfused_typed(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                               const void *C, const void *X, const void *row_bias, const void *col_bias,
                               const float *scalars, int epilogue_kind, void *D, void *Aux, void *acc_out,
                               void *workspace, size_t workspace_bytes, int dtype, void *stream);

/*
 * gemm_epi_run_ws -- gemm_epi_run_ext that may split the K range of tiles
 * across workgroups (stream-K scheduling, the Python examples article's
 * "Basic GEMM" swizzling option) when the problem has too few tiles to keep
 * every compute unit busy.  The partial sums of a split tile go to the
 * workspace; the last workgroup to finish its part of the tile adds them up,
 * in k order, and applies the epilogue (the epilogue is not linear, so it
 * only ever sees the full sum).  Where splitting does not pay, the call is
 * exactly gemm_epi_run_ext and the workspace is not touched, with one
 * exception.  Operands that miss the fast kernel's layout rules (the 16-byte
 * alignment rule of the Custom Epilogue Example's "Constraints": K or N not a
 * multiple of 8, or a tensor not 16-byte aligned) are staged through the
 * workspace when it is large enough.  The call copies them into aligned
 * buffers whose rows are padded with zeros, runs the fast kernel on those and
 * copies padded outputs back, all on `stream` (the zero products leave every
 * sum unchanged, so the results are gemm_epi_run_ext's, up to the sign of a
 * zero).  Where the staged problem has few tiles and a long K, it is also
 * split as above (the partial sums first, then the staged copies).  With a
 * smaller workspace, or none, such a call runs gemm_epi_run_ext's general
 * kernel instead.  Staging never writes the counter block below.
 *
 *   workspace        device pointer, 16-byte aligned, of at least the size
 *                    gemm_epi_plan_ws reports in out[6] (0 when neither a
 *                    split nor staging is planned: NULL is then accepted);
 *                    owned by the caller.  It
 *                    must be zero-filled before its first use (e.g. one
 *                    hipMemset); every call leaves it ready for the next,
 *                    whatever the shape: the per-tile counters sit in a
 *                    block of fixed size at its start (16 KiB, one int32 per
 *                    tile of a split; at most 4096 tiles are split), the
 *                    partial sums after it.
 *   workspace_bytes  its size in bytes.
 *
 * Calls that share one workspace must not overlap in time (two streams
 * running them concurrently race).  The sum of a split tile is ordered the
 * same way on every call, so results are deterministic; they can differ
 * from gemm_epi_run_ext's in the last bits of fp32 summation order
 * (identical on integer-valued inputs).  Status codes as gemm_epi_run_ext,
 * plus GEMM_EPI_ERR_WORKSPACE.
 */
int gemm_epi_run_ws(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                    const void *X, const void *row_bias, const void *col_bias, const float *scalars, int epilogue_kind,
                    void *D, void *Aux, void *acc_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gemm_epi_run_ws_typed -- gemm_epi_run_ws with the element type of the
 * 16-bit tensors as an argument, as in gemm_epi_run_typed.  The split or
 * staging (gemm_epi_plan_ws) and the workspace do not depend on dtype; where
 * neither is planned the call is exactly gemm_epi_run_typed.  Status codes as
 * gemm_epi_run_ws, plus GEMM_EPI_ERR_DTYPE.
 */
int gemm_epi_run_ws_typed(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                          const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                          int epilogue_kind, void *D, void *Aux, void *acc_out, void *workspace,
                          size_t workspace_bytes, int dtype, void *stream);

/*
 * gemm_epi_run_ws_static -- gemm_epi_run_ws_typed without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split's counters and partial sums live in a device array inside the
 * library: 16 MiB + 16 KiB on each GPU the library runs on, held until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); on a device's first call it looks up the
 * array's address and clears its counter block with a kernel on `stream`
 * (under graph capture that kernel is captured with the call and runs at
 * each replay, ahead of the split).
 * Its splits use at most 128 workgroups (so its plan can differ from
 * gemm_epi_plan_ws's, which allows 256; results are the same on integer
 * inputs and within the fp32 summation order otherwise); where no split
 * pays the call is exactly gemm_epi_run_typed (it does not stage operands).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, two threads) race.  `stream` must belong to the calling thread's current
 * device.  Status codes as gemm_epi_run_ws_typed; GEMM_EPI_ERR_WORKSPACE if a
 * split would not fit the array; GEMM_EPI_ERR_HIP if the array cannot be
 * located (for example the current device's index is 64 or more).
 */
int gemm_epi_run_ws_static(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                           const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                           int epilogue_kind, void *D, void *Aux, void *acc_out, int dtype, void *stream);

/* gemm_epi_plan_ext for gemm_epi_run_ws: out[0..5] as gemm_epi_plan (out[4] is
 * the number of workgroups, the split's workgroup count when it splits), and
 * out[6] the workspace bytes the call needs (0: no split and no staging).  A
 * call that stages its operands reports the fast kernel's tile, out[3] = 1. */
int gemm_epi_plan_ws(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                     const void *X, const void *row_bias, const void *col_bias, int epilogue_kind, const void *D,
                     const void *Aux, const void *acc_out, int64_t out[7]);

/* A static, human-readable name for a status code ("unknown status" for
 * values outside the enum).  Never NULL. */
const char *gemm_epi_status_string(int status);

/* The hipError_t value behind the calling thread's most recent
 * GEMM_EPI_ERR_HIP (0 if there was none).  Thread-local. */
int gemm_epi_last_hip_error(void);

/*
 * gemm_epi_plan -- host-only query: the kernel configuration gemm_epi_run
 * would launch for these arguments, without launching anything.
 *   out[0] tile rows (BM), out[1] tile columns (BN), out[2] K step (BK),
 *   out[3] 1 for the 16-byte fast path, 0 for the general kernel,
 *   out[4] number of workgroups, out[5] threads per workgroup.
 * Returns the same argument-check status gemm_epi_run would return (pointers
 * are checked for NULL and alignment only, never dereferenced).
 */
int gemm_epi_plan(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                  const void *X, int epilogue_kind, const void *D, const void *Aux, int64_t out[6]);

/* gemm_epi_plan for the arguments of gemm_epi_run_ext. */
int gemm_epi_plan_ext(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                      const void *X, const void *row_bias, const void *col_bias, int epilogue_kind, const void *D,
                      const void *Aux, const void *acc_out, int64_t out[6]);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_EPI_H */
