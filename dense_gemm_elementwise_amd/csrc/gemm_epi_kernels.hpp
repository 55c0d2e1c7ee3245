// gemm_epi_kernels.hpp -- gfx950 (CDNA4) kernels for the fused fp16 GEMM +
// elementwise epilogue.
//
// One workgroup computes one BM x BN tile of one batch entry:
//   acc = A[l][m0:m0+BM, :] @ B[l][:, n0:n0+BN]      (fp16 in, fp32 MFMA acc)
// then applies the epilogue to acc in registers and writes D (and the second
// output) once.  The operation is the GEMM with a fused epilogue of the
// CUTLASS Operator API tutorial "Custom epilogue fusions for GEMMs" and the
// CUTLASS "Custom Epilogue Example" (Overview: matmul, scale/add and
// activation in one kernel instead of three).
//
// Design for gfx950 (not a translation of the pages' Blackwell kernels):
//  * WGM x WGN wave64s per workgroup; each wave owns a (BM/WGM) x (BN/WGN)
//    accumulator tile built from v_mfma_f32_16x16x32_f16 (MI = 16) or
//    v_mfma_f32_32x32x16_f16 (MI = 32) blocks.  With two waves per SIMD
//    (8 waves), one wave's MFMAs run while the other waits on LDS or a
//    barrier.
//  * K is walked in steps of BK through a ring of NSTAGES LDS stages, so the
//    loads of a stage are issued NSTAGES-1 stages before it is used.  The
//    fast path fills LDS with buffer_load_dwordx4 ... lds (global -> LDS
//    without VGPRs).  Each thread's DMA offsets are fixed; a stage only moves
//    the buffer descriptor's base, and lanes outside the matrix get an
//    out-of-range offset that the buffer unit turns into zeros, so M, N and K
//    tails cost no extra code in the inner loop.
//  * A tiles are stored row-major (BK*2 bytes per row); B tiles k-row-major.
//    The 16-byte chunks of each row are XOR-swizzled so that the MFMA operand
//    reads (ds_read_b128 for A, ds_read_b64_tr_b16 for B, which transposes
//    the N-contiguous B rows into the K-contiguous operand on the fly) hit
//    distinct banks.
//  * The epilogue moves each wave's accumulator through LDS, one MFMA row
//    block at a time, so that every lane owns 4 consecutive columns; C / X
//    are prefetched into registers one block ahead and D / Aux written with
//    8-byte vectors, predicated at the M / N edges.  (Reading C / X straight
//    in the MFMA register layout would touch 16 or 32 rows per instruction;
//    the row-contiguous layout keeps each instruction on 4 rows.)
//  * Workgroup ids are remapped so that the tiles one XCD runs together are
//    neighbours (they share A row panels and B column panels in that XCD's
//    L2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gemm_epi {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 16-bit tensor elements travel as raw bits in _Float16 storage; BF selects
// how the bits read: IEEE binary16, or bfloat16 (the upper half of an IEEE
// binary32: widening is a shift, narrowing is the hardware's
// round-to-nearest-even conversion).
template <bool BF>
__device__ __forceinline__ float ld16(_Float16 h)
{
    if constexpr (BF)
        return __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
    else
        return (float)h;
}
template <bool BF>
__device__ __forceinline__ _Float16 st16(float f)
{
    if constexpr (BF)
        return __builtin_bit_cast(_Float16, (__bf16)f);
    else
        return (_Float16)f;
}

// Element type of the epilogue tensors (C, X, the biases, D, Aux), by EPI:
// EPI_AB the 16-bit type of A and B; EPI_F32 fp32 (widening is then the
// identity and narrowing does not round); EPI_OTHER16 the other 16-bit type
// (bfloat16 for fp16 A and B, fp16 for bfloat16 ones).
enum EpiMode : int { EPI_AB = 0, EPI_F32 = 1, EPI_OTHER16 = 2 };
template <bool BF, int EPI>
struct EpiElem {
    static constexpr bool EBF = EPI == EPI_OTHER16 ? !BF : BF;
    using T = _Float16;
    static __device__ __forceinline__ float ld(T v) { return ld16<EBF>(v); }
    static __device__ __forceinline__ T st(float f) { return st16<EBF>(f); }
};
template <bool BF>
struct EpiElem<BF, EPI_F32> {
    using T = float;
    static __device__ __forceinline__ float ld(T v) { return v; }
    static __device__ __forceinline__ T st(float f) { return f; }
};
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

#define GE_LDS(T) __attribute__((address_space(3))) T

enum Kind : int {
    LINCOMB = 0,
    AUX_SCALE = 1,
    LINCOMB_X_ACC = 2,
    RELU = 3,
    SQUARE = 4,
    RELU_SQUARE = 5,
    RELU_AUX_STORE = 6,
    RELU_SCALE_ACC = 7,
    BIAS_ROW_COL = 8,
    SIGMOID = 9,
    TANH = 10,
    GELU = 11,
    SILU = 12,
    LEAKY_RELU = 13,
    HARDSWISH = 14,
    // not a public kind: the GEMM stage of the unfused composition, which
    // writes only the fp32 accumulator
    ACC_STORE = 16
};

__host__ __device__ constexpr bool kind_has_aux(int k)
{
    return k == AUX_SCALE || k == LINCOMB_X_ACC || k == SQUARE || k == RELU_SQUARE || k == RELU_AUX_STORE ||
           k == RELU_SCALE_ACC;
}
__host__ __device__ constexpr bool kind_reads_x(int k) { return k == LINCOMB_X_ACC; }
__host__ __device__ constexpr bool kind_reads_c(int k) { return k != BIAS_ROW_COL && k != ACC_STORE; }
__host__ __device__ constexpr bool kind_reads_bias(int k) { return k == BIAS_ROW_COL; }
__host__ __device__ constexpr bool kind_has_acc_out(int k) { return k == RELU_SCALE_ACC || k == ACC_STORE; }
__host__ __device__ constexpr bool kind_writes_d(int k) { return k != ACC_STORE; }

// The 16-bit tensors travel as raw bits; C, X, D, Aux and the biases hold
// fp32 values instead when the kernel is built with EPI_F32 (the kernel
// reads them through its epilogue element type).
struct Params {
    const _Float16 *A;
    const _Float16 *B;
    const _Float16 *C;
    const _Float16 *X;
    _Float16 *D;
    _Float16 *Aux;
    const _Float16 *row_bias;  // N values, shared by the batch entries
    const _Float16 *col_bias;  // M values, shared by the batch entries
    float *acc_out;            // (L, M, N) fp32 accumulator output
    int M, N, K;      // each < 2^31 (checked on the host)
    // rows of each batch entry of B, and the bound of its k rows, when they
    // differ from K (0: K).  The staged path pads A's rows to a multiple of 8
    // with zeros and runs K = that length over an unpadded B: the rows of B
    // past b_rows read as zeros.  Only the fast path reads it.
    int b_rows;
    int tiles_m, tiles_n;
    int num_tiles;    // L * tiles_m * tiles_n
    int group_m;      // tile rows per L2 group (>= 1)
    float alpha, beta, s;
    // stream-K split (only read by the kernels built for it): the L*tiles
    // (tile, k stage) units in tile-major order, sk_q or sk_q + 1 of them per
    // workgroup (the first sk_r workgroups take one more)
    int64_t sk_q, sk_r;
    float *partials;  // 2 slots of BM*BN floats per workgroup
    int *counters;    // one per tile, zero between calls
};

// ---------------------------------------------------------------------------
// Epilogue math, fp32.  d = first output, a = second output (if any); rb /
// cb are the row-broadcast bias of the element's column and the
// column-broadcast bias of its row.  The roundings are fixed here, not left
// to the compiler's contraction of multiply-adds (which follows the shape of
// the calling code): alpha*acc + beta*c is fma(alpha, acc, beta*c), + s*x is
// one more fma, and nothing else is contracted.  So every kernel that applies
// an epilogue (the fused GEMM, the elementwise stage of the unfused
// composition) gives bit-identical outputs.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Activations, fp32, written from the mathematics (no library call).  Their
// error is a few fp32 units in the last place or about 1e-6 relative, far
// below the fp16 output's 2^-11.  Quotients use the hardware reciprocal
// (v_rcp_f32, 1 ulp) instead of the correctly rounded division, a sequence of
// about ten instructions that made the GELU epilogue VALU-bound.
// ---------------------------------------------------------------------------
// e^x = 2^(x log2 e) on the hardware base-2 exponential (v_exp_f32).  It
// returns no subnormals, so a factor that may fall below 2^-126 is formed
// as a product of two halves, e^x = e^(x/2) e^(x/2): the multiply rounds
// once into the subnormal range (the kernels run with fp32 subnormals
// enabled), which the bfloat16 outputs can hold down to 2^-133.
__device__ __forceinline__ float act_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float act_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
// sigmoid(x) = 1 / (1 + e^-x) for x >= 0 and e^x / (1 + e^x) for x < 0, with
// e^-|x| = v v, v = e^(-|x|/2): nothing overflows, and far left the result is
// e^x itself, subnormal included
__device__ __forceinline__ float act_sigmoid(float x)
{
#pragma clang fp contract(off)
    const float v = act_exp(-0.5f * __builtin_fabsf(x));
    const float e = v * v;
    const float r = act_rcp(1.0f + e);
    return x >= 0.0f ? r : e * r;
}
// tanh: for |x| < 1/4 its Maclaurin series to x^9 (truncation below 1e-8
// relative); otherwise (1 - e^-2|x|) / (1 + e^-2|x|) with the sign of x, where
// e^-2|x| <= 0.61 so nothing cancels
__device__ __forceinline__ float act_tanh(float x)
{
#pragma clang fp contract(off)
    const float ax = __builtin_fabsf(x);
    if (ax < 0.25f) {
        const float x2 = x * x;
        float p = 62.0f / 2835.0f;
        p = __builtin_fmaf(p, x2, -17.0f / 315.0f);
        p = __builtin_fmaf(p, x2, 2.0f / 15.0f);
        p = __builtin_fmaf(p, x2, -1.0f / 3.0f);
        return __builtin_fmaf(x * x2, p, x);
    }
    const float e = act_exp(-2.0f * ax);
    return __builtin_copysignf((1.0f - e) * act_rcp(1.0f + e), x);
}
// x > 0 times a factor below 1 that rounded to exactly 1 in fp32 (sigmoid(x)
// and Phi(x) far right): the exact product lies below x by less than one
// fp32 ulp.  Rounding x on to a 16-bit output goes wrong where x is a 16-bit
// midpoint: the tie goes to the even neighbour, sometimes the upper one,
// while the exact value lies below the midpoint.  Of x and its lower
// neighbour, the one with an odd last bit (the product rounded to odd) is
// never such a midpoint, and rounds to the 16-bit value of the exact
// product; as an fp32 output it is within one ulp of it.
__device__ __forceinline__ float act_just_below(float x)
{
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    return x < __builtin_inff() ? __builtin_bit_cast(float, b - (~b & 1u)) : x;
}
// gelu(x) = x Phi(x), Phi(x) = erfc(-x / sqrt 2) / 2, in the form that keeps
// relative accuracy in the left tail: with z = |x| / sqrt 2,
// x >= 0: x (1 - erfc(z) / 2); x < 0: x erfc(z) / 2.  erfc(z) = e^{-z^2} P(t),
// t = 2 / (2 + z), P a degree-8 polynomial fitted to the scaled
// complementary error function by fit_erfc.py (relative error 7e-8).
// e^{-z^2} = h h with h = e^{-z^2/2}, multiplied in last: past x = -13.2 the
// result is subnormal in fp32
__device__ __forceinline__ float act_gelu(float x)
{
#pragma clang fp contract(off)
    constexpr float c[9] = {-2.037919330e-04f, 2.859725058e-01f, 2.504409850e-01f, 3.914754093e-01f,
                            -2.268847674e-01f, 7.775521874e-01f, -6.962806582e-01f, 2.504747510e-01f,
                            -3.254655749e-02f};
    const float z = __builtin_fabsf(x) * 0.707106781186547524f;
    const float t = 2.0f * act_rcp(2.0f + z);
    float p = c[8];
#pragma unroll
    for (int k = 7; k >= 0; k--) p = __builtin_fmaf(p, t, c[k]);
    const float h = act_exp(-0.5f * (z * z));
    if (x < 0.0f) return (((0.5f * x) * p) * h) * h;
    const float f = 1.0f - 0.5f * ((p * h) * h);
    return f == 1.0f && x > 0.0f ? act_just_below(x) : x * f;
}
// silu(x) = x sigmoid(x); for x < 0, x e^x / (1 + e^x) with the product
// x e^x formed as (x v) v, v = e^(x/2)
__device__ __forceinline__ float act_silu(float x)
{
#pragma clang fp contract(off)
    const float v = act_exp(-0.5f * __builtin_fabsf(x));
    const float e = v * v;
    const float r = act_rcp(1.0f + e);
    if (x < 0.0f) return ((x * v) * v) * r;
    return r == 1.0f && x > 0.0f ? act_just_below(x) : x * r;
}
__device__ __forceinline__ float act_hardswish(float x)
{
#pragma clang fp contract(off)
    const float r = x * __builtin_fminf(__builtin_fmaxf(x + 3.0f, 0.0f), 6.0f) * (1.0f / 6.0f);
    // x <= -3: exactly zero, with x's sign (x times +0).  Written out, because
    // the clamp's lowering differs between kernels and one of them returned
    // +0 there.
    return x <= -3.0f ? __builtin_copysignf(0.0f, x) : r;
}

template <int KIND>
__device__ __forceinline__ void epi_elem(float acc, float c, float x, float rb, float cb, float alpha, float beta,
                                         float s, float &d, float &a)
{
#pragma clang fp contract(off)
    const float lin = __builtin_fmaf(alpha, acc, beta * c);
    if constexpr (KIND == LINCOMB) {
        d = lin;
    } else if constexpr (KIND == AUX_SCALE) {
        a = lin;
        d = s * lin;
    } else if constexpr (KIND == LINCOMB_X_ACC) {
        a = acc;
        d = __builtin_fmaf(s, x, lin);
    } else if constexpr (KIND == RELU) {
        d = lin > 0.0f ? lin : 0.0f;
    } else if constexpr (KIND == SQUARE) {
        d = lin;
        a = lin * lin;
    } else if constexpr (KIND == RELU_SQUARE) {
        const float t = lin > 0.0f ? lin : 0.0f;
        d = t;
        a = t * t;
    } else if constexpr (KIND == RELU_AUX_STORE) {
        a = lin;
        d = lin > 0.0f ? lin : 0.0f;
    } else if constexpr (KIND == RELU_SCALE_ACC) {
        const float t = lin > 0.0f ? lin : 0.0f;
        a = t;
        d = s * t;
    } else if constexpr (KIND == BIAS_ROW_COL) {
        d = __builtin_fmaf(alpha, acc, rb) + cb;
    } else if constexpr (KIND == SIGMOID) {
        d = act_sigmoid(lin);
    } else if constexpr (KIND == TANH) {
        d = act_tanh(lin);
    } else if constexpr (KIND == GELU) {
        d = act_gelu(lin);
    } else if constexpr (KIND == SILU) {
        d = act_silu(lin);
    } else if constexpr (KIND == LEAKY_RELU) {
        d = lin > 0.0f ? lin : s * lin;
    } else if constexpr (KIND == HARDSWISH) {
        d = act_hardswish(lin);
    } else {  // ACC_STORE: nothing but the accumulator itself is written
        d = acc;
    }
}

// ---------------------------------------------------------------------------
// Tile scheduling: hardware workgroup id -> (batch, tile row, tile column).
// Workgroups are handed to the 8 XCDs round-robin (id % 8), so consecutive
// logical tiles are given to ids that land on the same XCD; within a batch
// entry tiles are ordered in groups of p.group_m tile rows, column-major
// inside a group, so the tiles an XCD runs together share operand panels.
// ---------------------------------------------------------------------------
// logical index of workgroup w among nwg: consecutive on one XCD
__device__ __forceinline__ int xcd_logical_id(int nwg, int w)
{
    const int xcd = w & 7, j = w >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + j;
}

// logical tile t -> (batch, tile row, tile column) in the grouped order
__device__ __forceinline__ void tile_coords(const Params &p, int t, int &l, int &tm, int &tn)
{
    const int tpb = p.tiles_m * p.tiles_n;
    l = t / tpb;
    const int r = t - l * tpb;
    const int group_m = p.group_m;
    const int gsize_full = group_m * p.tiles_n;
    const int g = r / gsize_full;
    const int first_m = g * group_m;
    const int gm = min(p.tiles_m - first_m, group_m);
    const int rr = r - g * gsize_full;
    tm = first_m + rr % gm;
    tn = rr / gm;
}

__device__ __forceinline__ void map_tile(const Params &p, int &l, int &tm, int &tn)
{
    tile_coords(p, xcd_logical_id(p.num_tiles, blockIdx.x), l, tm, tn);
}

// Stream-K bookkeeping.  Units are (tile, k stage) pairs in tile-major order;
// workgroup w (logical) owns units [sk_begin(w), sk_begin(w + 1)).
__device__ __forceinline__ int64_t sk_begin(const Params &p, int w)
{
    return (int64_t)w * p.sk_q + (w < p.sk_r ? w : p.sk_r);
}
__device__ __forceinline__ int sk_owner(const Params &p, int64_t u)  // the workgroup owning unit u
{
    const int64_t big = p.sk_r * (p.sk_q + 1);
    return u < big ? (int)(u / (p.sk_q + 1)) : (int)(p.sk_r + (u - big) / p.sk_q);
}
// A workgroup contributes partial sums to at most two tiles: the one its
// range starts in (slot 2w) and the one it ends in (slot 2w + 1).
__device__ __forceinline__ int sk_slot(const Params &p, int w, int t, int nk_tile)
{
    return 2 * w + (sk_begin(p, w) / nk_tile == t ? 0 : 1);
}

// Swizzles (in 16-byte chunk units).  An A row holds A_CHUNKS = BK/8 chunks;
// row r stores logical chunk c at physical chunk c ^ swz_a(r).  A B k-row
// holds BN/8 chunks; k-row kr stores logical chunk c at c ^ swz_b(kr).
//
// An A operand read (ds_read_b128) has 16 or 32 consecutive rows at one
// logical chunk per group of lanes.  The swizzle depends on the row pair
// only (row >> 1): the two rows of a pair keep their relative position and
// each pair moves to its own chunk.  Swizzles that also mix the row's low bit
// into the chunk conflict 2-way on gfx950 for this read, with 128-byte and
// with 64-byte rows and for both MFMA shapes (measured with the LDS
// bank-conflict counter).  256-byte rows each span all 64 banks, so there
// the low bit has to go in as well: 16 rows, 16 chunks.
template <int A_CHUNKS>
__device__ __forceinline__ int swz_a(int row)
{
    if constexpr (A_CHUNKS == 16)
        return ((row >> 1) & 7) | ((row & 1) << 3);  // 256-byte rows
    else if constexpr (A_CHUNKS == 8)
        return (row >> 1) & 7;  // 128-byte rows
    else
        return (row >> 1) & 3;  // 64-byte rows
}
//
// The B transpose reads differ by MFMA shape.  MI = 32: the 32 lanes served
// together read 4 consecutive k-rows x 4 consecutive chunks.  MI = 16: they
// read k-rows r..r+3 and r+8..r+11 x 2 consecutive chunks, so the swizzle also
// separates k-rows 8 apart.  With 8-chunk (128-byte) k-rows, even and odd
// k-rows fall in opposite halves of the 64 banks, and the four k-rows of one
// parity (bits 1 and 3 of the k-row) take the four chunk pairs: a 2-way
// conflict left by 2 * (krow & 3) cost 32% of the 64 x 64 tile's LDS cycles.
template <int B_CHUNKS, int MI>
__device__ __forceinline__ int swz_b(int krow)
{
    if constexpr (B_CHUNKS >= 16 && MI == 32)
        return (0xCA60 >> ((krow & 3) * 4)) & 15;          // 0, 6, 10, 12 for krow % 4 = 0..3
    else if constexpr (B_CHUNKS >= 16)
        return 2 * ((krow & 3) | (((krow >> 3) & 1) << 2));  // 0, 2, .., 14 over krow % 4 and bit 3
    else if constexpr (MI == 16)
        return 2 * (((krow >> 1) & 1) | (((krow >> 3) & 1) << 1));  // 8-chunk rows: 0, 2, 4, 6
    else
        return 2 * (krow & 3);                              // 8-chunk rows: 0, 2, 4, 6
}

// ---------------------------------------------------------------------------
// 16-byte global -> LDS DMA: buffer_load_dwordx4 ... lds writes lane i's 16
// bytes to LDS address M0 + 16*i.  Written as inline asm so that the compiler
// does not treat every later LDS read as dependent on it (it would otherwise
// wait for all outstanding DMA before each read, which serialises the
// prefetch with the MFMA work); the kernel waits for the DMA itself before
// the barrier that publishes a stage.
// ---------------------------------------------------------------------------
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t num_bytes)
{
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);  // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)num_bytes);
    r[3] = 0x00020000;  // raw buffer, 32-bit data format
    return r;
}

// M0 is a reserved register for the compiler; the kernels use it for nothing
// else (no other LDS DMA, s_sendmsg or movrel), so clobbering it here is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const i32x4 &rsrc, uint32_t lds_addr, int voffset)
{
    const int m0v = __builtin_amdgcn_readfirstlane((int)lds_addr);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(m0v), "v"(voffset), "s"(rsrc)
        : "memory", "m0");
}
// The same DMA split in two, so that each part can sit in its own gap between
// MFMAs: m0_set<OFF> writes M0 = base + OFF with one scalar instruction (base
// uniform, in an SGPR); dma16_issue then loads into LDS at M0.  The M0 write
// needs one wait state before the load, which the MFMA between them gives;
// nothing else in the main loop uses M0.
template <uint32_t OFF>
__device__ __forceinline__ void m0_set(uint32_t base)
{
    asm volatile("s_add_u32 m0, %0, %1" : : "s"(base), "i"(OFF) : "memory", "m0");
}
__device__ __forceinline__ void dma16_issue(const i32x4 &rsrc, int voffset)
{
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voffset), "s"(rsrc) : "memory");
}
#pragma clang diagnostic pop

// Waits until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order).  N is a compile-time constant.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    static_assert(N <= 16 || N == 18 || N == 20 || N == 24 || N == 28 || N == 30 || N == 32 || N == 36 ||
                      N == 40 || N == 42 || N == 48 || N == 54 || N == 56 || N == 60,
                  "add this vmcnt value to wait_vmcnt");
#define GE_VMCNT_CASE(n) \
    if constexpr (N == n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory");
    GE_VMCNT_CASE(0) GE_VMCNT_CASE(1) GE_VMCNT_CASE(2) GE_VMCNT_CASE(3) GE_VMCNT_CASE(4) GE_VMCNT_CASE(5)
    GE_VMCNT_CASE(6) GE_VMCNT_CASE(7) GE_VMCNT_CASE(8) GE_VMCNT_CASE(9) GE_VMCNT_CASE(10) GE_VMCNT_CASE(11)
    GE_VMCNT_CASE(12) GE_VMCNT_CASE(13) GE_VMCNT_CASE(14) GE_VMCNT_CASE(15) GE_VMCNT_CASE(16)
    GE_VMCNT_CASE(18) GE_VMCNT_CASE(20) GE_VMCNT_CASE(24) GE_VMCNT_CASE(28) GE_VMCNT_CASE(30)
    GE_VMCNT_CASE(32) GE_VMCNT_CASE(36) GE_VMCNT_CASE(40) GE_VMCNT_CASE(42) GE_VMCNT_CASE(48)
    GE_VMCNT_CASE(54) GE_VMCNT_CASE(56) GE_VMCNT_CASE(60)
#undef GE_VMCNT_CASE
}

// Workgroup barrier ordering LDS only: the fences are restricted to the LDS
// address space, so the wave waits for its own LDS operations but not for its
// outstanding global loads and stores (__syncthreads() would wait for those
// too).  Being compiler-visible, the fences also tell the wait-count pass
// that earlier LDS reads have completed.
__device__ __forceinline__ void barrier_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's LDS accesses before and after it.  Enough when a wave
// only reads LDS that it wrote itself (a wave's LDS operations execute in
// order).
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local"); }


__device__ __forceinline__ uint32_t lds_addr_of(const void *p)
{
    return (uint32_t)(uintptr_t)(const GE_LDS(char) *)p;
}

// ---------------------------------------------------------------------------
// Main loop of the 4-wave tiles (256 x 256, 128 x 256, 256 x 128, 128 x 128): one wave
// per SIMD, each owning a (BM/2) x (BN/2) accumulator tile held in the
// accumulation registers (AGPRs; for 256 x 256, 64 blocks of
// v_mfma_f32_16x16x32 and 256 fp32 values per lane).  Against eight waves of
// 64 x 128 the 256 x 256 tile reads a third fewer LDS bytes per MFMA (the
// operand bytes of a wave tile grow with its perimeter, the MFMAs with its
// area), which is what bounds the 8-wave loop.  The figures below are those
// of the 256 x 256 tile.
//
// With one wave per SIMD nothing else covers a stall, so the instruction
// stream is fixed by hand:
//  * K is walked in k steps of 32.  B arrives in 32-deep stages (32 k-rows
//    of 512 bytes) through a ring of 4 slots; A in 64-deep chunks (256 rows
//    of 128 bytes) through a ring of 3 slots.  A DMA instruction moves 1 KB;
//    its cost goes with the cache lines it touches, so A rows of a full
//    128-byte line (8 per instruction) cost half of 64-byte rows (16 half
//    lines), measured as a third of the DMA time of the 32-deep A stages.
//  * One barrier at the start of k step t publishes what k step t+1 reads
//    (B stage t+1; A chunk (t+1)/2) and frees what k step t has finished
//    reading.  Every k step issues 8 DMAs per wave: B stage t+4 into the B
//    slot of stage t, and half of A chunk (t+5)/2 into the slot of chunk
//    (t+5)/2 - 3.  Each lands three k steps (about 3k cycles) before it is
//    read, so one vmcnt value (16: the two newer steps' DMAs) serves every
//    wait.  Past the last stage the rings are still fed, with zero-record
//    descriptors, to keep that count.
//  * A slots sit in [0, 96 KB), B slots in [96 KB, 160 KB); every LDS read is
//    a base register plus an immediate offset below 64 KB.
//  * Each k step spreads its memory work over the gaps between its 64
//    MFMAs (about two instructions fit in the shadow of one): the 24 operand
//    reads of the next k step (8 A ds_read_b128, 16 B ds_read_b64_tr_b16),
//    evenly, and each of the 8 DMAs in three parts (descriptor, M0, issue)
//    in three consecutive gaps.  The order is pinned with scheduling
//    barriers.  Slots and register buffers repeat every 12 k steps, which
//    the loop unrolls.
//  * The MFMAs are inline asm with "+a" accumulator operands: with the
//    builtins the register allocator moved accumulators between the AGPR
//    and VGPR files inside the loop.  The hardware does not interlock an
//    MFMA result against a later non-MFMA reader and the compiler cannot see
//    inside the asm, so wait states are inserted by hand (agpr_fence).
// ---------------------------------------------------------------------------
constexpr int W4_BK = 32;      // k step, and the B stage depth
constexpr int W4_NS = 4;       // B ring slots
constexpr int W4_NA = 3;       // A ring slots
constexpr int W4_PERIOD = 12;  // k steps after which slots and buffers repeat

// k split of the 64 x 64 x 128 tile's main loop (the kernel says how)
inline constexpr int KS_SPLIT = 4, KS_WGM = 1, KS_WGN = 2;

// The tiles the 4-wave main loop runs: 256 x 256, 128 x 256, 256 x 128 and
// 128 x 128, four waves in a 2 x 2 grid, each owning a (BM/2) x (BN/2) tile
// of TM x TN 16 x 16 accumulator blocks.
template <int BM, int BN>
struct W4Cfg {
    static_assert((BM == 256 || BM == 128) && (BN == 256 || BN == 128), "4-wave tile");
    static constexpr int TM = BM / 32, TN = BN / 32;
    static constexpr int A_SLOT = BM * 128;        // a 64-deep A chunk: BM rows of 128 bytes
    static constexpr int B_ROW = BN * 2;           // bytes per B k-row
    static constexpr int B_CHUNKS = BN / 8;        // 16-byte chunks per B k-row
    static constexpr int B_SLOT = W4_BK * B_ROW;   // a 32-deep B stage
    static constexpr int B_BASE = W4_NA * A_SLOT;
    static constexpr int LDS = B_BASE + W4_NS * B_SLOT;
    static constexpr int NA = BM / 64;             // A DMAs per wave and k step (half a chunk)
    static constexpr int NB = BN / 64;             // B DMAs per wave and k step (one stage)
    static constexpr int ND = NA + NB;
    static constexpr int NMF = TM * TN;            // MFMAs per wave and k step
    static constexpr int NR = TM + 2 * TN;         // operand reads per wave and k step
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(NMF >= 2 * ND + 2 && NMF >= NR, "the gap schedule needs room");
};

template <bool W4, int BM, int BN>
constexpr int w4_lds()
{
    if constexpr (W4)
        return W4Cfg<BM, BN>::LDS;
    else
        return 0;
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

template <bool BF>
__device__ __forceinline__ void mfma16_agpr(f32x4 &acc, const half8 &a, const half8 &b)
{
    if constexpr (BF)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Orders every accumulator write before it against every access after it
// (each asm takes one row of accumulator blocks as in-out operands, in
// program order) and covers the last write with wait states: MFMAs in inline
// asm are opaque to the compiler's hazard recognizer, so the gap between a
// VALU write and an MFMA read, and between an MFMA result and an ordinary
// read, is inserted here.
template <int TM, int TN>
__device__ __forceinline__ void agpr_fence(f32x4 (&acc)[TM][TN])
{
    static_assert(TN == 4 || TN == 8, "rows of 4 or 8 blocks");
#pragma unroll
    for (int i = 0; i < TM; i++) {
        if constexpr (TN == 8) {
            if (i + 1 < TM)
                asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]),
                             "+a"(acc[i][4]), "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
            else
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                             : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]),
                               "+a"(acc[i][4]), "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
        } else {
            if (i + 1 < TM)
                asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]));
            else
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                             : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]));
        }
    }
}

template <int BM, int BN, bool BF>
__device__ __forceinline__ void mainloop_w4(f32x4 (&acc)[BM / 32][BN / 32], const _Float16 *Al, const _Float16 *Bl,
                                            int M, int N, int K, int KB, int m0, int n0, int kb, int nk, char *smem)
{
    using C = W4Cfg<BM, BN>;
    constexpr int TM = C::TM, TN = C::TN, NA = C::NA, NB = C::NB, ND = C::ND, NMF = C::NMF, NR = C::NR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    constexpr uint32_t kParked = 0x7FFFFFF0u;
    const uint32_t smem_lds = lds_addr_of(smem);
    const int kbase = kb * W4_BK;   // first k column of this segment
    const int nka = (nk + 1) >> 1;  // A chunks

    // DMA offsets.  A half-chunk h (rows BM/2 h .. BM/2 h + BM/2 - 1) is BM/16
    // instructions, NA per wave: instruction q of wave w fills rows
    // 8 (BM/16 h + 4q + w) .. + 7, lane -> row + lane / 8, physical chunk
    // lane % 8.  B stage: BN/16 instructions of 1 KB, NB per wave (block
    // 4q + w).
    uint32_t a_voff[2][NA], b_voff[NB];
    int a_kcol[2][NA];  // first k column of the lane's A chunk, for the chunk that crosses K
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int q = 0; q < NA; q++) {
            const int row = (h * (BM / 16) + q * 4 + wave) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz_a<8>(row);
            const int gm = m0 + row;
            a_kcol[h][q] = c * 8;
            a_voff[h][q] = gm < M ? (uint32_t)(gm * K + c * 8) * 2u : kParked;
        }
#pragma unroll
    for (int q = 0; q < NB; q++) {
        const int lin = (q * 4 + wave) * 64 + lane;
        const int krow = lin / C::B_CHUNKS;
        const int cb = (lin % C::B_CHUNKS) ^ swz_b<C::B_CHUNKS, 16>(krow);
        const int gn = n0 + cb * 8;
        b_voff[q] = gn < N ? (uint32_t)(krow * N + gn) * 2u : kParked;
    }
    const uint32_t lds_w = (uint32_t)__builtin_amdgcn_readfirstlane((int)(smem_lds + wave * 1024));
    // descriptors of B stage s and A chunk c (zero records past the end)
    auto rsrc_b = [&](int s) {
        const int k0 = kbase + s * W4_BK;
        return make_rsrc(Bl + (int64_t)k0 * N, s < nk ? (uint32_t)((int64_t)(KB - k0) * N * 2) : 0u);
    };
    auto rsrc_a = [&](int c) {
        const int k0 = kbase + c * 64;
        return make_rsrc(Al + k0, c < nka ? (uint32_t)(((int64_t)M * K - k0) * 2) : 0u);
    };
    // A offsets of the last chunk, the only one that can cross K (columns past
    // K are the next row's: parked)
    uint32_t a_voff_last[2][NA];
    {
        const int k0l = kbase + (nka - 1) * 64;
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int q = 0; q < NA; q++) a_voff_last[h][q] = k0l + a_kcol[h][q] < K ? a_voff[h][q] : kParked;
    }
    // LDS address (M0, less this wave's 1 KB) of DMA g of a k step: g < NA:
    // A instruction g of chunk half h into A slot sa; else B instruction g - NA
    // into B slot sb
    auto dma_lds = [](int g, int h, int sa, int sb) {
        return g < NA ? (uint32_t)(sa * C::A_SLOT + (h * (BM / 16) + g * 4) * 1024)
                      : (uint32_t)(C::B_BASE + sb * C::B_SLOT + (g - NA) * 4096);
    };

    // Operand reads.  A block i of k step t: lane (li + 16 lg) reads row
    // wm*BM/2 + 16 i + li, k columns 8 lg..8 lg+7 of the step's half of the
    // chunk (logical 16-byte chunk 4 (t & 1) + lg; one ds_read_b128).  The
    // swizzle depends on row bits 1-3, so block i is block 0 + 2 KB i, and the
    // step's half flips address bit 6.  B block j: two ds_read_b64_tr_b16,
    // lane 4e + r of 16-lane group g pointing at k-row 8 g + 4 h + e,
    // columns 4 r..4 r+3 of the block; h moves 4 k-rows (same swizzle), j has
    // its own address.
    const int li = lane & 15, lg = lane >> 4, lq = lane & 15;
    const int a_row = wm * (BM / 2) + li;
    const char *a_rd[W4_NA][2];
#pragma unroll
    for (int sl = 0; sl < W4_NA; sl++)
#pragma unroll
        for (int kk = 0; kk < 2; kk++)
            a_rd[sl][kk] = smem + sl * C::A_SLOT + a_row * 128 + (((kk * 4 + lg) ^ swz_a<8>(a_row)) * 16);
    const char *b_rd[TN];
#pragma unroll
    for (int j = 0; j < TN; j++) {
        const int n = wn * (BN / 2) + j * 16 + 4 * (lq & 3);
        const int krow = 8 * lg + (lq >> 2);
        b_rd[j] = smem + C::B_BASE + krow * C::B_ROW + (((n >> 3) ^ swz_b<C::B_CHUNKS, 16>(krow)) * 16) +
                  (n & 7) * 2;
    }
    auto read_a = [&](int sa, int kk, int i) { return *(const half8 *)(a_rd[sa][kk] + i * 2048); };
    auto read_b = [&](int sb, int j, int h) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (GE_LDS(fp16x4_t) *)(b_rd[j] + sb * C::B_SLOT + h * 4 * C::B_ROW));
    };

    half8 fa[2][TM], fb[2][TN];
    fp16x4_t fbh[TN][2];
    auto join_b = [&](int P) {
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const half4 lo = __builtin_bit_cast(half4, fbh[j][0]), hi = __builtin_bit_cast(half4, fbh[j][1]);
            fb[P][j] = half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    };
    // operand read r of a k step: A block, or half h of a B block; the first
    // 3 min(TM, TN) interleave A, B h0, B h1, the rest follow in order
    constexpr int MN = TM < TN ? TM : TN;
    // (all indices compile-time, so that the fragments stay in registers)
    auto do_read = [&](auto R_, auto P_, int sa, int kk, int sb) {
        constexpr int r = decltype(R_)::value, P = decltype(P_)::value;
        if constexpr (r < 3 * MN) {
            constexpr int g = r / 3, k = r % 3;
            if constexpr (k == 0)
                fa[P][g] = read_a(sa, kk, g);
            else
                fbh[g][k - 1] = read_b(sb, g, k - 1);
        } else if constexpr (TM > TN) {
            fa[P][MN + r - 3 * MN] = read_a(sa, kk, MN + r - 3 * MN);
        } else {
            constexpr int x = r - 3 * MN;
            fbh[MN + x / 2][x % 2] = read_b(sb, MN + x / 2, x % 2);
        }
    };

    // One k step t, t % 12 = D (compile time): MFMAs on the fragments in
    // buffer D % 2; operand reads of step t+1 into the other buffer; the ND
    // DMAs (B stage t+4, half (t+1) % 2 of A chunk (t+5)/2).  With one wave
    // per SIMD (two on the 128 x 128 tile, from two workgroups), only two or
    // three other instructions fit in the shadow of one MFMA, so the work is
    // spread over the NMF gaps after the MFMAs: read r in gap r NMF / NR; DMA
    // d in three gaps from d NMF / ND on (its A offset, M0, the load; the
    // MFMA between M0 and the load gives the wait state the load needs).
    // Near the end the DMAs fetch stages past the end (zero records) and the
    // last step's reads fetch into registers nobody uses: every branch stays
    // outside the pinned sequence.
    auto kstep = [&](auto D_, int t) {
        constexpr int D = decltype(D_)::value;
        constexpr int P = D & 1;
        constexpr int SB = D % W4_NS;                  // B slot of step t, refilled with stage t+4
        constexpr int SBN = (D + 1) % W4_NS;           // B slot of step t+1
        constexpr int SAN = ((D + 1) >> 1) % W4_NA;    // A slot of step t+1
        constexpr int KKN = (D + 1) & 1;               // its half of the chunk
        constexpr int SAD = ((D + 5) >> 1) % W4_NA;    // A slot refilled in this step
        constexpr int HD = (D + 1) & 1;                // the half refilled
        const int ca = (t + 5) >> 1;
        i32x4 ra, rb;  // built in the gaps of the first A and the first B DMA
        bool last_chunk;
        int dvoff[NA];
        // (static_for, not a pragma: a loop the unroller declines would index
        // the accumulators at run time and move them to scratch memory)
        static_for<NMF>([&](auto M_) {
            constexpr int m = decltype(M_)::value;
            mfma16_agpr<BF>(acc[m / TN][m % TN], fa[P][m / TN], fb[P][m % TN]);
            static_for<NR>([&](auto R_) {
                constexpr int r = decltype(R_)::value;
                if (r * NMF / NR == m) do_read(R_, std::integral_constant<int, P ^ 1>{}, SAN, KKN, SBN);
            });
            static_for<ND>([&](auto G_) {
                constexpr int g = decltype(G_)::value;
                constexpr int g0 = g * NMF / ND;
                if (m == g0) {
                    if constexpr (g == 0) {
                        ra = rsrc_a(ca);
                        last_chunk = ca == nka - 1;
                    }
                    if constexpr (g == NA) rb = rsrc_b(t + W4_NS);
                    if constexpr (g < NA) dvoff[g] = (int)(last_chunk ? a_voff_last[HD][g] : a_voff[HD][g]);
                } else if (m == g0 + 1) {
                    constexpr uint32_t OFF = g < NA ? (uint32_t)(SAD * C::A_SLOT + (HD * (BM / 16) + g * 4) * 1024)
                                                    : (uint32_t)(C::B_BASE + SB * C::B_SLOT + (g - NA) * 4096);
                    m0_set<OFF>(lds_w);
                } else if (m == g0 + 2) {
                    if constexpr (g < NA)
                        dma16_issue(ra, dvoff[g]);
                    else
                        dma16_issue(rb, (int)b_voff[g - NA]);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        join_b(P ^ 1);
    };

    // prologue, as virtual steps -5..-1 of the same pattern: A chunk 0 half 0;
    // then B stages 0..3 with A chunk 0 half 1, chunk 1, chunk 2 half 0
    {
        const i32x4 ra0 = rsrc_a(0), ra1 = rsrc_a(1), ra2 = rsrc_a(2);
        auto a_off = [&](int c, int h, int g) { return (int)(c == nka - 1 ? a_voff_last[h][g] : a_voff[h][g]); };
#pragma unroll
        for (int g = 0; g < NA; g++) dma16(ra0, lds_w + dma_lds(g, 0, 0, 0), a_off(0, 0, g));
#pragma unroll
        for (int s = 0; s < W4_NS; s++) {
            const i32x4 rb = rsrc_b(s);
            const int ca = (s + 1) >> 1, h = (s + 1) & 1;
            const i32x4 &ra = ca == 0 ? ra0 : (ca == 1 ? ra1 : ra2);
#pragma unroll
            for (int g = 0; g < ND; g++)
                dma16(g < NA ? ra : rb, lds_w + dma_lds(g, h, ca, s), g < NA ? a_off(ca, h, g) : (int)b_voff[g - NA]);
        }
    }
    wait_vmcnt<3 * ND>();  // B stage 0 and A chunk 0 (the DMAs of the three newer steps may fly)
    barrier_lds();
    static_for<NR>([&](auto R_) { do_read(R_, std::integral_constant<int, 0>{}, 0, 0, 0); });
    join_b(0);
    agpr_fence(acc);  // the accumulators' zeroing (VALU) before the first MFMA reads them

    // Step t: the DMAs of step t-3 have landed (those of the two newer steps
    // may still be in flight), then the barrier publishes what step t+1 reads
    // and frees the B slot that step t refills, which every wave read (for
    // step t) in step t-1.  The last step publishes nothing but still needs
    // the barrier: its DMAs (a stage past the end, zeros) write that slot,
    // and without it a fast wave zeroes operands a slow wave is still reading.
    auto step = [&](auto D_, int t) {
        wait_vmcnt<2 * ND>();
        barrier_lds();
        kstep(D_, t);
    };
#pragma unroll 1
    for (int t = 0; t < nk; t += W4_PERIOD) {
        step(std::integral_constant<int, 0>{}, t);
#define GE_W4_STEP(d) \
        if (t + d < nk) step(std::integral_constant<int, d>{}, t + d);
        GE_W4_STEP(1) GE_W4_STEP(2) GE_W4_STEP(3) GE_W4_STEP(4) GE_W4_STEP(5) GE_W4_STEP(6)
        GE_W4_STEP(7) GE_W4_STEP(8) GE_W4_STEP(9) GE_W4_STEP(10) GE_W4_STEP(11)
#undef GE_W4_STEP
    }
    // The DMAs of the last three steps (stages past the end: zero records, but
    // they still write their ring slots) may be in flight; the epilogue's
    // slabs reuse A slot 0, so they must have landed before its first write.
    wait_vmcnt<0>();
    agpr_fence(acc);  // the last MFMAs' results before the epilogue reads them
}


// ---------------------------------------------------------------------------
// Range-checked buffer loads and stores of the fast-path epilogue.  A lane
// whose element lies past the descriptor's record count reads zeros and its
// store is dropped by the buffer unit, so the epilogue needs no per-lane
// branch: with branches the compiler's wait-count pass lost track of the
// loads in flight and waited for all of them before every store.  AUX = 2
// marks the access non-temporal.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t epi_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
template <typename V, int AUX>
__device__ __forceinline__ V buf_load(__amdgpu_buffer_rsrc_t r, int off)
{
    if constexpr (sizeof(V) == 16)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    else if constexpr (sizeof(V) == 8)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
    else if constexpr (sizeof(V) == 4)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX));
    else
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX));
}
template <typename V, int AUX>
__device__ __forceinline__ void buf_store(V v, __amdgpu_buffer_rsrc_t r, int off)
{
    if constexpr (sizeof(V) == 16)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, AUX);
    else
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), r, off, 0, AUX);
}

// ---------------------------------------------------------------------------
// The kernel.  VEC = fast path (16-byte global->LDS DMA, 8-byte epilogue
// vectors); otherwise every global access is element-wise and guarded and
// LDS is filled through registers.
// ---------------------------------------------------------------------------
// The 16 bytes at byte offset b (0 or 2) of the 20 bytes lo:x.
__device__ __forceinline__ i32x4 realign16(const i32x4 &lo, int x, uint32_t b)
{
    const uint32_t d[5] = {(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)lo[2], (uint32_t)lo[3], (uint32_t)x};
    i32x4 r;
#pragma unroll
    for (int i = 0; i < 4; i++) r[i] = (int)__builtin_amdgcn_alignbyte(d[i + 1], d[i], b);
    return r;
}
// Keeps the first n 16-bit elements of v (none if n <= 0), zeroes the rest.
__device__ __forceinline__ i32x4 keep_first(i32x4 v, int n)
{
#pragma unroll
    for (int d = 0; d < 4; d++)
        v[d] &= (int)((2 * d < n ? 0x0000FFFFu : 0u) | (2 * d + 1 < n ? 0xFFFF0000u : 0u));
    return v;
}

template <int BM, int BN, int BK, int NSTAGES, int WGM, int WGN, int MI, int KIND, bool VEC, bool SK = false,
          bool BF = false, int EPI = EPI_AB>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_epi_kernel(Params p)
{
    constexpr int NW = WGM * WGN;                // waves per workgroup
    constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
    static_assert(MI == 32 || MI == 16, "MFMA block is 32x32x16 or 16x16x32");
    constexpr int TM = WM / MI, TN = WN / MI;    // MFMA blocks per wave
    constexpr int KSTEP = MI == 32 ? 16 : 32;    // k per MFMA
    constexpr int NACC = MI == 32 ? 16 : 4;      // accumulator registers per block
    using acc_t = typename std::conditional<MI == 32, f32x16, f32x4>::type;
    static_assert(TM >= 1 && TN >= 1, "tile too small");
    static_assert(BK == 32 || BK == 64 || BK == 128, "BK must be 32, 64 or 128");
    static_assert(NSTAGES >= 2, "at least two stages");
    constexpr int A_ROW = BK * 2;     // bytes per A row in LDS
    constexpr int A_CHUNKS = BK / 8;  // 16-byte chunks per A row
    constexpr int A_STAGE = BM * A_ROW;
    constexpr int B_ROW = BN * 2;     // bytes per B k-row in LDS
    constexpr int B_CHUNKS = BN / 8;
    constexpr int B_STAGE = BK * B_ROW;
    constexpr int STAGE = A_STAGE + B_STAGE;
    constexpr int MAIN_BYTES = NSTAGES * STAGE;
    // epilogue slab: one MFMA row-block (MI rows) of the wave tile in fp32.
    // LDS bank rules measured on gfx950 (bank-conflict counter, per-lane
    // address probes): 4-byte accesses serve 32 lanes per cycle and conflict
    // unless their words differ mod 32; 16-byte reads serve 32 lanes per
    // cycle and conflict unless their 4-word chunks differ mod 128 words.
    // Wave tiles up to 64 wide use an unpadded pitch, so that the rows one
    // 16-byte read covers (4 rows of 32, or 2 of 64) tile 128 words, and swap
    // the 16-word halves of rows 4..7 (mod 8), so that the rows r and r + 4
    // which one half-wave of accumulator stores writes land on opposite
    // halves of the 32 banks.  128-wide tiles keep a 4-word pad: each lane
    // reads 8 columns, and the pad interleaves adjacent rows' chunks.
    constexpr int SLAB = MI;
    constexpr bool SLAB_SWZ = WN <= 64;
    constexpr int EPI_LD = SLAB_SWZ ? WN : WN + (MI == 32 ? 8 : 4);
    constexpr int EPI_BYTES = NW * SLAB * EPI_LD * 4;
    // the 4-wave tiles (256 x 256, 128 x 256, 256 x 128, 128 x 128) run the
    // hand-scheduled main loop
    constexpr bool W4 = NW == 4 && BM >= 128 && BN >= 128 && BK == W4_BK && NSTAGES == W4_NS && MI == 16 && VEC && !SK;
    constexpr int W4_LDS = w4_lds<W4, BM, BN>();
    // The 64 x 64 x 128 tile splits the k range of every stage over its waves
    // in the main loop: KS_WGM x KS_WGN spatial groups, KS_SPLIT k groups.
    // Each wave reads a quarter of the stage's k range for a 64 x 32 block of
    // the tile: half the LDS fragment bytes of eight 16 x 32 wave tiles over
    // the whole range (1024 x 1024 x 4096: 12% faster; 1024^3: 3%).  The k
    // groups' partial sums meet in LDS, in a fixed order, before the
    // epilogue, which keeps the 4 x 2 grid of 16 x 32 wave tiles.
    constexpr bool KS = !W4 && BM == 64 && BN == 64 && BK == 128 && NW == 8 && MI == 16 && VEC && !SK;
    constexpr int KSPLIT = KS ? KS_SPLIT : 1;
    constexpr int ML_WGM = KS ? KS_WGM : WGM, ML_WGN = KS ? KS_WGN : WGN;
    static_assert(!KS || ML_WGM * ML_WGN * KSPLIT == NW, "k split covers the waves");
    constexpr int ML_WM = BM / ML_WGM, ML_WN = BN / ML_WGN;  // main-loop wave tile
    constexpr int ML_TM = ML_WM / MI, ML_TN = ML_WN / MI;
    constexpr int SMEM0 = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
    constexpr int SMEM = W4 ? (W4_LDS > EPI_BYTES ? W4_LDS : EPI_BYTES) : SMEM0;
    static_assert(SMEM <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    const int M = p.M, N = p.N, K = p.K;
    // B's rows per batch entry (the general path keeps K: the host sets b_rows
    // only for the fast path)
    const int KB = VEC && p.b_rows > 0 ? p.b_rows : K;
    const int nk_tile = (K + BK - 1) / BK;
    __shared__ int sk_ticket;

    // One segment: the k stages [kb, ke) of tile t = (l, tm, tn).  It ends
    // with the epilogue, unless it covers only part of the tile's k range
    // (stream-K), in which case it publishes its partial sum and only the
    // last contributor of the tile goes on to the epilogue.
    auto segment = [&](const int l, const int tm, const int tn, const int t, const int kb, const int ke,
                       const int lw) {
    const int m0 = tm * BM, n0 = tn * BN;
    const _Float16 *Al = p.A + (int64_t)l * M * K;
    const _Float16 *Bl = p.B + (int64_t)l * KB * N;

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < NACC; r++) acc[i][j][r] = 0.0f;
    // the main loop's accumulators: acc itself, or the k group's partial sums
    acc_t acc_ks[KS ? ML_TM : 1][KS ? ML_TN : 1];
    if constexpr (KS) {
#pragma unroll
        for (int i = 0; i < ML_TM; i++)
#pragma unroll
            for (int j = 0; j < ML_TN; j++)
#pragma unroll
                for (int r = 0; r < NACC; r++) acc_ks[i][j][r] = 0.0f;
    }
    auto &accm = [&]() -> auto & {
        if constexpr (KS)
            return acc_ks;
        else
            return acc;
    }();

    const int nk = ke - kb;  // k stages in this segment

    if constexpr (W4) {
        mainloop_w4<BM, BN, BF>(acc, Al, Bl, M, N, K, KB, m0, n0, kb, nk, smem);
    } else {
    // ---- global -> LDS --------------------------------------------------
    // One wave instruction fills 1 KB: 1024 / A_ROW rows of A, or
    // 1024 / B_ROW k-rows of B.  DMA_PER_STAGE = this thread's DMA
    // instructions per stage.
    constexpr int A_BLKS = A_STAGE / 1024;
    constexpr int B_BLKS = B_STAGE / 1024;
    constexpr int A_ROWS_PER_BLK = 1024 / A_ROW;
    constexpr int DMA_PER_STAGE = (A_BLKS + B_BLKS) / NW;
    static_assert(A_BLKS % NW == 0 && B_BLKS % NW == 0, "stage must split evenly over the waves");
    static_assert(B_ROW <= 1024 && 1024 % B_ROW == 0, "B row must divide 1 KB");

    // Fast-path DMA addressing.  Every DMA chunk of this thread sits at a
    // fixed byte offset from the first k column (A) / k-row (B) of its stage,
    // so the offsets are computed once; a stage moves the buffer base to its
    // k0 instead (a few scalar instructions) and shrinks the record count with
    // it.  Lanes outside M (A) or N (B) keep the offset 0x7FFFFFF0, beyond
    // every record count (one batch entry spans < 2^31 - 64 bytes), so they
    // read zeros at every stage.  B k-rows at or past K fall beyond the shrunk record count
    // by themselves; A k columns past K lie inside the buffer (they are the
    // next row), so a stage that crosses K takes per-lane checked offsets.
    constexpr int A_DMA = A_BLKS / NW, B_DMA = B_BLKS / NW;
    constexpr uint32_t kParked = 0x7FFFFFF0u;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t smem_lds = lds_addr_of(smem);
    uint32_t a_voff[A_DMA], b_voff[B_DMA];
    if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < A_DMA; q++) {
            const int row = (q * NW + wave) * A_ROWS_PER_BLK + lane / A_CHUNKS;
            const int c = (lane % A_CHUNKS) ^ swz_a<A_CHUNKS>(row);
            const int gm = m0 + row;
            a_voff[q] = gm < M ? (uint32_t)(gm * K + c * 8) * 2u : kParked;
        }
#pragma unroll
        for (int q = 0; q < B_DMA; q++) {
            const int lin = (q * NW + wave) * 64 + lane;  // chunk index within the stage
            const int krow = lin / B_CHUNKS;
            const int c = (lin % B_CHUNKS) ^ swz_b<B_CHUNKS, MI>(krow);
            const int gn = n0 + c * 8;
            b_voff[q] = gn < N ? (uint32_t)(krow * N + gn) * 2u : kParked;
        }
    }

    // General path (K or N not a multiple of 8, or an unaligned tensor):
    // global -> registers -> LDS, into the same swizzled layout.  Each thread
    // stages G_A + G_B 16-byte chunks a stage.  An operand of less than
    // 2 GiB is read with a 16-byte buffer load from the 4-byte aligned address
    // at or below the chunk and one more 4-byte load, and the chunk, at any
    // even byte offset, is cut out of
    // that window in registers (elements past K or N, and rows past M or K,
    // are zeroed); a larger operand is read element by element.  In the main
    // loop the loads of stage t+2 are issued before stage t's MFMAs and
    // written to LDS after its last MFMAs are issued, into the slot the
    // barrier before them freed, so that their latency hides behind a stage
    // of MFMAs and their realignment runs beside the MFMAs.
    constexpr int G_A = VEC ? 1 : A_BLKS / NW, G_B = VEC ? 1 : B_BLKS / NW;
    i32x4 g_lo[G_A + G_B];
    int g_hi[G_A + G_B];
    const uint32_t a_mis = (uint32_t)((uintptr_t)Al & 15), b_mis = (uint32_t)((uintptr_t)Bl & 15);
    const bool a_buf = (int64_t)M * K * 2 + 1024 < ((int64_t)1 << 31);
    const bool b_buf = (int64_t)K * N * 2 + 1024 < ((int64_t)1 << 31);
    const __amdgpu_buffer_rsrc_t g_ra =
        epi_rsrc((const char *)Al - a_mis, a_buf ? (uint32_t)((a_mis + (int64_t)M * K * 2 + 15) & ~15) : 0u);
    const __amdgpu_buffer_rsrc_t g_rb =
        epi_rsrc((const char *)Bl - b_mis, b_buf ? (uint32_t)((b_mis + (int64_t)K * N * 2 + 15) & ~15) : 0u);
    // chunk q of this thread: A row and k chunk, or B k-row and column chunk
    auto a_chunk = [&](int q, int &row, int &pchunk, int &c) {
        row = (q * NW + wave) * A_ROWS_PER_BLK + lane / A_CHUNKS;
        pchunk = lane % A_CHUNKS;
        c = pchunk ^ swz_a<A_CHUNKS>(row);
    };
    auto b_chunk = [&](int q, int &krow, int &pchunk, int &c) {
        const int lin = (q * NW + wave) * 64 + lane;
        krow = lin / B_CHUNKS;
        pchunk = lin % B_CHUNKS;
        c = pchunk ^ swz_b<B_CHUNKS, MI>(krow);
    };
    auto g_issue = [&](int k0) {
#pragma unroll
        for (int q = 0; q < G_A; q++) {
            int row, pchunk, c;
            a_chunk(q, row, pchunk, c);
            const int gm = m0 + row, gk = k0 + c * 8;
            if (a_buf) {
                const uint32_t byte = a_mis + (uint32_t)(((int64_t)gm * K + gk) * 2);
                const int off = gm < M ? (int)(byte & ~3u) : 0x7FFFFFE0;
                g_lo[q] = buf_load<i32x4, 0>(g_ra, off);
                g_hi[q] = buf_load<int, 0>(g_ra, off + 16);
            } else {
                half8 v;
#pragma unroll
                for (int e = 0; e < 8; e++)
                    v[e] = (gm < M && gk + e < K) ? Al[(int64_t)gm * K + gk + e] : (_Float16)0.0f;
                g_lo[q] = __builtin_bit_cast(i32x4, v);
            }
        }
#pragma unroll
        for (int q = 0; q < G_B; q++) {
            int krow, pchunk, c;
            b_chunk(q, krow, pchunk, c);
            const int gk = k0 + krow, gn = n0 + c * 8;
            if (b_buf) {
                const uint32_t byte = b_mis + (uint32_t)(((int64_t)gk * N + gn) * 2);
                const int off = gk < K ? (int)(byte & ~3u) : 0x7FFFFFE0;
                g_lo[G_A + q] = buf_load<i32x4, 0>(g_rb, off);
                g_hi[G_A + q] = buf_load<int, 0>(g_rb, off + 16);
            } else {
                half8 v;
#pragma unroll
                for (int e = 0; e < 8; e++)
                    v[e] = (gk < K && gn + e < N) ? Bl[(int64_t)gk * N + gn + e] : (_Float16)0.0f;
                g_lo[G_A + q] = __builtin_bit_cast(i32x4, v);
            }
        }
    };
    auto g_commit = [&](int stage, int k0) {
        const int a_off = stage * STAGE;
        const int b_off = a_off + A_STAGE;
#pragma unroll
        for (int q = 0; q < G_A; q++) {
            int row, pchunk, c;
            a_chunk(q, row, pchunk, c);
            const int gm = m0 + row, gk = k0 + c * 8;
            i32x4 v = g_lo[q];
            if (a_buf) v = realign16(g_lo[q], g_hi[q], (a_mis + (uint32_t)(((int64_t)gm * K + gk) * 2)) & 3u);
            *(i32x4 *)(smem + a_off + row * A_ROW + pchunk * 16) = keep_first(v, gm < M ? K - gk : 0);
        }
#pragma unroll
        for (int q = 0; q < G_B; q++) {
            int krow, pchunk, c;
            b_chunk(q, krow, pchunk, c);
            const int gk = k0 + krow, gn = n0 + c * 8;
            i32x4 v = g_lo[G_A + q];
            if (b_buf)
                v = realign16(g_lo[G_A + q], g_hi[G_A + q], (b_mis + (uint32_t)(((int64_t)gk * N + gn) * 2)) & 3u);
            *(i32x4 *)(smem + b_off + krow * B_ROW + pchunk * 16) = keep_first(v, gk < K ? N - gn : 0);
        }
    };

    auto load_stage = [&](int stage, int k0) {
        const int a_off = stage * STAGE;
        const int b_off = a_off + A_STAGE;
        if constexpr (VEC) {
            const uint32_t a_lds = smem_lds + a_off + wave_u * 1024;
            const uint32_t b_lds = smem_lds + b_off + wave_u * 1024;
            const i32x4 ra = make_rsrc(Al + k0, (uint32_t)(((int64_t)M * K - k0) * 2));
            const i32x4 rb = make_rsrc(Bl + (int64_t)k0 * N, (uint32_t)((int64_t)(KB - k0) * N * 2));
            if (k0 + BK <= K) {
#pragma unroll
                for (int q = 0; q < A_DMA; q++) dma16(ra, a_lds + q * NW * 1024, (int)a_voff[q]);
            } else {
#pragma unroll
                for (int q = 0; q < A_DMA; q++) {
                    const int row = (q * NW + wave) * A_ROWS_PER_BLK + lane / A_CHUNKS;
                    const int c = (lane % A_CHUNKS) ^ swz_a<A_CHUNKS>(row);
                    dma16(ra, a_lds + q * NW * 1024, (int)(k0 + c * 8 < K ? a_voff[q] : kParked));
                }
            }
#pragma unroll
            for (int q = 0; q < B_DMA; q++) dma16(rb, b_lds + q * NW * 1024, (int)b_voff[q]);
        } else {
            g_issue(k0);
            g_commit(stage, k0);
        }
    };

    // ---- LDS -> MFMA operand fragments -------------------------------------
    // A operand: lane (i + MI*g) holds row i of the block, k = 8g..8g+7 of the
    // k step (one ds_read_b128).  B operand: lane (j + MI*g) holds column j,
    // k = 8g..8g+7.  ds_read_b64_tr_b16 gives lane q of a 16-lane block the 4
    // values of column q from 4 k-rows, when lane 4e + r of the block points
    // at k-row e, columns 4r..4r+3; two such reads make one B operand.
    //  MI = 32: 16-lane block b covers columns 16*(b&1).., k-group g = b>>1.
    //  MI = 16: 16-lane block b covers the block's 16 columns, k-group g = b.
    const int li = lane % MI, lg = lane / MI;
    const int lb = lane >> 4, lq = lane & 15;
    // this wave's place in the main loop: its block of the tile, and its k
    // group (k steps ml_wk * KSTEPS .. ml_wk * KSTEPS + KSTEPS - 1 of every stage)
    constexpr int KSTEPS = BK / KSTEP / KSPLIT;
    const int ml_wk = KS ? wave / (ML_WGM * ML_WGN) : 0;
    const int ml_wm = KS ? wave % (ML_WGM * ML_WGN) / ML_WGN : wm;
    const int ml_wn = KS ? wave % ML_WGN : wn;
    auto read_frags = [&](int stage, int kk, half8 (&af)[ML_TM], half8 (&bf)[ML_TN]) {
        const char *a_src = smem + stage * STAGE;
        const char *b_src = a_src + A_STAGE;
        kk += ml_wk * KSTEPS;
#pragma unroll
        for (int i = 0; i < ML_TM; i++) {
            const int row = ml_wm * ML_WM + i * MI + li;
            const int c = (kk * (KSTEP / 8) + lg) ^ swz_a<A_CHUNKS>(row);
            af[i] = *(const half8 *)(a_src + row * A_ROW + c * 16);
        }
#pragma unroll
        for (int j = 0; j < ML_TN; j++) {
            const int n = MI == 32 ? ml_wn * ML_WN + j * 32 + 16 * (lb & 1) + 4 * (lq & 3)
                                   : ml_wn * ML_WN + j * 16 + 4 * (lq & 3);
            const int kgrp = MI == 32 ? (lb >> 1) : lb;
            half8 b;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int krow = kk * KSTEP + 8 * kgrp + 4 * h + (lq >> 2);
                const int c = (n >> 3) ^ swz_b<B_CHUNKS, MI>(krow);
                fp16x4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                    (GE_LDS(fp16x4_t) *)(b_src + krow * B_ROW + c * 16 + (n & 7) * 2));
                const half4 t4 = __builtin_bit_cast(half4, t);
                b[4 * h + 0] = t4[0];
                b[4 * h + 1] = t4[1];
                b[4 * h + 2] = t4[2];
                b[4 * h + 3] = t4[3];
            }
            bf[j] = b;
        }
    };

    auto mfmas = [&](const half8 (&af)[ML_TM], const half8 (&bf)[ML_TN]) {
#pragma unroll
        for (int i = 0; i < ML_TM; i++)
#pragma unroll
            for (int j = 0; j < ML_TN; j++) {
                if constexpr (BF) {
                    const bf16x8 a8 = __builtin_bit_cast(bf16x8, af[i]), b8 = __builtin_bit_cast(bf16x8, bf[j]);
                    if constexpr (MI == 32)
                        accm[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, accm[i][j], 0, 0, 0);
                    else
                        accm[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, accm[i][j], 0, 0, 0);
                } else if constexpr (MI == 32) {
                    accm[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], accm[i][j], 0, 0, 0);
                } else {
                    accm[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], accm[i][j], 0, 0, 0);
                }
            }
    };

    // Waits until this thread's DMA for the stage about to be published has
    // landed, when `newer` later stages (a compile-time count) may still be in
    // flight behind it; near the end of K fewer were issued, and it waits for
    // all.
    auto wait_stage = [&](auto newer, bool steady) {
        if constexpr (VEC) {
            if (steady)
                wait_vmcnt<decltype(newer)::value * DMA_PER_STAGE>();
            else
                wait_vmcnt<0>();
        }
    };
    using newer_prologue = std::integral_constant<int, NSTAGES - 1>;
    using newer_steady = std::integral_constant<int, NSTAGES - 2>;

    // ---- main loop ---------------------------------------------------------
    // A ring of NSTAGES LDS slots; stage j lives in slot j % NSTAGES.  Stages
    // 0..NSTAGES-1 are fetched up front; the barrier that publishes stage j
    // (everyone's DMA for it landed) also frees the slot of stage j-1, into
    // which stage j-1+NSTAGES is fetched right away.  Operand fragments are double-buffered in registers one
    // 16-wide k step ahead of the MFMAs; the barrier sits between the last
    // fragment reads of a stage and its last MFMAs, so the MFMA pipe keeps
    // working across it.
    half8 fa[2][ML_TM], fb[2][ML_TN];
#pragma unroll
    for (int st = 0; st < NSTAGES; st++)
        if (st < nk) load_stage(st, (kb + st) * BK);
    wait_stage(newer_prologue{}, nk >= NSTAGES);
    if constexpr (!VEC) __syncthreads();
    barrier_lds();
    read_frags(0, 0, fa[0], fb[0]);

    // Fragment buffers alternate with every k step across the whole K loop;
    // P (compile time) is the buffer holding the first k step of a stage.
    // When a stage has an odd number of k steps, P flips from stage to
    // stage, so the stage loop is unrolled by two.
    //
    // A stage that is followed by another: its last k step publishes the next
    // stage (barrier) and starts reading it before its own last MFMAs.
    auto stage_with_next = [&](int kt, int cur, int nxt, auto P) {
        constexpr int p0 = decltype(P)::value;
        if constexpr (!VEC)
            if (kt + NSTAGES < nk) g_issue((kb + kt + NSTAGES) * BK);
#pragma unroll
        for (int kk = 0; kk + 1 < KSTEPS; kk++) {
            read_frags(cur, kk + 1, fa[(p0 + kk + 1) & 1], fb[(p0 + kk + 1) & 1]);
            mfmas(fa[(p0 + kk) & 1], fb[(p0 + kk) & 1]);
        }
        wait_stage(newer_steady{}, kt + NSTAGES <= nk);  // stage kt+1 landed (this thread's part)
        if constexpr (!VEC) __syncthreads();
        barrier_lds();  // everyone's part landed; stage kt's slot is free
        if constexpr (VEC)
            if (kt + NSTAGES < nk) load_stage(cur, (kb + kt + NSTAGES) * BK);
        read_frags(nxt, 0, fa[(p0 + KSTEPS) & 1], fb[(p0 + KSTEPS) & 1]);
        mfmas(fa[(p0 + KSTEPS - 1) & 1], fb[(p0 + KSTEPS - 1) & 1]);
        if constexpr (!VEC)
            if (kt + NSTAGES < nk) g_commit(cur, (kb + kt + NSTAGES) * BK);
    };
    auto last_stage = [&](int cur, auto P) {
        constexpr int p0 = decltype(P)::value;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) {
            if (kk + 1 < KSTEPS) read_frags(cur, kk + 1, fa[(p0 + kk + 1) & 1], fb[(p0 + kk + 1) & 1]);
            mfmas(fa[(p0 + kk) & 1], fb[(p0 + kk) & 1]);
        }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    auto next_slot = [](int c) { return c + 1 == NSTAGES ? 0 : c + 1; };
    int cur = 0;  // ring slot of stage kt
    int kt = 0;
    if constexpr (KSTEPS % 2 == 0) {
#pragma unroll 1
        for (; kt + 1 < nk; kt++) {
            stage_with_next(kt, cur, next_slot(cur), P0{});
            cur = next_slot(cur);
        }
        last_stage(cur, P0{});
    } else {
#pragma unroll 1
        for (; kt + 2 < nk; kt += 2) {
            stage_with_next(kt, cur, next_slot(cur), P0{});
            cur = next_slot(cur);
            stage_with_next(kt + 1, cur, next_slot(cur), P1{});
            cur = next_slot(cur);
        }
        if (kt + 1 < nk) {  // two stages left: kt (buffer 0) and kt+1 (buffer 1)
            stage_with_next(kt, cur, next_slot(cur), P0{});
            cur = next_slot(cur);
            last_stage(cur, P1{});
        } else {            // one stage left, starting in buffer 0
            last_stage(cur, P0{});
        }
    }

    if constexpr (KS) {
        // The k groups' partial sums meet in LDS.  Block (rb, cb) of the tile
        // (MI x MI) of k group g is 1 KB at ((g * NBLK + rb * NBC + cb) * 64 +
        // lane) * 16 bytes, in the accumulator register layout: both the
        // stores and the loads move 1 KB per wave instruction, contiguous.
        // (Keeping each wave's own share of its epilogue blocks in registers
        // and storing only the rest measured no faster.)
        constexpr int NBC = BN / MI, NBLK = (BM / MI) * NBC;
        static_assert(KSPLIT * NBLK * 1024 <= (MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES), "LDS budget");
        float *red = (float *)smem;
        barrier_lds();  // every wave is done with the operand ring
#pragma unroll
        for (int i = 0; i < ML_TM; i++)
#pragma unroll
            for (int j = 0; j < ML_TN; j++) {
                const int b = ml_wk * NBLK + (ml_wm * ML_TM + i) * NBC + ml_wn * ML_TN + j;
                *(f32x4 *)(red + (b * 64 + lane) * 4) = accm[i][j];
            }
        barrier_lds();
        // the epilogue's wave tile (wm, wn): the sum over k groups 0, 1, .. in order
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int b = (wm * TM + i) * NBC + wn * TN + j;
                f32x4 v[KSPLIT];
#pragma unroll
                for (int g = 0; g < KSPLIT; g++) v[g] = *(const f32x4 *)(red + ((g * NBLK + b) * 64 + lane) * 4);
                acc[i][j] = v[0];
#pragma unroll
                for (int g = 1; g < KSPLIT; g++) acc[i][j] += v[g];
            }
    }

    }  // main loop (W4 or general)

    // ---- stream-K: partial sums of a split tile -------------------------------
    if constexpr (SK) {
        if (kb != 0 || ke != nk_tile) {
            constexpr int SLOT = BM * BN;  // floats
            const int64_t u0 = (int64_t)t * nk_tile;
            const int w_first = sk_owner(p, u0), w_last = sk_owner(p, u0 + nk_tile - 1);
            const int ncontrib = w_last - w_first + 1;
            // This contributor's sum in the accumulator register layout, 16 bytes
            // per lane and store: one instruction writes 1 KB, contiguous.  The
            // device-scope release fence makes it visible to every XCD before the
            // tile's counter is incremented; the last contributor's acquire fence
            // makes every contributor's sum visible to it.
            constexpr int NQ = NACC / 4;
            float *mine = p.partials + (int64_t)sk_slot(p, lw, t, nk_tile) * SLOT;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
#pragma unroll
                    for (int q = 0; q < NQ; q++) {
                        f32x4 v;
#pragma unroll
                        for (int e = 0; e < 4; e++) v[e] = acc[i][j][4 * q + e];
                        *(f32x4 *)(mine + ((((wave * TM + i) * TN + j) * NQ + q) * 64 + lane) * 4) = v;
                    }
            __threadfence();  // release (device scope)
            __syncthreads();
            if (tid == 0)
                sk_ticket = __hip_atomic_fetch_add(p.counters + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (sk_ticket != ncontrib - 1) return;  // another contributor finishes this tile
            __threadfence();  // acquire (device scope)
            // The sum in contributor (k) order, the same whichever contributor is
            // last.  All of one contributor's loads are issued before any add, so
            // each contributor costs one memory round trip, not one per load.
            for (int c = 0; c < ncontrib; c++) {
                const float *src = p.partials + (int64_t)sk_slot(p, w_first + c, t, nk_tile) * SLOT;
                f32x4 v[TM][TN][NQ];
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
#pragma unroll
                        for (int q = 0; q < NQ; q++)
                            v[i][j][q] = *(const f32x4 *)(src + ((((wave * TM + i) * TN + j) * NQ + q) * 64 + lane) * 4);
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
#pragma unroll
                        for (int q = 0; q < NQ; q++)
#pragma unroll
                            for (int e = 0; e < 4; e++)
                                acc[i][j][4 * q + e] = c == 0 ? v[i][j][q][e] : acc[i][j][4 * q + e] + v[i][j][q][e];
            }
            if (tid == 0)  // every contributor has arrived: ready for the next call
                __hip_atomic_store(p.counters + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // ---- epilogue ----------------------------------------------------------
    // The wave tile is handled one MFMA row-block (SLAB rows) at a time.  In a
    // slab, pass p covers rows 4p..4p+3; lane owns row 4p + lane/16 and CPL
    // consecutive columns from CPL*(lane%16) (+ a second group at WN/2 for a
    // 128-wide tile read 4 columns per lane).  A 32-wide wave tile has 8
    // lanes per row and covers rows 8p..8p+7 (lane_row below): with 16,
    // half the lanes would idle (64 x 64 tile: 4-13% faster launches).  CPL = 8 where the wave tile is
    // 128 wide: 16-byte loads and stores, half the vector memory instructions
    // of 4 columns per lane (measured 5% faster on the 16-batch products).  A
    // kind with the fp32 accumulator output keeps 4 columns per lane on the
    // 8-wave tiles: with 8, each 16-byte fp32 store instruction would fill
    // only half of every cache line it touches (measured 6% slower).  On the
    // 4-wave tiles with 128-wide wave tiles it takes 8 as well: with 4 their
    // epilogue runs out of VGPRs and spills.  C / X (and the column bias) of a slab are loaded
    // into registers one slab ahead, so the loads' latency hides behind the
    // previous slab's work; a lane's columns are the same in every slab, so its
    // row-bias values are loaded once.
    // With fp32 epilogue tensors a lane keeps 4 columns: 16-byte vectors again.
    constexpr bool F32E = EPI == EPI_F32;
    constexpr int CPL = WN % 128 == 0 && (!kind_has_acc_out(KIND) || W4) && !F32E ? 8 : 4;
    using E = EpiElem<BF, EPI>;
    using et = typename E::T;
    using hvec = typename std::conditional<F32E, f32x4,
                                           typename std::conditional<CPL == 8, half8, half4>::type>::type;
    const et *const pC = (const et *)p.C, *const pX = (const et *)p.X;
    const et *const prb = (const et *)p.row_bias, *const pcb = (const et *)p.col_bias;
    et *const pD = (et *)p.D, *const pAux = (et *)p.Aux;
    // A pass covers 64 / LPR consecutive slab rows with LPR lanes per row.
    constexpr int LPR = WN / CPL >= 16 ? 16 : WN / CPL;
    static_assert(LPR == 16 || (LPR == 8 && SLAB == 16), "epilogue lane mapping");
    constexpr int EPI_PASSES = SLAB * LPR / 64;
    constexpr int EPI_GROUPS = CPL == 4 && WN >= 128 ? 2 : 1;
    constexpr int EPI_HALF = WN / 2;
    constexpr bool HAS_C = kind_reads_c(KIND);
    constexpr bool HAS_X = kind_reads_x(KIND);
    constexpr bool HAS_BIAS = kind_reads_bias(KIND);
    constexpr int CP = HAS_C ? EPI_PASSES : 1, XP = HAS_X ? EPI_PASSES : 1, BP = HAS_BIAS ? EPI_PASSES : 1;
    const float alpha = p.alpha, beta = p.beta, s = p.s;
    const int64_t mn_base = (int64_t)l * M * N;
    auto lane_col = [&](int h) { return CPL * (lane % LPR) + h * EPI_HALF; };
    auto lane_row = [&](int pass) { return LPR == 8 ? pass * 8 + (lane >> 3) : pass * 4 + (lane >> 4); };
    // word index of (row, col) in a slab
    auto slab_at = [](int row, int col) { return row * EPI_LD + (SLAB_SWZ ? col ^ (((row >> 2) & 1) << 4) : col); };
    // Outputs are stored non-temporally (each is written once and never read
    // back here): they stream to HBM without taking L2 lines from the operand
    // panels (16-batch RELU_SQUARE 215 -> 183 us, 8192^3 LINCOMB_X_ACC -1%).
    // With two elementwise inputs (C and X) the loads are non-temporal too
    // (another -1%); with C alone that measured 5% slower than plain loads.
    //
    // The fast path addresses the tile's rows of each epilogue tensor through
    // a buffer descriptor whose record count ends at row min(M, m0 + BM):
    // rows past M are out of range by construction, and a lane whose columns
    // lie past N gets the parked offset (N % 8 == 0: a lane's columns are all
    // in or all out).  The host keeps BM * N * 4 bytes below the parked offset.
    constexpr int LD_AUX = HAS_X ? 2 : 0;
    const int rows_here = min(M - m0, BM);
    const int64_t tbase = mn_base + (int64_t)m0 * N;  // element offset of the tile's first row
    const uint32_t ebytes = (uint32_t)rows_here * (uint32_t)N * (uint32_t)sizeof(et);
    const __amdgpu_buffer_rsrc_t rC = epi_rsrc(pC + tbase, ebytes), rX = epi_rsrc(pX + tbase, ebytes);
    const __amdgpu_buffer_rsrc_t rD = epi_rsrc(pD + tbase, ebytes), rAux = epi_rsrc(pAux + tbase, ebytes);
    const __amdgpu_buffer_rsrc_t rAcc = epi_rsrc(p.acc_out + tbase, (uint32_t)rows_here * (uint32_t)N * 4u);
    // byte offset of (slab i, pass, column group h) within the tile's rows, or parked
    auto epi_off = [&](int i, int pass, int h, int es) {
        const int gn = n0 + wn * WN + lane_col(h);
        const int off = ((wm * WM + i * SLAB + lane_row(pass)) * N + gn) * es;
        const int out = -(int)(gn >= N);  // all ones past N (a mask, not a branch)
        return (off & ~out) | ((int)0x7FFFFFF0 & out);
    };
    // C of every slab is loaded at once when the epilogue starts (the operand
    // fragment registers are free by then): more loads in flight.  X and the
    // column bias go EPD slabs ahead, and so does C when it is fp32 (all of it
    // would take 128 registers) or when the wave tile has 8 slabs (the 4-wave
    // tiles 256 rows tall: 128 registers again).  EPD is 1 on the 8-wave
    // tiles, whose two waves per SIMD overlap each other's loads; the 4-wave
    // tiles keep 3 slabs of C and X in flight (one wave per SIMD, or two from
    // two workgroups on 128 x 128).
    constexpr bool PRE_C = VEC && HAS_C && !F32E && TM <= 4;
    constexpr int EPD = W4 ? 3 : 1;
    constexpr int NBX = EPD + 1;
    constexpr int NBC = PRE_C ? TM : NBX;
    hvec cbuf[NBC][CP][EPI_GROUPS];
    hvec xbuf[NBX][XP][EPI_GROUPS];
    et cbias[NBX][BP];
    auto cslot = [](int i) { return PRE_C ? i : i % NBX; };
    hvec rbias[EPI_GROUPS];
    const __amdgpu_buffer_rsrc_t rcb = epi_rsrc(pcb, (uint32_t)M * sizeof(et));
    const __amdgpu_buffer_rsrc_t rrb = epi_rsrc(prb, (uint32_t)N * sizeof(et));
    // loads slab i's C (with_c) and its X and column bias (with_x)
    auto epi_prefetch = [&](int i, hvec (&cb)[CP][EPI_GROUPS], hvec (&xb)[XP][EPI_GROUPS], et (&colb)[BP],
                            bool with_c, bool with_x) {
#pragma unroll
        for (int pass = 0; pass < EPI_PASSES; pass++) {
            const int gm = m0 + wm * WM + i * SLAB + lane_row(pass);
            if constexpr (HAS_BIAS)  // one value per row, zero past M
                if (with_x) colb[pass] = buf_load<et, 0>(rcb, gm * (int)sizeof(et));
#pragma unroll
            for (int h = 0; h < EPI_GROUPS; h++) {
                const int off = epi_off(i, pass, h, (int)sizeof(et));
                if constexpr (HAS_C)
                    if (with_c) cb[pass][h] = buf_load<hvec, LD_AUX>(rC, off);
                if constexpr (HAS_X)
                    if (with_x) xb[pass][h] = buf_load<hvec, LD_AUX>(rX, off);
            }
        }
    };

    // the first slab's loads fly while the accumulators go to LDS
    if constexpr (VEC) {
        if constexpr (HAS_BIAS) {
#pragma unroll
            for (int h = 0; h < EPI_GROUPS; h++) {
                const int gn = n0 + wn * WN + lane_col(h);
                rbias[h] = buf_load<hvec, 0>(rrb, gn < N ? gn * (int)sizeof(et) : (int)0x7FFFFFF0);
            }
        }
#pragma unroll
        for (int i = 0; i < EPD && i < TM; i++) epi_prefetch(i, cbuf[cslot(i)], xbuf[i], cbias[i], true, true);
        if constexpr (PRE_C) {
#pragma unroll
            for (int i = EPD; i < TM; i++) epi_prefetch(i, cbuf[i], xbuf[EPD], cbias[EPD], true, false);
        }
    }
    barrier_lds();  // every wave is done with the main loop's LDS, which the epilogue reuses

    float *slab = (float *)(smem + wave * (SLAB * EPI_LD * 4));
#pragma unroll
    for (int i = 0; i < TM; i++) {  // fully unrolled: acc must stay in registers
        // acc block row i of this wave -> its LDS slab (SLAB x WN fp32).  Output
        // layouts: MI = 32: lane l, register r holds row 8(r/4) + 4(l/32) + r%4,
        // column l%32; MI = 16: row 4(l/16) + r, column l%16.
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < NACC; r++) {
                const int row = MI == 32 ? 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) : 4 * (lane >> 4) + r;
                const int col = j * MI + (lane % MI);
                slab[slab_at(row, col)] = acc[i][j][r];
            }
        wave_lds_sync();  // each wave reads back only its own slab
        if constexpr (VEC) {
            if (i + EPD < TM)
                epi_prefetch(i + EPD, cbuf[cslot(i + EPD)], xbuf[(i + EPD) % NBX], cbias[(i + EPD) % NBX], !PRE_C,
                             true);
        }
#pragma unroll
        for (int pass = 0; pass < EPI_PASSES; pass++) {
            const int srow = lane_row(pass);
            const int gm = m0 + wm * WM + i * SLAB + srow;
#pragma unroll
            for (int h = 0; h < EPI_GROUPS; h++) {
                const int scol = lane_col(h);
                if (scol >= WN) continue;
                const int gn = n0 + wn * WN + scol;
                float av[CPL];
#pragma unroll
                for (int q = 0; q < CPL / 4; q++) {
                    const f32x4 a4 = *(const f32x4 *)(slab + slab_at(srow, scol + 4 * q));
#pragma unroll
                    for (int e = 0; e < 4; e++) av[4 * q + e] = a4[e];
                }
                if constexpr (VEC) {
                    hvec c4 = {}, x4 = {}, rb4 = {};
                    float cbv = 0.0f;
                    if constexpr (HAS_C) c4 = cbuf[cslot(i)][pass][h];
                    if constexpr (HAS_X) x4 = xbuf[i % NBX][pass][h];
                    if constexpr (HAS_BIAS) {
                        rb4 = rbias[h];
                        cbv = E::ld(cbias[i % NBX][pass]);
                    }
                    hvec d4, e4;
#pragma unroll
                    for (int e = 0; e < CPL; e++) {
                        float d, a = 0.0f;
                        epi_elem<KIND>(av[e], E::ld(c4[e]), E::ld(x4[e]), E::ld(rb4[e]), cbv, alpha, beta, s, d, a);
                        d4[e] = E::st(d);
                        e4[e] = E::st(a);
                    }
                    const int off = epi_off(i, pass, h, (int)sizeof(et));
                    if constexpr (kind_writes_d(KIND)) buf_store<hvec, 2>(d4, rD, off);
                    if constexpr (kind_has_aux(KIND)) buf_store<hvec, 2>(e4, rAux, off);
                    if constexpr (kind_has_acc_out(KIND)) {
                        const int off4 = epi_off(i, pass, h, 4);
#pragma unroll
                        for (int q = 0; q < CPL / 4; q++)
                            buf_store<f32x4, 2>(f32x4{av[4 * q], av[4 * q + 1], av[4 * q + 2], av[4 * q + 3]}, rAcc,
                                                off4 < 0x7FFFFFF0 ? off4 + 16 * q : off4);
                    }
                } else {
                    if (gm >= M) continue;
                    const int64_t o = mn_base + (int64_t)gm * N + gn;
                    const float cbv = HAS_BIAS ? E::ld(pcb[gm]) : 0.0f;
#pragma unroll
                    for (int e = 0; e < CPL; e++) {
                        if (gn + e >= N) break;
                        const float c = HAS_C ? E::ld(pC[o + e]) : 0.0f;
                        const float x = HAS_X ? E::ld(pX[o + e]) : 0.0f;
                        const float rb = HAS_BIAS ? E::ld(prb[gn + e]) : 0.0f;
                        float d, a = 0.0f;
                        epi_elem<KIND>(av[e], c, x, rb, cbv, alpha, beta, s, d, a);
                        if constexpr (kind_writes_d(KIND)) pD[o + e] = E::st(d);
                        if constexpr (kind_has_aux(KIND)) pAux[o + e] = E::st(a);
                        if constexpr (kind_has_acc_out(KIND)) p.acc_out[o + e] = av[e];
                    }
                }
            }
        }
        wave_lds_sync();  // slab reads done before the next block row overwrites it
        // 4-wave tile: keep the next block row's accumulator reads (AGPR ->
        // VGPR) from being hoisted above this one, which runs out of VGPRs
        if constexpr (W4) __builtin_amdgcn_sched_barrier(0);
    }
    };  // segment

    if constexpr (!SK) {
        int l, tm, tn;
        map_tile(p, l, tm, tn);
        segment(l, tm, tn, 0, 0, nk_tile, 0);
    } else {
        // stream-K: this workgroup's contiguous range of (tile, k stage) units
        const int lw = xcd_logical_id(gridDim.x, blockIdx.x);
        int64_t u = sk_begin(p, lw);
        const int64_t ue = sk_begin(p, lw + 1);
        while (u < ue) {
            const int t = (int)(u / nk_tile);
            const int kb = (int)(u - (int64_t)t * nk_tile);
            const int ke = (int)min((int64_t)nk_tile, (int64_t)kb + (ue - u));
            int l, tm, tn;
            tile_coords(p, t, l, tm, tn);
            segment(l, tm, tn, t, kb, ke, lw);
            u += ke - kb;
            __syncthreads();  // LDS free before the next segment's DMA
        }
    }
}

// ---------------------------------------------------------------------------
// The elementwise stage of the unfused composition: the same epilogue math on
// an fp32 accumulator that a separate GEMM launch wrote to HBM.  It exists to
// measure what the fusion saves (one more launch, the accumulator's write and
// read); its results equal the fused kernel's bit for bit.  One row of one
// batch entry per iteration of a block, so a lane knows its row and column
// without a division; VEC: 4 consecutive columns per lane (N % 4 == 0,
// 16-byte aligned accumulator, 8-byte aligned 16-bit tensors).  BF: the
// 16-bit tensors are bfloat16.
// ---------------------------------------------------------------------------
struct EpiParams {
    const float *acc;  // (L, M, N) fp32 accumulator
    const _Float16 *C;
    const _Float16 *X;
    const _Float16 *row_bias;
    const _Float16 *col_bias;
    _Float16 *D;
    _Float16 *Aux;
    int64_t rows;  // L * M
    int M, N;
    float alpha, beta, s;
};

template <int KIND, bool VEC, bool BF = false>
__global__ __launch_bounds__(256) void epilogue_kernel(EpiParams q)
{
    const float alpha = q.alpha, beta = q.beta, s = q.s;
    for (int64_t row = blockIdx.x; row < q.rows; row += gridDim.x) {
        const int m = (int)(row % q.M);
        const int64_t base = row * q.N;
        const float cbv = kind_reads_bias(KIND) ? ld16<BF>(q.col_bias[m]) : 0.0f;
        if constexpr (VEC) {
            for (int n = 4 * threadIdx.x; n < q.N; n += 4 * blockDim.x) {
                const int64_t o = base + n;
                const f32x4 a4 = *(const f32x4 *)(q.acc + o);
                half4 c4 = {}, x4 = {}, rb4 = {};
                if constexpr (kind_reads_c(KIND)) c4 = *(const half4 *)(q.C + o);
                if constexpr (kind_reads_x(KIND)) x4 = *(const half4 *)(q.X + o);
                if constexpr (kind_reads_bias(KIND)) rb4 = *(const half4 *)(q.row_bias + n);
                half4 d4, e4;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    float d, a = 0.0f;
                    epi_elem<KIND>(a4[e], ld16<BF>(c4[e]), ld16<BF>(x4[e]), ld16<BF>(rb4[e]), cbv, alpha, beta, s, d,
                                   a);
                    d4[e] = st16<BF>(d);
                    e4[e] = st16<BF>(a);
                }
                *(half4 *)(q.D + o) = d4;
                if constexpr (kind_has_aux(KIND)) *(half4 *)(q.Aux + o) = e4;
            }
        } else {
            for (int n = threadIdx.x; n < q.N; n += blockDim.x) {
                const int64_t o = base + n;
                const float c = kind_reads_c(KIND) ? ld16<BF>(q.C[o]) : 0.0f;
                const float x = kind_reads_x(KIND) ? ld16<BF>(q.X[o]) : 0.0f;
                const float rb = kind_reads_bias(KIND) ? ld16<BF>(q.row_bias[n]) : 0.0f;
                float d, a = 0.0f;
                epi_elem<KIND>(q.acc[o], c, x, rb, cbv, alpha, beta, s, d, a);
                q.D[o] = st16<BF>(d);
                if constexpr (kind_has_aux(KIND)) q.Aux[o] = st16<BF>(a);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Staging copies of the workspace path.  A tensor that breaks the fast
// path's layout rules (a row length that is not a multiple of 8 elements, or
// a base address that is not 16-byte aligned) is copied into an aligned
// buffer whose rows are padded with zeros to a multiple of 8 elements, and an
// output is written there and copied back afterwards.  Pure copies of raw
// element bits (T: 2 or 4 bytes) at any element-aligned address, one row of
// one batch entry per iteration of a block.
// ---------------------------------------------------------------------------
struct StageCopy {
    const void *src;
    void *dst;
    int64_t L;
    int64_t rows, cols;  // the unpadded tensor (L, rows, cols)
    int64_t prows, pcols;  // the padded one: prows >= rows, pcols >= cols
};

// The copies of one call go in one launch: blockIdx.y picks the tensor.
constexpr int kMaxStageCopies = 5;
struct StageCopies {
    StageCopy c[kMaxStageCopies];
};

// Both copies move one element per lane and access, adjacent lanes on
// adjacent elements, so each wave access covers one contiguous span (128
// bytes of 2-byte elements) whatever the rows' alignment; four accesses per
// lane are in flight at a time.
constexpr int kStageUnroll = 4;

// padded (L, prows, pcols) <- src (L, rows, cols), zeros past rows and cols
// (q.dst).
template <typename T>
__global__ __launch_bounds__(256) void stage_pad_kernel(StageCopies qs)
{
    const StageCopy &q = qs.c[blockIdx.y];
    const int64_t nrows = q.L * q.prows;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t l = row / q.prows, r = row - l * q.prows;
        const int64_t cols = r < q.rows ? q.cols : 0;  // source elements in this row
        const T *s = (const T *)q.src + (l * q.rows + (r < q.rows ? r : 0)) * q.cols;
        T *d = (T *)q.dst + row * q.pcols;
        for (int64_t c0 = threadIdx.x; c0 < q.pcols; c0 += 256 * kStageUnroll) {
            T v[kStageUnroll];
#pragma unroll
            for (int u = 0; u < kStageUnroll; u++) {
                const int64_t c = c0 + 256 * u;
                v[u] = c < cols ? s[c] : (T)0;
            }
#pragma unroll
            for (int u = 0; u < kStageUnroll; u++) {
                const int64_t c = c0 + 256 * u;
                if (c < q.pcols) d[c] = v[u];
            }
        }
    }
}

// dst (L, rows, cols) <- the first rows and cols of padded (L, prows, pcols)
// (q.src).
template <typename T>
__global__ __launch_bounds__(256) void stage_unpad_kernel(StageCopies qs)
{
    const StageCopy &q = qs.c[blockIdx.y];
    const int64_t nrows = q.L * q.rows;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t l = row / q.rows, r = row - l * q.rows;
        const T *s = (const T *)q.src + (l * q.prows + r) * q.pcols;
        T *d = (T *)q.dst + row * q.cols;
        for (int64_t c0 = threadIdx.x; c0 < q.cols; c0 += 256 * kStageUnroll) {
            T v[kStageUnroll];
#pragma unroll
            for (int u = 0; u < kStageUnroll; u++) {
                const int64_t c = c0 + 256 * u;
                v[u] = c < q.cols ? s[c] : (T)0;
            }
#pragma unroll
            for (int u = 0; u < kStageUnroll; u++) {
                const int64_t c = c0 + 256 * u;
                if (c < q.cols) d[c] = v[u];
            }
        }
    }
}

}  // namespace gemm_epi
