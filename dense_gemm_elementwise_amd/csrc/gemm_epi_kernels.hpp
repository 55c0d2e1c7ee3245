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
//  * 256 threads = 4 wave64s in a 2 x 2 grid; each wave owns a
//    (BM/2) x (BN/2) accumulator tile built from v_mfma_f32_32x32x16_f16.
//  * K is walked in steps of BK = 64 through two LDS stages.  The fast path
//    fills LDS with buffer_load_dwordx4 ... lds (global -> LDS without
//    VGPRs); lanes whose 16-byte chunk lies outside the matrix get an
//    out-of-range offset, which the buffer unit turns into zeros, so M, N and
//    K tails need no extra code in the inner loop.
//  * A tiles are stored row-major (128 B per row); B tiles k-row-major.  The
//    16-byte chunks of each row are XOR-swizzled so that the MFMA operand
//    reads (ds_read_b128 for A, ds_read_b64_tr_b16 for B, which transposes
//    the N-contiguous B rows into the K-contiguous operand on the fly) hit
//    distinct banks.
//  * The epilogue moves each wave's accumulator through LDS so that every
//    lane owns 4 consecutive columns; C / X are then read and D / Aux written
//    with 8-byte vectors, one pass, predicated at the M / N edges.
//  * Workgroup ids are remapped so that the tiles one XCD runs together are
//    neighbours (they share A row panels and B column panels in that XCD's
//    L2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm_epi {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define GE_LDS(T) __attribute__((address_space(3))) T

enum Kind : int { LINCOMB = 0, AUX_SCALE = 1, LINCOMB_X_ACC = 2, RELU = 3, SQUARE = 4, RELU_SQUARE = 5 };

__host__ __device__ constexpr bool kind_has_aux(int k)
{
    return k == AUX_SCALE || k == LINCOMB_X_ACC || k == SQUARE || k == RELU_SQUARE;
}
__host__ __device__ constexpr bool kind_reads_x(int k) { return k == LINCOMB_X_ACC; }

struct Params {
    const _Float16 *A;
    const _Float16 *B;
    const _Float16 *C;
    const _Float16 *X;
    _Float16 *D;
    _Float16 *Aux;
    int M, N, K;      // each < 2^31 (checked on the host)
    int tiles_m, tiles_n;
    int num_tiles;    // L * tiles_m * tiles_n
    float alpha, beta, s;
};

constexpr int BK = 64;          // K step per LDS stage
constexpr int NTHREADS = 256;   // 4 waves
constexpr int GROUP_M = 4;      // tile rows per L2 group

// ---------------------------------------------------------------------------
// Epilogue math, fp32.  d = first output, a = second output (if any).
// ---------------------------------------------------------------------------
template <int KIND>
__device__ __forceinline__ void epi_elem(float acc, float c, float x, float alpha, float beta, float s, float &d,
                                         float &a)
{
    if constexpr (KIND == LINCOMB) {
        d = alpha * acc + beta * c;
    } else if constexpr (KIND == AUX_SCALE) {
        float t = alpha * acc + beta * c;
        a = t;
        d = s * t;
    } else if constexpr (KIND == LINCOMB_X_ACC) {
        a = acc;
        d = (alpha * acc + beta * c) + s * x;
    } else if constexpr (KIND == RELU) {
        float t = alpha * acc + beta * c;
        d = t > 0.0f ? t : 0.0f;
    } else if constexpr (KIND == SQUARE) {
        float t = alpha * acc + beta * c;
        d = t;
        a = t * t;
    } else {  // RELU_SQUARE
        float t = alpha * acc + beta * c;
        t = t > 0.0f ? t : 0.0f;
        d = t;
        a = t * t;
    }
}

// ---------------------------------------------------------------------------
// Tile scheduling: hardware workgroup id -> (batch, tile row, tile column).
// Workgroups are handed to the 8 XCDs round-robin (id % 8), so consecutive
// logical tiles are given to ids that land on the same XCD; within a batch
// entry tiles are ordered in groups of GROUP_M tile rows, column-major inside
// a group, so the tiles an XCD runs together share operand panels.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void map_tile(const Params &p, int &l, int &tm, int &tn)
{
    const int nwg = p.num_tiles;
    const int w = blockIdx.x;
    const int xcd = w & 7, j = w >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    const int t = xcd * per + (xcd < rem ? xcd : rem) + j;
    const int tpb = p.tiles_m * p.tiles_n;
    l = t / tpb;
    const int r = t - l * tpb;
    const int gsize_full = GROUP_M * p.tiles_n;
    const int g = r / gsize_full;
    const int first_m = g * GROUP_M;
    const int gm = min(p.tiles_m - first_m, GROUP_M);
    const int rr = r - g * gsize_full;
    tm = first_m + rr % gm;
    tn = rr / gm;
}

// Swizzles (in 16-byte chunk units).  A rows hold 8 chunks; row r stores
// logical chunk c at physical chunk c ^ swz_a(r).  B k-rows hold BN/8 chunks;
// k-row kr stores logical chunk c at c ^ swz_b(kr).  Both keep every MFMA
// operand read conflict-free whether the LDS serves 128 or 256 bytes a clock:
// an A read has 16 consecutive rows at one logical chunk, a B transpose read
// has 4 consecutive k-rows x 4 consecutive chunks.
__device__ __forceinline__ int swz_a(int row) { return (row & 7) ^ ((row >> 3) & 1); }
template <int B_CHUNKS>
__device__ __forceinline__ int swz_b(int krow)
{
    if constexpr (B_CHUNKS >= 16)
        return (0xCA60 >> ((krow & 3) * 4)) & 15;  // 0, 6, 10, 12 for krow % 4 = 0..3
    else
        return 2 * (krow & 3);                     // 8-chunk rows: 0, 2, 4, 6
}

// ---------------------------------------------------------------------------
// 16-byte global -> LDS DMA: buffer_load_dwordx4 ... lds writes lane i's 16
// bytes to LDS address M0 + 16*i.  Written as inline asm so that the compiler
// does not treat every later LDS read as dependent on it (it would otherwise
// wait for all outstanding DMA before each read, which serialises the
// prefetch with the MFMA work); the kernel waits for the DMA itself
// (s_waitcnt vmcnt(0) before the barrier that publishes a stage).
// ---------------------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));

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
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr_of(const void *p)
{
    return (uint32_t)(uintptr_t)(const GE_LDS(char) *)p;
}

// ---------------------------------------------------------------------------
// The kernel.  VEC = fast path (16-byte global->LDS DMA, 8-byte epilogue
// vectors); otherwise every global access is element-wise and guarded and
// LDS is filled through registers.
// ---------------------------------------------------------------------------
template <int BM, int BN, int KIND, bool VEC>
__global__ __launch_bounds__(NTHREADS) void gemm_epi_kernel(Params p)
{
    constexpr int WM = BM / 2, WN = BN / 2;    // wave tile
    constexpr int TM = WM / 32, TN = WN / 32;  // 32x32 MFMA blocks per wave
    static_assert(TM >= 1 && TN >= 1, "tile too small");
    constexpr int A_STAGE = BM * BK * 2;  // bytes
    constexpr int B_STAGE = BK * BN * 2;
    constexpr int STAGE = A_STAGE + B_STAGE;
    constexpr int B_ROW = BN * 2;  // bytes per B k-row in LDS
    constexpr int MAIN_BYTES = 2 * STAGE;
    constexpr int EPI_LD = WN + 8;  // fp32 row pitch of an epilogue slab
    constexpr int EPI_BYTES = 4 * 32 * EPI_LD * 4;
    constexpr int SMEM = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int l, tm, tn;
    map_tile(p, l, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    const _Float16 *Al = p.A + (int64_t)l * M * K;
    const _Float16 *Bl = p.B + (int64_t)l * K * N;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    const int nk = (K + BK - 1) / BK;

    // ---- global -> LDS --------------------------------------------------
    // A: BM rows x 8 chunks; one wave instruction fills 1 KB = 8 rows.
    // B: BK k-rows x BN/8 chunks; one wave instruction fills 1 KB.
    constexpr int A_BLKS = A_STAGE / 1024;
    constexpr int B_BLKS = B_STAGE / 1024;
    constexpr int B_CHUNKS = BN / 8;
    static_assert(A_BLKS % 4 == 0 && B_BLKS % 4 == 0, "stage must split evenly over 4 waves");
    static_assert(B_ROW <= 1024 && 1024 % B_ROW == 0, "B row must divide 1 KB");

    i32x4 rsrc_a = {}, rsrc_b = {};
    if constexpr (VEC) {
        // one buffer per batch entry; every offset is < 2^31 (checked on the host)
        rsrc_a = make_rsrc(Al, (uint32_t)((int64_t)M * K * 2));
        rsrc_b = make_rsrc(Bl, (uint32_t)((int64_t)K * N * 2));
    }
    const uint32_t smem_lds = lds_addr_of(smem);

    auto load_stage = [&](int stage, int k0) {
        const int a_off = stage * STAGE;
        const int b_off = a_off + A_STAGE;
        if constexpr (VEC) {
#pragma unroll
            for (int q = 0; q < A_BLKS / 4; q++) {
                const int blk = q * 4 + wave;
                const int row = blk * 8 + (lane >> 3);
                const int c = (lane & 7) ^ swz_a(row);
                const int gm = m0 + row, gk = k0 + c * 8;
                const int off = (gm < M && gk < K) ? (gm * K + gk) * 2 : 0x7FFFFFF0;
                dma16(rsrc_a, smem_lds + a_off + blk * 1024, off);
            }
#pragma unroll
            for (int q = 0; q < B_BLKS / 4; q++) {
                const int blk = q * 4 + wave;
                const int lin = blk * 64 + lane;  // chunk index within the stage
                const int krow = lin / B_CHUNKS;
                const int c = (lin % B_CHUNKS) ^ swz_b<B_CHUNKS>(krow);
                const int gk = k0 + krow, gn = n0 + c * 8;
                const int off = (gk < K && gn < N) ? (gk * N + gn) * 2 : 0x7FFFFFF0;
                dma16(rsrc_b, smem_lds + b_off + blk * 1024, off);
            }
        } else {
            // element-wise guarded loads through registers, same LDS layout
#pragma unroll 1
            for (int q = 0; q < A_BLKS / 4; q++) {
                const int blk = q * 4 + wave;
                const int row = blk * 8 + (lane >> 3);
                const int pchunk = lane & 7;
                const int c = pchunk ^ swz_a(row);
                const int gm = m0 + row;
                half8 v;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const int gk = k0 + c * 8 + e;
                    v[e] = (gm < M && gk < K) ? Al[(int64_t)gm * K + gk] : (_Float16)0.0f;
                }
                *(half8 *)(smem + a_off + row * 128 + pchunk * 16) = v;
            }
#pragma unroll 1
            for (int q = 0; q < B_BLKS / 4; q++) {
                const int blk = q * 4 + wave;
                const int lin = blk * 64 + lane;
                const int krow = lin / B_CHUNKS;
                const int pchunk = lin % B_CHUNKS;
                const int c = pchunk ^ swz_b<B_CHUNKS>(krow);
                const int gk = k0 + krow;
                half8 v;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const int gn = n0 + c * 8 + e;
                    v[e] = (gk < K && gn < N) ? Bl[(int64_t)gk * N + gn] : (_Float16)0.0f;
                }
                *(half8 *)(smem + b_off + krow * B_ROW + pchunk * 16) = v;
            }
        }
    };

    // ---- LDS -> MFMA operand fragments -------------------------------------
    // A operand of v_mfma_f32_32x32x16_f16: lane (i + 32g) holds row i,
    // k = 8g..8g+7 of the 32 x 16 block.  B operand: lane (j + 32g) holds
    // column j, k = 8g..8g+7; ds_read_b64_tr_b16 gives lane q of a 16-lane
    // block the 4 values of column q from 4 k-rows, when lane 4e + r of the
    // block points at k-row e, columns 4r..4r+3.
    const int li = lane & 31, lg = lane >> 5;
    const int lb = lane >> 4, lq = lane & 15;
    auto read_frags = [&](int stage, int kk, half8 (&af)[TM], half8 (&bf)[TN]) {
        const char *a_src = smem + stage * STAGE;
        const char *b_src = a_src + A_STAGE;
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const int row = wm * WM + i * 32 + li;
            const int c = (kk * 2 + lg) ^ swz_a(row);
            af[i] = *(const half8 *)(a_src + row * 128 + c * 16);
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int n = wn * WN + j * 32 + 16 * (lb & 1) + 4 * (lq & 3);
            half8 b;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int krow = kk * 16 + 8 * (lb >> 1) + 4 * h + (lq >> 2);
                const int c = (n >> 3) ^ swz_b<B_CHUNKS>(krow);
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

    auto mfmas = [&](const half8 (&af)[TM], const half8 (&bf)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    };

    // ---- main loop ---------------------------------------------------------
    // Two LDS stages.  Operand fragments are double-buffered in registers and
    // read one 16-wide k step ahead of the MFMAs that use them; the barrier
    // that publishes stage kt+1 sits between the last fragment reads of stage
    // kt and its last MFMAs, so the MFMA pipe keeps working across it.
    // Stage kt+2 is fetched into the buffer stage kt used, right after that
    // barrier (by then every wave has finished reading stage kt).
    constexpr int KSTEPS = BK / 16;
    half8 fa[2][TM], fb[2][TN];
    load_stage(0, 0);
    if constexpr (VEC) wait_dma();
    __syncthreads();
    if (nk > 1) load_stage(1, BK);
    read_frags(0, 0, fa[0], fb[0]);
#pragma unroll 1
    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) {
            if (kk + 1 < KSTEPS) {
                read_frags(cur, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
            } else if (kt + 1 < nk) {
                if constexpr (VEC) wait_dma();  // this thread's part of stage kt+1 landed
                __syncthreads();                // all of stage kt+1 landed; stage kt is free
                if (kt + 2 < nk) load_stage(cur, (kt + 2) * BK);
                read_frags(cur ^ 1, 0, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
            }
            mfmas(fa[kk & 1], fb[kk & 1]);
        }
    }
    __syncthreads();  // LDS is reused by the epilogue

    // ---- epilogue ----------------------------------------------------------
    const float alpha = p.alpha, beta = p.beta, s = p.s;
    float *slab = (float *)(smem + wave * (32 * EPI_LD * 4));
    const int64_t mn_base = (int64_t)l * M * N;
#pragma unroll
    for (int i = 0; i < TM; i++) {  // fully unrolled: acc must stay in registers
        // acc block row i of this wave -> LDS slab (32 x WN fp32)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int col = j * 32 + (lane & 31);
                slab[row * EPI_LD + col] = acc[i][j][r];
            }
        __syncthreads();
        // each pass: 4 rows; lane owns columns 4*(lane%16) + {0..3} (+ WN/2)
        constexpr int HALF = WN / 2;
        constexpr int GROUPS = WN >= 128 ? 2 : 1;
#pragma unroll 2
        for (int pass = 0; pass < 8; pass++) {
            const int srow = pass * 4 + (lane >> 4);
            const int gm = m0 + wm * WM + i * 32 + srow;
#pragma unroll
            for (int h = 0; h < GROUPS; h++) {
                const int scol = 4 * (lane & 15) + h * HALF;
                if (scol >= WN) continue;
                const int gn = n0 + wn * WN + scol;
                const f32x4 a4 = *(const f32x4 *)(slab + srow * EPI_LD + scol);
                if (gm >= M) continue;
                const int64_t o = mn_base + (int64_t)gm * N + gn;
                if constexpr (VEC) {
                    if (gn >= N) continue;  // N % 8 == 0: a 4-column group is all in or all out
                    const half4 c4 = *(const half4 *)(p.C + o);
                    half4 x4 = {};
                    if constexpr (kind_reads_x(KIND)) x4 = *(const half4 *)(p.X + o);
                    half4 d4, e4;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        float d, a = 0.0f;
                        epi_elem<KIND>(a4[e], (float)c4[e], (float)x4[e], alpha, beta, s, d, a);
                        d4[e] = (_Float16)d;
                        e4[e] = (_Float16)a;
                    }
                    *(half4 *)(p.D + o) = d4;
                    if constexpr (kind_has_aux(KIND)) *(half4 *)(p.Aux + o) = e4;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        if (gn + e >= N) break;
                        const float c = (float)p.C[o + e];
                        const float x = kind_reads_x(KIND) ? (float)p.X[o + e] : 0.0f;
                        float d, a = 0.0f;
                        epi_elem<KIND>(a4[e], c, x, alpha, beta, s, d, a);
                        p.D[o + e] = (_Float16)d;
                        if constexpr (kind_has_aux(KIND)) p.Aux[o + e] = (_Float16)a;
                    }
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace gemm_epi
