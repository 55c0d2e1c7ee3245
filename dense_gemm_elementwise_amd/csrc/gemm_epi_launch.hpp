// gemm_epi_launch.hpp -- tile configurations, kernel launchers and the kind
// dispatch shared by the translation units of libgemm_epi.so (the fp16 one,
// which also holds the C ABI, and the bfloat16 one).
#pragma once
#include <hip/hip_runtime.h>
#include <type_traits>

#include "gemm_epi.h"
#include "gemm_epi_kernels.hpp"

namespace gemm_epi {

struct TileCfg {
    int bm, bn;      // output tile
    int bk, stages;  // K step per LDS stage, LDS stages in the ring
    int wgm, wgn;    // wave grid (threads = 64 * wgm * wgn)
    int mi;          // MFMA block: 32 (32x32x16) or 16 (16x16x32)
};

// The tile configurations compiled into the library (fast path), and the one
// general-path configuration.  The 256 x 256, 128 x 256, 256 x 128 and 128 x 128
// tiles run four waves of (BM/2) x (BN/2) on the hand-scheduled main loop
// (mainloop_w4: accumulators in AGPRs, 32-deep k steps); two 128 x 128
// workgroups fit on a compute unit (80 KiB of LDS each), and against the
// eight-wave ring it replaced that tile is 18% faster at 2048^3 and 29% at
// 3072^3, with the same bits.  The 64 x 64 tile (small problems, one wave of
// workgroups or less) has latency-bound stages, so fewer, deeper ones are
// what counts: BK = 64 (1024^3: 12.0 -> 9.7 us against BK = 32; more stages
// in the ring did not help), and BK = 128 (kSmallDeep) once K >= 256, where
// it is 1-8% faster again (with four waves of 32 x 32 the break-even was
// K = 512; the eight waves below moved it to 256).  Eight waves of 16 x 32 (two per SIMD, where
// one such workgroup is all a compute unit gets) hide more of that latency
// than four of 32 x 32: 3% at 1024^3, 6% on 256^3.  The stream-K build of
// the 128 x 128 tile keeps four waves of 64 x 64 on the ring (eight were
// 2-13% slower there).
inline constexpr TileCfg kTiles[] = {{256, 256, 32, 4, 2, 2, 16}, {128, 256, 32, 4, 2, 2, 16},
                                     {256, 128, 32, 4, 2, 2, 16}, {128, 128, 32, 4, 2, 2, 16},
                                     {64, 64, 64, 4, 4, 2, 16}};
// Epilogue tensors of another type than A and B keep 8-wave forms of the
// 128 x 256, 256 x 128 and 128 x 128 tiles (the host gives them these tiles
// in place of 256 x 256 and the 4-wave 128 x 128): their wider epilogue does
// not fit the 4-wave tiles' registers.
inline constexpr TileCfg kTile128x256W8 = {128, 256, 64, 2, 2, 4, 16};
inline constexpr TileCfg kTile256x128W8 = {256, 128, 64, 2, 4, 2, 16};
inline constexpr TileCfg kTile128x128W8 = {128, 128, 64, 3, 4, 2, 32};
inline constexpr TileCfg kSmallDeep = {64, 64, 128, 4, 4, 2, 16};
// The same with a 2-stage ring (64 KiB of LDS instead of 128): two workgroups
// fit on a compute unit, which pays once the grid has more tiles than there
// are compute units (1280^2 grids, 400 tiles: 24% faster) and costs where a
// unit holds only one (192 tiles: 16% slower; 16 tiles: 39%).
inline constexpr TileCfg kSmallDeepWide = {64, 64, 128, 2, 4, 2, 16};
inline constexpr int64_t kSmallDeepMinK = 256;
// The general path's tiles: eight waves of 32 x 64 (against four of 64 x 64:
// 4096 x 4096 x 4095 19% faster, 1001^3 43%), and eight of 64 x 64 on a
// 256 x 128 tile for grids that fill the chip several times (4096 x 4096 x
// 4095: 294 against 336 us; 1001^3: 53 against 31 us, so the tile model
// chooses).
inline constexpr TileCfg kGeneral = {128, 128, 64, 2, 4, 2, 32};
inline constexpr TileCfg kGeneralWide = {256, 128, 64, 2, 4, 2, 16};

// Calls f(std::integral_constant<int, KIND>) for a public kind (checked by
// check_args before any call).
template <typename F>
hipError_t dispatch_kind(int kind, F &&f)
{
    switch (kind) {
    case GEMM_EPI_LINCOMB: return f(std::integral_constant<int, LINCOMB>{});
    case GEMM_EPI_AUX_SCALE: return f(std::integral_constant<int, AUX_SCALE>{});
    case GEMM_EPI_LINCOMB_X_ACC: return f(std::integral_constant<int, LINCOMB_X_ACC>{});
    case GEMM_EPI_RELU: return f(std::integral_constant<int, RELU>{});
    case GEMM_EPI_SQUARE: return f(std::integral_constant<int, SQUARE>{});
    case GEMM_EPI_RELU_SQUARE: return f(std::integral_constant<int, RELU_SQUARE>{});
    case GEMM_EPI_RELU_AUX_STORE: return f(std::integral_constant<int, RELU_AUX_STORE>{});
    case GEMM_EPI_RELU_SCALE_ACC: return f(std::integral_constant<int, RELU_SCALE_ACC>{});
    case GEMM_EPI_BIAS_ROW_COL: return f(std::integral_constant<int, BIAS_ROW_COL>{});
    case GEMM_EPI_SIGMOID: return f(std::integral_constant<int, SIGMOID>{});
    case GEMM_EPI_TANH: return f(std::integral_constant<int, TANH>{});
    case GEMM_EPI_GELU: return f(std::integral_constant<int, GELU>{});
    case GEMM_EPI_SILU: return f(std::integral_constant<int, SILU>{});
    case GEMM_EPI_LEAKY_RELU: return f(std::integral_constant<int, LEAKY_RELU>{});
    default: return f(std::integral_constant<int, HARDSWISH>{});
    }
}

template <int BM, int BN, int BK, int NS, int WGM, int WGN, int MI, int KIND, bool VEC, bool SK = false,
          bool BF = false, int EPI = EPI_AB>
hipError_t launch_one(const Params &p, hipStream_t stream, int grid)
{
    // hipLaunchKernel reports this launch's own status (hipGetLastError would
    // also report, and clear, an error an earlier unrelated call left)
    Params arg = p;
    void *args[] = {(void *)&arg};
    return hipLaunchKernel((const void *)&gemm_epi_kernel<BM, BN, BK, NS, WGM, WGN, MI, KIND, VEC, SK, BF, EPI>,
                           dim3(grid), dim3(64 * WGM * WGN), args, 0, stream);
}

#define GE_LAUNCH(T, KIND, VEC) \
    launch_one<T.bm, T.bn, T.bk, T.stages, T.wgm, T.wgn, T.mi, KIND, VEC, false, BF, EPI>(p, stream, p.num_tiles)

// The fused kernel of one kind on tile configuration t (the general-path
// kernel when vec is false); BF: A and B are bfloat16; EPI: the epilogue
// tensors' type (EpiMode).
template <int KIND, bool BF = false, int EPI = EPI_AB>
hipError_t launch_kind(const Params &p, const TileCfg &t, bool vec, hipStream_t stream)
{
    if (!vec) {
        if (t.bm == kGeneralWide.bm && t.bn == kGeneralWide.bn) return GE_LAUNCH(kGeneralWide, KIND, false);
        return GE_LAUNCH(kGeneral, KIND, false);
    }
    // the 4-wave tiles are built for epilogue tensors of the type of A and B
    // only (the host gives the others the 8-wave tiles of the same shape)
    if constexpr (EPI == EPI_AB) {
        if (t.bm == kTiles[0].bm && t.bn == kTiles[0].bn) return GE_LAUNCH(kTiles[0], KIND, true);
        if (t.bm == kTiles[1].bm && t.bn == kTiles[1].bn) return GE_LAUNCH(kTiles[1], KIND, true);
        if (t.bm == kTiles[2].bm && t.bn == kTiles[2].bn) return GE_LAUNCH(kTiles[2], KIND, true);
        if (t.bm == kTiles[3].bm && t.bn == kTiles[3].bn) return GE_LAUNCH(kTiles[3], KIND, true);
    } else {
        if (t.bm == kTile128x256W8.bm && t.bn == kTile128x256W8.bn) return GE_LAUNCH(kTile128x256W8, KIND, true);
        if (t.bm == kTile256x128W8.bm && t.bn == kTile256x128W8.bn) return GE_LAUNCH(kTile256x128W8, KIND, true);
        if (t.bm == kTile128x128W8.bm && t.bn == kTile128x128W8.bn) return GE_LAUNCH(kTile128x128W8, KIND, true);
    }
    if (t.bk == kSmallDeep.bk && t.stages == kSmallDeepWide.stages) return GE_LAUNCH(kSmallDeepWide, KIND, true);
    if (t.bk == kSmallDeep.bk) return GE_LAUNCH(kSmallDeep, KIND, true);
    return GE_LAUNCH(kTiles[4], KIND, true);
}

#undef GE_LAUNCH

// The stream-K build (the fused kernel walking a contiguous range of
// (tile, k stage) units per workgroup) exists for this tile only: the 8-wave
// 256 x 256 tile has no registers to spare for the range loop.
inline constexpr TileCfg kSkTile = {128, 128, 64, 3, 2, 2, 32};

template <int KIND, bool BF = false>
hipError_t launch_kind_sk(const Params &p, int groups, hipStream_t stream)
{
    constexpr TileCfg T = kSkTile;
    return launch_one<T.bm, T.bn, T.bk, T.stages, T.wgm, T.wgn, T.mi, KIND, true, true, BF>(p, stream, groups);
}

// The bfloat16 kernels are defined in gemm_epi_bf16.hip, a translation unit
// of its own so that the two element types compile in parallel: the fused
// call, its stream-K build, and the GEMM stage of the unfused composition.
hipError_t launch_fused_bf16(int kind, const Params &p, const TileCfg &t, bool vec, hipStream_t stream);
hipError_t launch_sk_bf16(int kind, const Params &p, int groups, hipStream_t stream);
hipError_t launch_acc_store_bf16(const Params &p, const TileCfg &t, bool vec, hipStream_t stream);
// The fused call with fp32 epilogue tensors (C, X, the biases, D, Aux), A and
// B fp16 (gemm_epi_f32e.hip) or bfloat16 (gemm_epi_bf16_f32e.hip); and with
// the other 16-bit type for the epilogue tensors (gemm_epi_f16_bf16e.hip,
// gemm_epi_bf16_f16e.hip).
hipError_t launch_fused_f16_f32e(int kind, const Params &p, const TileCfg &t, bool vec, hipStream_t stream);
hipError_t launch_fused_bf16_f32e(int kind, const Params &p, const TileCfg &t, bool vec, hipStream_t stream);
hipError_t launch_fused_f16_bf16e(int kind, const Params &p, const TileCfg &t, bool vec, hipStream_t stream);
hipError_t launch_fused_bf16_f16e(int kind, const Params &p, const TileCfg &t, bool vec, hipStream_t stream);

}  // namespace gemm_epi
