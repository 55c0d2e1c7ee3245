// gemm_epi.hip -- C ABI of libgemm_epi.so: argument checks, kernel choice and
// launch of the fused fp16 GEMM + elementwise epilogue on gfx950.
//
// The entry points and their contracts are declared in include/gemm_epi.h.
// Every check runs on the host before any HIP call, so a bad argument never
// queues work and the checks run without a GPU.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "gemm_epi.h"
#include "gemm_epi_kernels.hpp"
#include "gemm_epi_launch.hpp"

using namespace gemm_epi;

namespace {

thread_local int g_last_hip_error = 0;

// Relative MFMA efficiency of a tile (bigger tiles reuse each LDS operand
// read over more MFMAs and amortise the epilogue better).  128 x 128 is a
// little above 3/4 so that 3 waves of it beat 1 of 256 x 256 (and 6 beat 2,
// 9 beat 3) instead of tying: two of its workgroups share a CU and cover each
// other's stalls, which the wave count does not see (measured 2-25% faster
// on such grids, 3072^3 to 5888^2 x 2048, with the same bits).
double tile_efficiency(int bm, int bn)
{
    const int area = bm * bn;
    if (area >= 256 * 256) return 1.0;
    if (area >= 256 * 128) return 0.9;
    if (area >= 128 * 128) return 0.76;
    return 0.4;
}

constexpr int kNumCUs = 256;

// Chooses the tile that minimises (waves of workgroups) x (tile area / its
// efficiency): big tiles when the grid fills the chip several times, smaller
// ones when big tiles would leave compute units idle.  Ties go to the tile
// that pads the problem least, then to the one whose long side lies along the
// problem's long side.  The 64 x 64 tile takes its deeper K step when K is
// long enough to fill its ring, with the shorter ring when the grid has more
// tiles than compute units.
TileCfg choose_tile(int64_t L, int64_t M, int64_t N, int64_t K, bool vec)
{
    if (!vec) {
        // the general path's two tiles, by the same cost
        auto cost = [&](const TileCfg &t) {
            const int64_t tiles = L * ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
            return (double)((tiles + kNumCUs - 1) / kNumCUs) * t.bm * t.bn / tile_efficiency(t.bm, t.bn);
        };
        return cost(kGeneralWide) < cost(kGeneral) ? kGeneralWide : kGeneral;
    }
    TileCfg best = kTiles[0];
    double best_cost = 1e300, best_pad = 1e300;
    int best_orient = 2;
    for (const TileCfg &t : kTiles) {
        const int64_t tm = (M + t.bm - 1) / t.bm, tn = (N + t.bn - 1) / t.bn;
        const int64_t tiles = L * tm * tn;
        const double waves = (double)((tiles + kNumCUs - 1) / kNumCUs);
        const double cost = waves * (double)t.bm * t.bn / tile_efficiency(t.bm, t.bn);
        const double pad = (double)tiles * t.bm * t.bn;
        const int orient = (t.bm == t.bn) ? 0 : ((t.bm > t.bn) == (M > N) ? 0 : 1);
        const bool better = cost < best_cost - 1e-9 ||
                            (cost < best_cost + 1e-9 &&
                             (pad < best_pad - 0.5 || (pad < best_pad + 0.5 && orient < best_orient)));
        if (better) {
            best_cost = cost;
            best_pad = pad;
            best_orient = orient;
            best = t;
        }
    }
    if (best.bm == kSmallDeep.bm && best.bn == kSmallDeep.bn && K >= kSmallDeepMinK) {
        const int64_t tiles = L * ((M + best.bm - 1) / best.bm) * ((N + best.bn - 1) / best.bn);
        return tiles > kNumCUs ? kSmallDeepWide : kSmallDeep;
    }
    return best;
}

// Epilogue tensors of another type than A and B (fp32, or the other 16-bit
// type) take the 8-wave tiles: the 256 x 128 (or 128 x 256) one where the
// choice is 256 x 256, and the 8-wave 128 x 128 one in place of the 4-wave
// 128 x 128 (the 4-wave tiles are built for one element type only).
TileCfg tile_for_mixed(const TileCfg &t, int64_t M, int64_t N)
{
    if (t.bm == kTiles[3].bm && t.bn == kTiles[3].bn) return kTile128x128W8;
    if (t.bm != kTiles[0].bm || t.bn != kTiles[0].bn) return t;
    return M >= N ? kTile256x128W8 : kTile128x256W8;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Host-side operand set of one call (the pointers gemm_epi_run_ext takes).
struct Operands {
    const void *A, *B, *C, *X, *row_bias, *col_bias;
    const void *D, *Aux, *acc_out;
};

int check_args(int64_t L, int64_t M, int64_t N, int64_t K, const Operands &o, int kind)
{
    if (L < 1 || M < 1 || N < 1 || K < 1) return GEMM_EPI_ERR_SHAPE;
    const int64_t lim = INT32_MAX;
    if (M > lim || N > lim || K > lim) return GEMM_EPI_ERR_SHAPE;
    // element counts of every tensor must fit int64 (and the grid must fit);
    // the fp32 accumulator output needs twice the bytes of an fp16 output
    if (L > INT64_MAX / M || L * M > INT64_MAX / K || L * M > INT64_MAX / N || L > INT64_MAX / K ||
        L * K > INT64_MAX / N || L * M * N > INT64_MAX / 4)
        return GEMM_EPI_ERR_SHAPE;
    if (!o.A || !o.B) return GEMM_EPI_ERR_NULL_INPUT;
    if (kind < GEMM_EPI_LINCOMB || kind > GEMM_EPI_HARDSWISH) return GEMM_EPI_ERR_KIND;
    if ((kind_reads_c(kind) && !o.C) || (kind_reads_x(kind) && !o.X) ||
        (kind_reads_bias(kind) && (!o.row_bias || !o.col_bias)))
        return GEMM_EPI_ERR_NULL_INPUT;
    if (!o.D || (kind_has_aux(kind) && !o.Aux) || (kind_has_acc_out(kind) && !o.acc_out))
        return GEMM_EPI_ERR_NULL_OUTPUT;
    const void *halves[] = {o.A, o.B, o.C, o.X, o.row_bias, o.col_bias, o.D, o.Aux};
    for (const void *h : halves)
        if (h && !aligned(h, 2)) return GEMM_EPI_ERR_ALIGN;
    if (o.acc_out && !aligned(o.acc_out, 4)) return GEMM_EPI_ERR_ALIGN;
    return GEMM_EPI_OK;
}

bool use_fast_path(int64_t M, int64_t N, int64_t K, const Operands &o, int kind)
{
    if (K % 8 != 0 || N % 8 != 0) return false;
    if (!aligned(o.A, 16) || !aligned(o.B, 16)) return false;
    if (kind_writes_d(kind) && !aligned(o.D, 16)) return false;
    if (kind_reads_c(kind) && !aligned(o.C, 16)) return false;
    if (kind_reads_x(kind) && !aligned(o.X, 16)) return false;
    if (kind_reads_bias(kind) && !aligned(o.row_bias, 16)) return false;
    if (kind_has_aux(kind) && !aligned(o.Aux, 16)) return false;
    if (kind_has_acc_out(kind) && !aligned(o.acc_out, 16)) return false;
    // 32-bit buffer offsets: one batch entry of A or B must span < 2 GiB
    const int64_t lim = (int64_t)1 << 31;
    if (M * K * 2 >= lim - 64 || K * N * 2 >= lim - 64) return false;
    // the epilogue addresses one tile's rows (at most 256) of an epilogue
    // tensor (at most 4-byte elements) below the parked offset 2^31 - 16
    if (256 * N * 4 >= lim - 64) return false;
    return true;
}

// ---- stream-K ---------------------------------------------------------------
// Tiles with a stream-K build: a workgroup walks a contiguous range of
// (tile, k stage) units, so a few tiles can keep every CU busy.
constexpr TileCfg kSkTiles[] = {kSkTile};

struct SkPlan {
    bool on = false;
    TileCfg t{};
    int groups = 0;
    int64_t tiles = 0, units = 0, K = 0;
    size_t workspace = 0;  // bytes: the counter block, then the partial slots
};

// Workspace layout of a split, the same for every plan: one int32 counter
// per tile at offset 0, in a block of fixed capacity (a split covers at most
// kSkMaxTiles tiles), then 2 partial-sum slots per workgroup.  A workspace
// that is reused for a shape with another workgroup count therefore finds
// its counters where the previous call left them at zero.
constexpr int64_t kSkMaxTiles = 4096;
constexpr size_t kSkCounterBytes = (size_t)kSkMaxTiles * 4;

size_t sk_partials_bytes(const TileCfg &t, int groups) { return (size_t)2 * groups * t.bm * t.bn * 4; }

// Chooses between the one-tile-per-workgroup grid and a stream-K split, and
// the split's workgroup count, by a cost model in units of (tile area /
// efficiency) x K: waves x K for the former; for the latter the busiest
// workgroup's k stages plus, when a tile is split, a fixed cost and a cost
// per contributor of the most-split tile.  Both were fitted to run times of a
// 256 x 256 x 65536 product split over 16..256 workgroups on MI355X (one k
// stage of the 128 x 128 x 64 tile took about 0.76 us): about 8.5 stages for
// the device-scope fences and the counter, and about 1.6 stages for each
// partial sum the last contributor reads back.  Contributors of one tile
// work at different k, so their operand streams (32 KB per k stage and
// workgroup) share little in L2: past about 5.5 TB/s of such streams (some
// 128 workgroups at that stage time) a stage takes longer in proportion, as
// measured on 512..1024-square tiles with K of 8192..65536.  Fewer
// workgroups mean more k stages each but fewer partial sums per tile, so the
// count is searched.  A split is taken only when it wins clearly (by 15%).
SkPlan plan_stream_k(int64_t L, int64_t M, int64_t N, int64_t K, bool vec, int max_groups = kNumCUs)
{
    constexpr double kFixedStages = 8.5, kPerContributorStages = 1.6;
    constexpr double kStageSeconds = 0.76e-6, kOperandBytesPerSecond = 5.5e12;
    SkPlan best;
    if (!vec) return best;
    const TileCfg dp = choose_tile(L, M, N, K, vec);
    const int64_t dp_tiles = L * ((M + dp.bm - 1) / dp.bm) * ((N + dp.bn - 1) / dp.bn);
    const double dp_cost = (double)((dp_tiles + kNumCUs - 1) / kNumCUs) * ((K + dp.bk - 1) / dp.bk) * dp.bk *
                           dp.bm * dp.bn / tile_efficiency(dp.bm, dp.bn);
    double best_cost = 0.85 * dp_cost;
    for (const TileCfg &t : kSkTiles) {
        const int64_t tiles = L * ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
        const int64_t nk = (K + t.bk - 1) / t.bk;
        const int64_t units = tiles * nk;
        if (tiles > kSkMaxTiles || units < 2) continue;
        const double stage = (double)t.bk * t.bm * t.bn / tile_efficiency(t.bm, t.bn);
        for (int groups = kNumCUs; groups >= 1; groups /= 2) {
            if (groups > max_groups) continue;
            if (groups > units) continue;
            const int64_t per = (units + groups - 1) / groups;
            const bool split = per < nk || units % groups != 0 || (units / groups) % nk != 0;
            // a tile's k stages meet at most this many workgroup ranges
            const int64_t contrib = split ? std::min<int64_t>((nk + per - 2) / per + 1, groups) : 1;
            const double stream = (double)groups * (t.bm + t.bn) * t.bk * 2 / kOperandBytesPerSecond;
            const double slowdown = std::max(1.0, stream / kStageSeconds);
            const double cost =
                (per * slowdown + (split ? kFixedStages + kPerContributorStages * (double)contrib : 0.0)) * stage;
            if (cost < best_cost) {
                best_cost = cost;
                best.on = true;
                best.t = t;
                best.groups = groups;
                best.tiles = tiles;
                best.units = units;
                best.workspace = kSkCounterBytes + sk_partials_bytes(t, groups);
                best.K = K;
            }
        }
    }
    return best;
}

// The stream-K split of a call: units per workgroup and the workspace's
// partial-sum slots and per-tile counters.
void set_sk_params(Params &p, const SkPlan &sk, void *workspace)
{
    p.sk_q = sk.units / sk.groups;
    p.sk_r = sk.units % sk.groups;
    p.counters = (int *)workspace;
    p.partials = (float *)((char *)workspace + kSkCounterBytes);
}

// The elementwise stage of the unfused composition.
template <int KIND, bool BF>
hipError_t launch_epilogue(const EpiParams &q, bool vec, hipStream_t stream)
{
    const int64_t blocks = q.rows < 8192 ? q.rows : 8192;
    void *args[] = {(void *)&q};
    const void *fn = vec ? (const void *)&epilogue_kernel<KIND, true, BF> : (const void *)&epilogue_kernel<KIND, false, BF>;
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

// Launches the planned stream-K split of a checked call on `workspace`
// (counters at offset 0, zero between calls; partial sums after them).
int launch_split(int64_t L, int64_t M, int64_t N, const Operands &o, const float *scalars, int kind,
                 const SkPlan &sk, void *workspace, int dtype, hipStream_t s, int64_t b_rows = 0)
{
    Params p = {};
    p.b_rows = (int)b_rows;
    p.A = (const _Float16 *)o.A;
    p.B = (const _Float16 *)o.B;
    p.C = (const _Float16 *)o.C;
    p.X = (const _Float16 *)o.X;
    p.D = (_Float16 *)o.D;
    p.Aux = (_Float16 *)o.Aux;
    p.row_bias = (const _Float16 *)o.row_bias;
    p.col_bias = (const _Float16 *)o.col_bias;
    p.acc_out = (float *)o.acc_out;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)sk.K;
    p.tiles_m = (int)((M + sk.t.bm - 1) / sk.t.bm);
    p.tiles_n = (int)((N + sk.t.bn - 1) / sk.t.bn);
    p.num_tiles = (int)sk.tiles;
    p.group_m = L > 1 ? 2 : 8;
    p.alpha = scalars[0];
    p.beta = scalars[1];
    p.s = scalars[2];
    set_sk_params(p, sk, workspace);
    hipError_t err;
    if (dtype == GEMM_EPI_BF16)
        err = launch_sk_bf16(kind, p, sk.groups, s);
    else
        err = dispatch_kind(kind, [&](auto k) { return launch_kind_sk<decltype(k)::value>(p, sk.groups, s); });
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return GEMM_EPI_ERR_HIP;
    }
    return GEMM_EPI_OK;
}

// ---- staging through the workspace -------------------------------------------
// Operands that break the fast path's layout rules (K or N not a multiple of
// 8, or a tensor not 16-byte aligned) are copied into aligned, zero-padded
// buffers in the workspace, so that the fast kernel runs on them; outputs
// that break them are written there and copied back.  K % 8 != 0 pads A's
// rows to K8 with zeros and runs the kernel with K = K8 over B's K rows (its
// rows past K read as zeros: Params::b_rows); the zero products add nothing.
// N % 8 != 0 gives B and every M x N tensor rows of N8 elements.  Otherwise
// only the misaligned tensors are copied.  The regions start after the
// stream-K counter block, which staging never touches.
struct StagePlan {
    bool on = false;
    int64_t K = 0, N = 0;  // the fast kernel's K and N
    bool a = false, b = false, c = false, x = false, rb = false, d = false, aux = false, acc = false;
    size_t off_a = 0, off_b = 0, off_c = 0, off_x = 0, off_rb = 0, off_d = 0, off_aux = 0, off_acc = 0;
    size_t bytes = 0;  // workspace bytes the staged call needs
};

StagePlan plan_staging(int64_t L, int64_t M, int64_t N, int64_t K, const Operands &o, int kind,
                       size_t base = kSkCounterBytes)
{
    StagePlan st;
    const bool kr = K % 8 != 0, nr = N % 8 != 0;
    st.K = (K + 7) / 8 * 8;
    st.N = (N + 7) / 8 * 8;
    st.a = kr || !aligned(o.A, 16);
    st.b = nr || !aligned(o.B, 16);
    st.c = kind_reads_c(kind) && (nr || !aligned(o.C, 16));
    st.x = kind_reads_x(kind) && (nr || !aligned(o.X, 16));
    st.rb = kind_reads_bias(kind) && (nr || !aligned(o.row_bias, 16));
    st.d = kind_writes_d(kind) && (nr || !aligned(o.D, 16));
    st.aux = kind_has_aux(kind) && (nr || !aligned(o.Aux, 16));
    st.acc = kind_has_acc_out(kind) && (nr || !aligned(o.acc_out, 16));
    // the staged call must meet the fast path's size rules (16-byte aligned
    // stand-ins for every pointer)
    const void *al = (const void *)(uintptr_t)4096;
    const Operands staged = {al, al, al, al, al, al, al, al, al};
    if (!use_fast_path(M, st.N, st.K, staged, kind)) return st;
    size_t off = base;
    auto take = [&](bool on, int64_t elems, int es) {
        if (!on) return (size_t)0;
        const size_t at = off;
        off = (off + (size_t)elems * es + 255) & ~(size_t)255;
        return at;
    };
    st.off_a = take(st.a, L * M * st.K, 2);
    st.off_b = take(st.b, L * K * st.N, 2);
    st.off_c = take(st.c, L * M * st.N, 2);
    st.off_x = take(st.x, L * M * st.N, 2);
    st.off_rb = take(st.rb, st.N, 2);
    st.off_d = take(st.d, L * M * st.N, 2);
    st.off_aux = take(st.aux, L * M * st.N, 2);
    st.off_acc = take(st.acc, L * M * st.N, 4);
    st.bytes = off;
    st.on = true;
    return st;
}

// A staged call, with a stream-K split of the staged shape where one pays:
// the split's partial sums follow the counter block and the staging regions
// follow them.
struct StagedCall {
    StagePlan st;
    SkPlan sk;
};

StagedCall plan_staged_call(int64_t L, int64_t M, int64_t N, int64_t K, const Operands &o, int kind)
{
    StagedCall c;
    c.st = plan_staging(L, M, N, K, o, kind);
    if (!c.st.on) return c;
    c.sk = plan_stream_k(L, M, c.st.N, c.st.K, true);
    if (c.sk.on) c.st = plan_staging(L, M, N, K, o, kind, kSkCounterBytes + sk_partials_bytes(c.sk.t, c.sk.groups));
    return c;
}

// One launch for a set of copies in the same direction and of one element
// size (a grid row per copy); no launch for an empty set.
struct StageBatch {
    StageCopies q = {};
    int n = 0;
    int64_t rows = 0;  // the most rows a copy walks
    void add(const void *src, void *dst, int64_t L, int64_t r, int64_t c, int64_t pr, int64_t pc, bool pad)
    {
        q.c[n++] = StageCopy{src, dst, L, r, c, pr, pc};
        rows = std::max(rows, L * (pad ? pr : r));
    }
};

template <typename T>
hipError_t launch_stage(bool pad, const StageBatch &b, hipStream_t stream)
{
    if (b.n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)(b.rows < 8192 ? b.rows : 8192);
    StageCopies q = b.q;
    void *args[] = {(void *)&q};
    const void *fn = pad ? (const void *)&stage_pad_kernel<T> : (const void *)&stage_unpad_kernel<T>;
    return hipLaunchKernel(fn, dim3(blocks, (unsigned)b.n), dim3(256), args, 0, stream);
}

// Runs a checked call through the staging plan: copies in, the fast kernel on
// the staged operand set, copies out, all on `stream`.
int launch_staged(int64_t L, int64_t M, int64_t N, int64_t K, const Operands &o, const float *scalars, int kind,
                  const StagedCall &call, void *workspace, int dtype, hipStream_t s)
{
    const StagePlan &st = call.st;
    char *ws = (char *)workspace;
    auto at = [&](bool on, size_t off, const void *orig) { return on ? (void *)(ws + off) : const_cast<void *>(orig); };
    Params p = {};
    p.A = (const _Float16 *)at(st.a, st.off_a, o.A);
    p.B = (const _Float16 *)at(st.b, st.off_b, o.B);
    p.C = (const _Float16 *)at(st.c, st.off_c, o.C);
    p.X = (const _Float16 *)at(st.x, st.off_x, o.X);
    p.row_bias = (const _Float16 *)at(st.rb, st.off_rb, o.row_bias);
    p.col_bias = (const _Float16 *)o.col_bias;
    p.D = (_Float16 *)at(st.d, st.off_d, o.D);
    p.Aux = (_Float16 *)at(st.aux, st.off_aux, o.Aux);
    p.acc_out = (float *)at(st.acc, st.off_acc, o.acc_out);
    const TileCfg t = choose_tile(L, M, st.N, st.K, true);
    const int64_t tm = (M + t.bm - 1) / t.bm, tn = (st.N + t.bn - 1) / t.bn;
    const int64_t tiles = L * tm * tn;
    if (tiles > INT32_MAX) return GEMM_EPI_ERR_SHAPE;
    p.M = (int)M;
    p.N = (int)st.N;
    p.K = (int)st.K;
    p.b_rows = (int)K;  // B (staged or not) keeps its K rows
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    p.num_tiles = (int)tiles;
    p.group_m = L > 1 ? 2 : 8;
    p.alpha = scalars[0];
    p.beta = scalars[1];
    p.s = scalars[2];

    hipError_t err = hipSuccess;
    auto step = [&](hipError_t e) {
        if (err == hipSuccess) err = e;
    };
    StageBatch in;
    if (st.a) in.add(o.A, (void *)p.A, L, M, K, M, st.K, true);
    if (st.b) in.add(o.B, (void *)p.B, L, K, N, K, st.N, true);
    if (st.c) in.add(o.C, (void *)p.C, L, M, N, M, st.N, true);
    if (st.x) in.add(o.X, (void *)p.X, L, M, N, M, st.N, true);
    if (st.rb) in.add(o.row_bias, (void *)p.row_bias, 1, 1, N, 1, st.N, true);
    step(launch_stage<uint16_t>(true, in, s));
    if (err == hipSuccess && call.sk.on) {
        const Operands so = {p.A, p.B, p.C, p.X, p.row_bias, p.col_bias, p.D, p.Aux, p.acc_out};
        const int rc = launch_split(L, M, st.N, so, scalars, kind, call.sk, workspace, dtype, s, K);
        if (rc != GEMM_EPI_OK) return rc;
    } else if (err == hipSuccess) {
        if (dtype == GEMM_EPI_BF16)
            step(launch_fused_bf16(kind, p, t, true, s));
        else
            step(dispatch_kind(kind, [&](auto k) { return launch_kind<decltype(k)::value>(p, t, true, s); }));
    }
    StageBatch out16, out32;
    if (st.d) out16.add(p.D, (void *)o.D, L, M, N, M, st.N, false);
    if (st.aux) out16.add(p.Aux, (void *)o.Aux, L, M, N, M, st.N, false);
    if (st.acc) out32.add(p.acc_out, (void *)o.acc_out, L, M, N, M, st.N, false);
    if (err == hipSuccess) step(launch_stage<uint16_t>(false, out16, s));
    if (err == hipSuccess) step(launch_stage<uint32_t>(false, out32, s));
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return GEMM_EPI_ERR_HIP;
    }
    return GEMM_EPI_OK;
}

// ---- the scratch-free stream-K call (gemm_epi_run_ws_static) ----------------
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the split's counters and
// partial sums live in this file-scope device array, one copy per GPU, held
// until the process ends.  Its splits use at most kStaticMaxGroups
// workgroups, whose two partial slots each fill it.  In host code `scratch`
// is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr int kStaticMaxGroups = 128;
constexpr size_t kStaticScratchBytes = kSkCounterBytes + (size_t)2 * kStaticMaxGroups * 128 * 128 * 4;  // 16 MiB + 16 KiB
static_assert(kSkTile.bm == 128 && kSkTile.bn == 128, "scratch sized for the 128 x 128 split tile");
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

__global__ void zero_words(int *p, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// The current device's scratch address.  On a device's first call it is
// looked up and its counter block cleared by a kernel on the caller's stream
// (ahead of the split in stream order; a kernel, not a memset node, so that a
// graph captured around the call replays correctly).
hipError_t device_scratch(hipStream_t stream, void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        int *words = (int *)ptr;
        int n = (int)(kSkCounterBytes / 4);
        void *args[] = {(void *)&words, (void *)&n};
        e = hipLaunchKernel((const void *)&zero_words, dim3(16), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *gemm_epi_status_string(int status)
{
    switch (status) {
    case GEMM_EPI_OK: return "ok";
    case GEMM_EPI_ERR_SHAPE: return "invalid shape: L, M, N, K must be >= 1 and every tensor size must fit";
    case GEMM_EPI_ERR_NULL_INPUT:
        return "an input the epilogue reads (A, B, C, X, a bias vector, or scalars) is not provided";
    case GEMM_EPI_ERR_NULL_OUTPUT: return "an output the epilogue writes (D, Aux, or acc_out) is not provided";
    case GEMM_EPI_ERR_KIND: return "unknown epilogue kind";
    case GEMM_EPI_ERR_ALIGN: return "a tensor pointer is not aligned to its element size";
    case GEMM_EPI_ERR_HIP: return "HIP launch error";
    case GEMM_EPI_ERR_WORKSPACE: return "the workspace is missing or smaller than the call needs";
    case GEMM_EPI_ERR_DTYPE: return "unknown element type";
    default: return "unknown status";
    }
}

int gemm_epi_last_hip_error(void) { return g_last_hip_error; }

int gemm_epi_plan_ext(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                      const void *X, const void *row_bias, const void *col_bias, int epilogue_kind, const void *D,
                      const void *Aux, const void *acc_out, int64_t out[6])
{
    const Operands o = {A, B, C, X, row_bias, col_bias, D, Aux, acc_out};
    int rc = check_args(L, M, N, K, o, epilogue_kind);
    if (rc != GEMM_EPI_OK) return rc;
    const bool vec = use_fast_path(M, N, K, o, epilogue_kind);
    const TileCfg t = choose_tile(L, M, N, K, vec);
    const int64_t tiles = L * ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    if (tiles > INT32_MAX) return GEMM_EPI_ERR_SHAPE;
    if (out) {
        out[0] = t.bm;
        out[1] = t.bn;
        out[2] = t.bk;
        out[3] = vec ? 1 : 0;
        out[4] = tiles;
        out[5] = 64 * t.wgm * t.wgn;
    }
    return GEMM_EPI_OK;
}

int gemm_epi_plan(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                  const void *X, int epilogue_kind, const void *D, const void *Aux, int64_t out[6])
{
    return gemm_epi_plan_ext(L, M, N, K, A, B, C, X, nullptr, nullptr, epilogue_kind, D, Aux, nullptr, out);
}

int gemm_epi_run_ext(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                     const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                     int epilogue_kind, void *D, void *Aux, void *acc_out, void *stream)
{
    return gemm_epi_run_typed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                              GEMM_EPI_F16, stream);
}

int gemm_epi_run_typed(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                       const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                       int epilogue_kind, void *D, void *Aux, void *acc_out, int dtype, void *stream)
{
    return gemm_epi_run_mixed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                              dtype, dtype, stream);
}

int gemm_epi_run_mixed(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                       const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                       int epilogue_kind, void *D, void *Aux, void *acc_out, int ab_dtype, int epi_dtype,
                       void *stream)
{
    const Operands o = {A, B, C, X, row_bias, col_bias, D, Aux, acc_out};
    int rc = check_args(L, M, N, K, o, epilogue_kind);
    if (rc != GEMM_EPI_OK) return rc;
    if (ab_dtype != GEMM_EPI_F16 && ab_dtype != GEMM_EPI_BF16) return GEMM_EPI_ERR_DTYPE;
    const bool f32e = epi_dtype == GEMM_EPI_F32;
    if (epi_dtype != ab_dtype && !f32e && epi_dtype != GEMM_EPI_F16 && epi_dtype != GEMM_EPI_BF16)
        return GEMM_EPI_ERR_DTYPE;
    const bool other16 = !f32e && epi_dtype != ab_dtype;
    if (!scalars) return GEMM_EPI_ERR_NULL_INPUT;
    if (f32e) {
        const void *words[] = {C, X, row_bias, col_bias, D, Aux};
        for (const void *w : words)
            if (w && !aligned(w, 4)) return GEMM_EPI_ERR_ALIGN;
    }
    const bool vec = use_fast_path(M, N, K, o, epilogue_kind);
    TileCfg t = choose_tile(L, M, N, K, vec);
    if (f32e || other16) t = tile_for_mixed(t, M, N);
    const int64_t tm = (M + t.bm - 1) / t.bm, tn = (N + t.bn - 1) / t.bn;
    const int64_t tiles = L * tm * tn;
    if (tiles > INT32_MAX) return GEMM_EPI_ERR_SHAPE;

    Params p = {};
    p.A = (const _Float16 *)A;
    p.B = (const _Float16 *)B;
    p.C = (const _Float16 *)C;  // the kernels read the epilogue tensors as their element type
    p.X = (const _Float16 *)X;
    p.D = (_Float16 *)D;
    p.Aux = (_Float16 *)Aux;
    p.row_bias = (const _Float16 *)row_bias;
    p.col_bias = (const _Float16 *)col_bias;
    p.acc_out = (float *)acc_out;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    p.num_tiles = (int)tiles;
    // L2 grouping: 8 tile rows share B column panels in a single large
    // product; batched products keep each XCD on few batch entries instead.
    p.group_m = L > 1 ? 2 : 8;
    p.alpha = scalars[0];
    p.beta = scalars[1];
    p.s = scalars[2];

    hipStream_t s = (hipStream_t)stream;
    hipError_t err;
    const bool bf = ab_dtype == GEMM_EPI_BF16;
    if (f32e)
        err = bf ? launch_fused_bf16_f32e(epilogue_kind, p, t, vec, s) : launch_fused_f16_f32e(epilogue_kind, p, t, vec, s);
    else if (other16)
        err = bf ? launch_fused_bf16_f16e(epilogue_kind, p, t, vec, s) : launch_fused_f16_bf16e(epilogue_kind, p, t, vec, s);
    else if (bf)
        err = launch_fused_bf16(epilogue_kind, p, t, vec, s);
    else
        err = dispatch_kind(epilogue_kind, [&](auto k) { return launch_kind<decltype(k)::value>(p, t, vec, s); });
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return GEMM_EPI_ERR_HIP;
    }
    return GEMM_EPI_OK;
}

int gemm_epi_run_unfused(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                         const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                         int epilogue_kind, void *D, void *Aux, void *acc_out, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    return gemm_epi_run_unfused_typed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux,
                                      acc_out, workspace, workspace_bytes, GEMM_EPI_F16, stream);
}

int gemm_epi_run_unfused_typed(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                               const void *C, const void *X, const void *row_bias, const void *col_bias,
                               const float *scalars, int epilogue_kind, void *D, void *Aux, void *acc_out,
                               void *workspace, size_t workspace_bytes, int dtype, void *stream)
{
    const Operands o = {A, B, C, X, row_bias, col_bias, D, Aux, acc_out};
    int rc = check_args(L, M, N, K, o, epilogue_kind);
    if (rc != GEMM_EPI_OK) return rc;
    if (dtype != GEMM_EPI_F16 && dtype != GEMM_EPI_BF16) return GEMM_EPI_ERR_DTYPE;
    if (!scalars) return GEMM_EPI_ERR_NULL_INPUT;
    // the accumulator goes to acc_out when the kind returns it, else to the workspace
    float *acc = (float *)(kind_has_acc_out(epilogue_kind) ? acc_out : workspace);
    if (!kind_has_acc_out(epilogue_kind)) {
        if (!workspace || workspace_bytes / 4 < (size_t)(L * M * N)) return GEMM_EPI_ERR_WORKSPACE;
        if (!aligned(workspace, 4)) return GEMM_EPI_ERR_ALIGN;
    }

    // stage 1: the GEMM, writing only the fp32 accumulator
    const Operands o1 = {A, B, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, acc};
    const bool vec1 = use_fast_path(M, N, K, o1, ACC_STORE);
    const TileCfg t = choose_tile(L, M, N, K, vec1);
    const int64_t tm = (M + t.bm - 1) / t.bm, tn = (N + t.bn - 1) / t.bn;
    const int64_t tiles = L * tm * tn;
    if (tiles > INT32_MAX) return GEMM_EPI_ERR_SHAPE;
    Params p = {};
    p.A = (const _Float16 *)A;
    p.B = (const _Float16 *)B;
    p.acc_out = acc;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.tiles_m = (int)tm;
    p.tiles_n = (int)tn;
    p.num_tiles = (int)tiles;
    p.group_m = L > 1 ? 2 : 8;
    p.alpha = 1.0f;
    hipStream_t s = (hipStream_t)stream;
    const bool bf = dtype == GEMM_EPI_BF16;
    hipError_t err = bf ? launch_acc_store_bf16(p, t, vec1, s) : launch_kind<ACC_STORE>(p, t, vec1, s);

    // stage 2: the epilogue, elementwise, from the accumulator in HBM
    if (err == hipSuccess) {
        EpiParams q;
        q.acc = acc;
        q.C = (const _Float16 *)C;
        q.X = (const _Float16 *)X;
        q.row_bias = (const _Float16 *)row_bias;
        q.col_bias = (const _Float16 *)col_bias;
        q.D = (_Float16 *)D;
        q.Aux = (_Float16 *)Aux;
        q.rows = L * M;
        q.M = (int)M;
        q.N = (int)N;
        q.alpha = scalars[0];
        q.beta = scalars[1];
        q.s = scalars[2];
        bool vec2 = N % 4 == 0 && aligned(acc, 16) && aligned(D, 8);
        if (kind_reads_c(epilogue_kind)) vec2 = vec2 && aligned(C, 8);
        if (kind_reads_x(epilogue_kind)) vec2 = vec2 && aligned(X, 8);
        if (kind_reads_bias(epilogue_kind)) vec2 = vec2 && aligned(row_bias, 8);
        if (kind_has_aux(epilogue_kind)) vec2 = vec2 && aligned(Aux, 8);
        if (bf)
            err = dispatch_kind(epilogue_kind,
                                [&](auto k) { return launch_epilogue<decltype(k)::value, true>(q, vec2, s); });
        else
            err = dispatch_kind(epilogue_kind,
                                [&](auto k) { return launch_epilogue<decltype(k)::value, false>(q, vec2, s); });
    }
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return GEMM_EPI_ERR_HIP;
    }
    return GEMM_EPI_OK;
}

int gemm_epi_plan_ws(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                     const void *X, const void *row_bias, const void *col_bias, int epilogue_kind, const void *D,
                     const void *Aux, const void *acc_out, int64_t out[7])
{
    const Operands o = {A, B, C, X, row_bias, col_bias, D, Aux, acc_out};
    int rc = check_args(L, M, N, K, o, epilogue_kind);
    if (rc != GEMM_EPI_OK) return rc;
    const bool vec = use_fast_path(M, N, K, o, epilogue_kind);
    if (!vec) {
        const StagedCall call = plan_staged_call(L, M, N, K, o, epilogue_kind);
        if (call.st.on) {
            const TileCfg t = call.sk.on ? call.sk.t : choose_tile(L, M, call.st.N, call.st.K, true);
            const int64_t tiles = L * ((M + t.bm - 1) / t.bm) * ((call.st.N + t.bn - 1) / t.bn);
            if (tiles > INT32_MAX) return GEMM_EPI_ERR_SHAPE;
            if (out) {
                out[0] = t.bm;
                out[1] = t.bn;
                out[2] = t.bk;
                out[3] = 1;
                out[4] = call.sk.on ? call.sk.groups : tiles;
                out[5] = 64 * t.wgm * t.wgn;
                out[6] = (int64_t)call.st.bytes;
            }
            return GEMM_EPI_OK;
        }
    }
    const SkPlan sk = plan_stream_k(L, M, N, K, vec);
    if (!sk.on) {
        int64_t o6[6];
        rc = gemm_epi_plan_ext(L, M, N, K, A, B, C, X, row_bias, col_bias, epilogue_kind, D, Aux, acc_out, o6);
        if (rc == GEMM_EPI_OK && out) {
            for (int q = 0; q < 6; q++) out[q] = o6[q];
            out[6] = 0;
        }
        return rc;
    }
    if (out) {
        out[0] = sk.t.bm;
        out[1] = sk.t.bn;
        out[2] = sk.t.bk;
        out[3] = 1;
        out[4] = sk.groups;
        out[5] = 64 * sk.t.wgm * sk.t.wgn;
        out[6] = (int64_t)sk.workspace;
    }
    return GEMM_EPI_OK;
}

int gemm_epi_run_ws(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                    const void *X, const void *row_bias, const void *col_bias, const float *scalars, int epilogue_kind,
                    void *D, void *Aux, void *acc_out, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm_epi_run_ws_typed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                                 workspace, workspace_bytes, GEMM_EPI_F16, stream);
}

int gemm_epi_run_ws_typed(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                          const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                          int epilogue_kind, void *D, void *Aux, void *acc_out, void *workspace,
                          size_t workspace_bytes, int dtype, void *stream)
{
    const Operands o = {A, B, C, X, row_bias, col_bias, D, Aux, acc_out};
    int rc = check_args(L, M, N, K, o, epilogue_kind);
    if (rc != GEMM_EPI_OK) return rc;
    if (dtype != GEMM_EPI_F16 && dtype != GEMM_EPI_BF16) return GEMM_EPI_ERR_DTYPE;
    if (!scalars) return GEMM_EPI_ERR_NULL_INPUT;
    const bool vec = use_fast_path(M, N, K, o, epilogue_kind);
    if (!vec) {
        const StagedCall call = plan_staged_call(L, M, N, K, o, epilogue_kind);
        if (call.st.on && workspace && workspace_bytes >= call.st.bytes && aligned(workspace, 16))
            return launch_staged(L, M, N, K, o, scalars, epilogue_kind, call, workspace, dtype, (hipStream_t)stream);
    }
    const SkPlan sk = plan_stream_k(L, M, N, K, vec);
    if (!sk.on)
        return gemm_epi_run_typed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux,
                                  acc_out, dtype, stream);
    if (!workspace || workspace_bytes < sk.workspace) return GEMM_EPI_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return GEMM_EPI_ERR_ALIGN;
    return launch_split(L, M, N, o, scalars, epilogue_kind, sk, workspace, dtype, (hipStream_t)stream);
}

int gemm_epi_run_ws_static(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                           const void *X, const void *row_bias, const void *col_bias, const float *scalars,
                           int epilogue_kind, void *D, void *Aux, void *acc_out, int dtype, void *stream)
{
    const Operands o = {A, B, C, X, row_bias, col_bias, D, Aux, acc_out};
    int rc = check_args(L, M, N, K, o, epilogue_kind);
    if (rc != GEMM_EPI_OK) return rc;
    if (dtype != GEMM_EPI_F16 && dtype != GEMM_EPI_BF16) return GEMM_EPI_ERR_DTYPE;
    if (!scalars) return GEMM_EPI_ERR_NULL_INPUT;
    const bool vec = use_fast_path(M, N, K, o, epilogue_kind);
    const SkPlan sk = plan_stream_k(L, M, N, K, vec, kStaticMaxGroups);
    if (!sk.on)
        return gemm_epi_run_typed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux,
                                  acc_out, dtype, stream);
    if (sk.workspace > kStaticScratchBytes) return GEMM_EPI_ERR_WORKSPACE;  // the plan cap makes this unreachable
    void *ws = nullptr;
    const hipError_t err = device_scratch((hipStream_t)stream, &ws);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return GEMM_EPI_ERR_HIP;
    }
    return launch_split(L, M, N, o, scalars, epilogue_kind, sk, ws, dtype, (hipStream_t)stream);
}

int gemm_epi_run(int64_t L, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *C,
                 const void *X, const float *scalars, int epilogue_kind, void *D, void *Aux, void *stream)
{
    return gemm_epi_run_ext(L, M, N, K, A, B, C, X, nullptr, nullptr, scalars, epilogue_kind, D, Aux, nullptr,
                            stream);
}

}  // extern "C"
