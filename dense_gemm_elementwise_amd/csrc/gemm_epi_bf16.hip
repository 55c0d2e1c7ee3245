// gemm_epi_bf16.hip -- the fused kernels instantiated for bfloat16 tensors
// (A, B, C, X, the biases, D and Aux all bfloat16; fp32 accumulation and
// epilogue): the one-tile-per-workgroup build, the stream-K build and the
// accumulator-only GEMM of the unfused composition.  The host code and the C
// ABI are in gemm_epi.hip.
#include <hip/hip_runtime.h>

#include "gemm_epi_launch.hpp"

namespace gemm_epi {

hipError_t launch_fused_bf16(int kind, const Params &p, const TileCfg &t, bool vec, hipStream_t stream)
{
    return dispatch_kind(kind, [&](auto k) { return launch_kind<decltype(k)::value, true>(p, t, vec, stream); });
}

hipError_t launch_sk_bf16(int kind, const Params &p, int groups, hipStream_t stream)
{
    return dispatch_kind(kind, [&](auto k) { return launch_kind_sk<decltype(k)::value, true>(p, groups, stream); });
}

hipError_t launch_acc_store_bf16(const Params &p, const TileCfg &t, bool vec, hipStream_t stream)
{
    return launch_kind<ACC_STORE, true>(p, t, vec, stream);
}

}  // namespace gemm_epi
