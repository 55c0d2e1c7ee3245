// gemm_epi_bf16_f16e.hip -- the fused kernels instantiated for bfloat16 A and B with fp16
// epilogue tensors (C, X, the biases, D and Aux); fp32 accumulation and
// epilogue as everywhere.  A translation unit of its own so that the element
// type combinations compile in parallel; the host code and the C ABI are in
// gemm_epi.hip.
#include <hip/hip_runtime.h>

#include "gemm_epi_launch.hpp"

namespace gemm_epi {

hipError_t launch_fused_bf16_f16e(int kind, const Params &p, const TileCfg &t, bool vec, hipStream_t stream)
{
    return dispatch_kind(kind, [&](auto k) {
        return launch_kind<decltype(k)::value, true, EPI_OTHER16>(p, t, vec, stream);
    });
}

}  // namespace gemm_epi
