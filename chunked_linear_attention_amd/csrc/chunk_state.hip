// Launch of the per-chunk states alone (the tile is in chunk_state.h); the
// forward pass normally runs them in one launch with the attention weights
// (chunk_scores_state.hip).
#include "chunk_state.h"

namespace gau {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void chunk_state_kernel(StateParams p) {
    extern __shared__ __align__(16) char lds[];
    state_tile<T>(p, xcd_remap(blockIdx.x, gridDim.x), lds);
}

template <typename T>
hipError_t launch(const StateParams& p, hipStream_t st) {
    constexpr int LDS = StateTile<T>::LDS;
    static_assert(LDS <= 160 * 1024, "state GEMM LDS over budget");
    hipError_t e = allow_lds<chunk_state_kernel<T>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_state_kernel<T>, dim3(state_blocks(p)), dim3(256), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_state(const StateParams& p, bool bf16_storage, hipStream_t st) {
    return bf16_storage ? launch<bf16>(p, st) : launch<float>(p, st);
}

}  // namespace gau
