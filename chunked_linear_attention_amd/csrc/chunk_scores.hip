// Launch of the per-chunk attention weights alone (the tile is in
// chunk_scores.h); the forward pass normally runs them in one launch with the
// chunk states (chunk_scores_state.hip).
#include "chunk_scores.h"

namespace gau {
namespace {

template <typename T, int TS>
__global__ __launch_bounds__(256) void chunk_scores_kernel(ScoresParams p) {
    extern __shared__ __align__(16) char lds[];
    scores_tile<T, TS>(p, xcd_remap(blockIdx.x, gridDim.x), lds);
}

template <typename T, int TS>
hipError_t launch_t(const ScoresParams& p, hipStream_t st) {
    constexpr int LDS = ScoresTile<T, TS>::LDS;
    hipError_t e = allow_lds<chunk_scores_kernel<T, TS>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_scores_kernel<T, TS>), dim3(scores_blocks(p)), dim3(256), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_scores(const ScoresParams& p, bool bf16_storage, hipStream_t st) {
    const bool wide = scores_tile_width(p.C) == 128;
    if (bf16_storage) return wide ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
    return wide ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace gau
