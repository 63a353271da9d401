// The per-chunk attention weights (chunk_scores.h) and the per-chunk states
// (chunk_state.h) in one launch.  The two are independent products of the
// projection's outputs; the state tiles come first (four K chunks each at
// C = 256) and the score tiles (K = s, two chunks) fill the CUs that the
// state tiles' last partial round leaves idle, instead of a launch of their
// own that is too small to fill the chip.
#include "chunk_scores.h"
#include "chunk_state.h"

namespace gau {
namespace {

template <typename T, int TS>
struct BothTiles {
    static constexpr int LDS = StateTile<T>::LDS > ScoresTile<T, TS>::LDS ? StateTile<T>::LDS : ScoresTile<T, TS>::LDS;
};

// Blocks [0, n_state) form state tiles, the rest score tiles; each range is
// spread over the XCDs in contiguous logical ranges of its own.
template <typename T, int TS>
__global__ __launch_bounds__(256) void chunk_scores_state_kernel(ScoresParams ps, StateParams pt, int n_state) {
    extern __shared__ __align__(16) char lds[];
    const int b = blockIdx.x;
    if (b < n_state)
        state_tile<T>(pt, xcd_remap(b, n_state), lds);
    else
        scores_tile<T, TS>(ps, xcd_remap(b - n_state, gridDim.x - n_state), lds);
}

template <typename T, int TS>
hipError_t launch_t(const ScoresParams& ps, const StateParams& pt, hipStream_t st) {
    constexpr int LDS = BothTiles<T, TS>::LDS;
    static_assert(LDS <= 160 * 1024, "LDS over budget");
    const int n_state = state_blocks(pt);
    const int blocks = n_state + scores_blocks(ps);
    hipError_t e = allow_lds<chunk_scores_state_kernel<T, TS>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_scores_state_kernel<T, TS>), dim3(blocks), dim3(256), LDS, st, ps, pt, n_state);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_scores_state(const ScoresParams& ps, const StateParams& pt, bool bf16_storage,
                                     hipStream_t st) {
    const bool wide = scores_tile_width(ps.C) == 128;
    if (bf16_storage) return wide ? launch_t<bf16, 128>(ps, pt, st) : launch_t<bf16, 64>(ps, pt, st);
    return wide ? launch_t<float, 128>(ps, pt, st) : launch_t<float, 64>(ps, pt, st);
}

}  // namespace gau
