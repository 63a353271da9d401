// Per-chunk attention weights of the local (quadratic) part:
//   A_g[i][j] = relu^2(quad_scale * q_quad_i . k_quad_j + Bias[i][j]),
//   Bias[i][j] = w[C-1 + j - i];  causal: A_g[i][j] = 0 for j > i (diagonal kept).
// Pages: relu^2(Q K^T + b) inside each chunk (wikillm "Method" step 1 and
// eq. 5; Su's post "Weak Attention" and "Mixed Chunking"); the bias as a
// Toeplitz matrix of a 2C-1 vector (papercache, appendix D, Code 4, n < 512);
// the listing scales Q K^T by 1/C before adding the bias and masks after
// relu^2 (wikillm, FLASH block pseudocode), which quad_scale carries.
//
// A batched GEMM over chunks on the shared MFMA core: each block forms one
// TS x TS (query x key) tile from Q_quad and K_quad rows (K = s), applies
// bias, relu^2 and the mask in the epilogue and stores A_g query-major in the
// layer's element type, the precision the attention GEMM reads it in.  Causal
// chunks compute only the tiles at or below the diagonal.
#include "gau_launch.h"
#include "gemm_core.h"

namespace gau {
namespace {

template <typename T, int TS>
__global__ __launch_bounds__(256) void chunk_scores_kernel(ScoresParams p) {
    extern __shared__ __align__(16) char lds[];
    using G = GemmCore<T, TS, TS, 2, 2>;
    constexpr int EB = Elem<T>::kBytes;
    const int nt = p.C / TS;
    const int npairs = p.causal ? nt * (nt + 1) / 2 : nt * nt;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int pair = bid % npairs;
    const int chunk = bid / npairs;
    int qt, kt;
    if (p.causal) {  // pair -> (qt, kt) with kt <= qt, row-major over the lower triangle
        qt = 0;
        while ((qt + 1) * (qt + 2) / 2 <= pair) ++qt;
        kt = pair - qt * (qt + 1) / 2;
    } else {
        qt = pair / nt;
        kt = pair % nt;
    }
    const int q0 = qt * TS, k0 = kt * TS;
    const int G_ = p.T / p.C;
    const int b = chunk / G_, g = chunk - b * G_;
    const size_t tok0 = (size_t)b * p.T + (size_t)g * p.C;
    const size_t pitch = (size_t)p.s * EB;

    // acc rows = keys (A operand K_quad), columns = queries: the packed store
    // then runs along the query-major rows of A_g.
    f32x16_t acc[G::MB][G::NB];
    G::zero(acc);
    G::run(acc, (const char*)p.Kq + (tok0 + k0) * pitch, pitch, TS, (const char*)p.Qq + (tok0 + q0) * pitch, pitch,
           TS, p.s, lds);

    const float qs = p.quad_scale;
    const float* w = p.relpos + (p.C - 1);
    const bool diag = p.causal && qt == kt;
    auto val = [&](int kr, int qc, float v) {
        const int i = q0 + qc, j = k0 + kr;  // query and key positions in the chunk
        float x = v * qs + w[j - i];
        x = x > 0.f ? x * x : 0.f;
        return (diag && j > i) ? 0.f : x;
    };
    char* A = (char*)p.A + ((size_t)chunk * p.C + q0) * p.C * EB + (size_t)k0 * EB;
    const int C = p.C;
    constexpr int STAGE = TS * (TS * EB + 16);
    constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
    G::template store_packed<T>(acc, lds, LDS, val,
                                [&](int q, int k) -> char* { return A + ((size_t)q * C + k) * EB; });
}

template <typename T, int TS>
hipError_t launch_t(const ScoresParams& p, hipStream_t st) {
    using G = GemmCore<T, TS, TS, 2, 2>;
    constexpr int EB = Elem<T>::kBytes;
    constexpr int STAGE = TS * (TS * EB + 16);
    constexpr int LDS = G::LDS_BYTES > STAGE ? G::LDS_BYTES : STAGE;
    const int nt = p.C / TS;
    const int npairs = p.causal ? nt * (nt + 1) / 2 : nt * nt;
    const int blocks = npairs * p.B * (p.T / p.C);
    hipError_t e = allow_lds<chunk_scores_kernel<T, TS>>(LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_scores_kernel<T, TS>), dim3(blocks), dim3(256), LDS, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_scores(const ScoresParams& p, bool bf16_storage, hipStream_t st) {
    if (bf16_storage) return p.C >= 128 ? launch_t<bf16, 128>(p, st) : launch_t<bf16, 64>(p, st);
    return p.C >= 128 ? launch_t<float, 128>(p, st) : launch_t<float, 64>(p, st);
}

}  // namespace gau
